"""Planted mistakes in the oracle (on the CPU) must fail its pins.

Each case swaps one oracle routine for a plausible wrong version and checks
that at least one pin test then fails.  This shows the pins constrain the
oracle rather than restate it.
"""

import numpy as np
import pytest

import oracle.attention
import oracle.bitpack
import oracle.codecs
import oracle.hadamard
import oracle.kvarn
import oracle.layer
import oracle.layout
from tests import (test_oracle_attention as TA, test_oracle_bases as TB,
                   test_oracle_codecs as TC, test_oracle_layer as TL,
                   test_oracle_layout as TO)


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_round_half_up_is_caught(monkeypatch):
    monkeypatch.setattr(oracle.codecs, "rne", lambda x: np.floor(np.asarray(x, np.float64) + 0.5))
    _fails(TC.test_encode_0_brute_force, 4)


def test_signed_max_levels_are_caught(monkeypatch):
    monkeypatch.setattr(oracle.codecs, "qmax_0", lambda b: 2 ** (b - 1))
    _fails(TC.test_encode_0_brute_force, 3)


def test_unrounded_min_is_caught(monkeypatch):
    monkeypatch.setattr(oracle.codecs, "rn16", lambda x: np.asarray(x, np.float64))
    _fails(TC.test_encode_1_brute_force, 4)


def test_wrong_sylvester_sign_is_caught(monkeypatch):
    def bad(n):
        H = np.ones((1, 1), dtype=np.int64)
        while H.shape[0] < n:
            H = np.block([[H, -H], [H, H]])
        return H
    monkeypatch.setattr(oracle.hadamard, "sylvester", bad)
    _fails(TA.test_sylvester_closed_forms)
    _fails(TA.test_transform_involution_and_dense)


def test_missing_inverse_scale_is_caught(monkeypatch):
    monkeypatch.setattr(oracle.kvarn, "unrotate",
                        lambda y, w: oracle.hadamard.transform(y) / np.asarray(w, np.float64))
    _fails(TB.test_kvarn_roundtrip_and_attention_identity)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    def bad(q, K, V, sm_scale):
        q, K, V = (np.asarray(a, np.float64) for a in (q, K, V))
        out = np.empty((q.shape[0], V.shape[2]))
        for h in range(q.shape[0]):
            g = h % K.shape[1]
            s = sm_scale * (K[:, g, :] @ q[h])
            p = np.exp(s - s.max())
            out[h] = (p / p.sum()) @ V[:, g, :]
        return out
    monkeypatch.setattr(oracle.attention, "attend", bad)
    _fails(TA.test_gqa_equals_repeated_kv)


def test_unnormalised_softmax_is_caught(monkeypatch):
    def bad(q, K, V, sm_scale):
        q, K, V = (np.asarray(a, np.float64) for a in (q, K, V))
        G = q.shape[0] // K.shape[1]
        out = np.empty((q.shape[0], V.shape[2]))
        for h in range(q.shape[0]):
            s = sm_scale * (K[:, h // G, :] @ q[h])
            out[h] = np.exp(s - s.max()) @ V[:, h // G, :]
        return out
    monkeypatch.setattr(oracle.attention, "attend", bad)
    _fails(TA.test_uniform_scores_give_mean)


def test_wrong_tail_slot_is_caught(monkeypatch):
    def bad(x, N):
        x = np.asarray(x)
        ring = np.zeros((x.shape[0], x.shape[2], N, 128), np.float16)
        for t in range(x.shape[1]):
            ring[:, :, (t + 1) % N, :] = x[:, t].astype(np.float16)
        return ring
    monkeypatch.setattr(oracle.layer, "tail_ring", bad)
    _fails(TL.test_tail_ring_slots)


def test_transposed_tile_is_caught(monkeypatch):
    def bad(rows):
        rows = np.asarray(rows, np.uint8)
        cap, R = rows.shape
        return rows.reshape(-1).copy()      # plain token-major rows, no tiling
    monkeypatch.setattr(oracle.layout, "tile_plane", bad)
    monkeypatch.setattr(TO, "tile_plane", bad)
    _fails(TO.test_tile_offsets_hand_worked)


def test_msb_first_packing_is_caught(monkeypatch):
    def bad(codes, b, signed):
        codes = np.asarray(codes, np.int64)
        L = codes.shape[-1]
        u = codes & ((1 << b) - 1)
        bit = (u[..., None] >> np.arange(b)[::-1]) & 1
        flat = bit.reshape(codes.shape[:-1] + (L * b,)).astype(np.uint8)
        return np.packbits(flat, axis=-1, bitorder="big")
    monkeypatch.setattr(TO, "pack_codes", bad)
    _fails(TO.test_hand_worked_bit_patterns)


def test_allocator_mutations_are_caught(monkeypatch):
    """The KV-COBRA oracle: a C1 that ignores the budget boundary, and a
    relaxation bound with the multiplier's sign flipped, each fail a pin."""
    import oracle.allocator as OA
    from tests import test_cobra_allocator as TCA

    good = OA.head_error

    def strict_c1(lam, ranks, bits, max_cost, gamma=OA.GAMMA):
        errs, pick = [float("inf")] * (max_cost + 1), [None] * (max_cost + 1)
        for c in range(max_cost + 1):
            for r in ranks:
                for b in bits:
                    if r * b < c and good(lam, r, b, gamma) < errs[c]:      # '<' for '<='
                        errs[c], pick[c] = good(lam, r, b, gamma), (r, b)
        return errs, pick
    monkeypatch.setattr(OA, "c1_curve", strict_c1)
    _fails(TCA.test_oracle_c1_and_plain_c2)
    monkeypatch.undo()

    real = OA.lagrangian_bound

    def flipped(spectra, ranks, bits, budget, gamma=OA.GAMMA):
        v, mu = real(spectra, ranks, bits, budget, gamma)
        return v + 2.0 * mu * budget, mu
    monkeypatch.setattr(OA, "lagrangian_bound", flipped)
    _fails(TCA.test_oracle_c1_and_plain_c2)
