"""GPU parity of the append kernel against the oracle: bit-exact codes,
scales, mins and precision tail for the unrotated codecs; the tie rule for
the Hadamard and low-rank bases.  Inputs are the seeded synthetic workloads
at sizes the oracle finishes in seconds, with ragged token counts, appends of
several chunk sizes (prefill and single tokens) and tails that wrap."""

import numpy as np
import pytest
import torch

import oracle.layer as OL
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

ALL = ["f16", "q8_0", "q6_0", "q5_0", "q4_0", "q3_0", "q2_0",
       "q8_1", "q6_1", "q5_1", "q4_1", "q3_1", "q2_1", "q1_1"]


def _append_chunks(cache, k, v, chunks, device):
    t = 0
    for n in chunks:
        cache.append(k[:, t:t + n].to(device), v[:, t:t + n].to(device))
        t += n
    torch.cuda.synchronize()
    return t


def _check_exact(cache, name, x, ospec, T, N):
    enc, packed, tail = H.oracle_layer_bytes(x, ospec, cache.capacity, N)
    got = H.download(cache, name)
    assert np.array_equal(got["codes"][: packed["codes"].size], packed["codes"]), name + " codes"
    if packed["scales"] is not None:
        assert np.array_equal(got["scales"], packed["scales"]), name + " scales"
    if packed["mins"] is not None:
        assert np.array_equal(got["mins"], packed["mins"]), name + " mins"
    if N > 0:
        assert np.array_equal(got["tail"], tail), name + " tail"


@pytest.mark.parametrize("kc,vc", [(c, ALL[(i + 3) % len(ALL)]) for i, c in enumerate(ALL)])
def test_plain_codecs_bit_exact(gpu, kc, vc):
    wl = synth.WORKLOADS["gqa4_q8k_q4v_tail1024"].with_(B=2, Hkv=2, Hq=8, T=200, N=64)
    k = synth.layer_rows(wl, 0, "k", T=wl.T)
    v = synth.layer_rows(wl, 0, "v", T=wl.T)
    gk, gv, ok_, ov = H.specs(wl, kcodec=kc, vcodec=vc)
    cache = H.new_cache(wl, 256, gk, gv, gpu)
    T = _append_chunks(cache, k, v, [130, 1, 1, 67, 1], gpu)
    assert cache.n_tokens == T == 200
    _check_exact(cache, "k", k.numpy(), ok_, T, wl.N)
    _check_exact(cache, "v", v.numpy(), ov, T, wl.N)


@pytest.mark.parametrize("name", ["tiny", "gqa4_q8k_q4v_tail1024"])
def test_workloads_bit_exact(gpu, name):
    wl = synth.WORKLOADS[name]
    T = 256 if name == "tiny" else 1500
    wl = wl.with_(T=T)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    gk, gv, ok_, ov = H.specs(wl)
    cache = H.new_cache(wl, 1536 if T > 256 else 256, gk, gv, gpu)
    _append_chunks(cache, k, v, [T - 3, 1, 1, 1], gpu)
    _check_exact(cache, "k", k.numpy(), ok_, T, wl.N)
    _check_exact(cache, "v", v.numpy(), ov, T, wl.N)


def test_extreme_blocks_bit_exact(gpu):
    """All-zero blocks, constant blocks, ties planted at x = (k + 1/2) d,
    tiny (subnormal-scale) and large magnitudes."""
    wl = synth.WORKLOADS["tiny"].with_(T=64)
    x = np.zeros((1, 64, 1, 128), np.float32)
    d0 = np.float32(np.float16(0.37))
    x[0, 1, 0, :] = 1.25                                          # constant row
    x[0, 2, 0, :32] = (np.arange(32) % 7 - 3 + 0.5) * d0          # exact ties
    x[0, 2, 0, 31] = 7 * d0
    x[0, 3, 0, :] = np.float32(1e-6) * np.arange(128)              # subnormal scales
    x[0, 4, 0, :] = np.float32(3000.0) * np.sin(np.arange(128))
    x[0, 5:, 0, :] = np.random.default_rng(0).standard_normal((59, 128))
    xt = torch.from_numpy(x)
    for kc, vc in [("q4_0", "q3_1"), ("q8_0", "q2_0"), ("q2_1", "q6_0"), ("q1_1", "q5_1")]:
        gk, gv, ok_, ov = H.specs(wl, kcodec=kc, vcodec=vc)
        cache = H.new_cache(wl, 64, gk, gv, gpu, N=64)
        _append_chunks(cache, xt, xt, [64], gpu)
        _check_exact(cache, "k", x, ok_, 64, 64)
        _check_exact(cache, "v", x, ov, 64, 64)


@pytest.mark.parametrize("codec", ["q3_0", "q4_0", "q8_1", "q2_1"])
def test_hadamard_tie_rule(gpu, codec):
    wl = synth.WORKLOADS["kvarn_q3_tail2048"].with_(B=2, T=700, N=128)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    gk, gv, ok_, ov = H.specs(wl, kcodec=codec, vcodec=codec)
    cache = H.new_cache(wl, 768, gk, gv, gpu)
    T = _append_chunks(cache, k, v, [600, 1, 99], gpu)
    for name, x, spec in (("k", k.numpy(), ok_), ("v", v.numpy(), ov)):
        encs, buf = H.unpack(cache, name, spec, T)
        for b in range(wl.B):
            for h in range(wl.Hkv):
                H.check_rotated_head(x[b, :, h, :], encs[b][h], spec, h)
        tail = OL.pack_tail(OL.tail_ring(x, wl.N))
        assert np.array_equal(buf["tail"], tail)


def test_lowrank_tie_rule(gpu):
    wl = synth.WORKLOADS["lowrank_1bpd"].with_(B=2, T=300)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    gk, gv, ok_, ov = H.specs(wl)
    cache = H.new_cache(wl, 320, gk, gv, gpu)
    T = _append_chunks(cache, k, v, [299, 1], gpu)
    total = 0
    for name, x, spec in (("k", k.numpy(), ok_), ("v", v.numpy(), ov)):
        encs, _ = H.unpack(cache, name, spec, T)
        for b in range(wl.B):
            for h in range(wl.Hkv):
                n, _ = H.check_rotated_head(x[b, :, h, :], encs[b][h], spec, h)
                total += n
    assert total <= 50


def test_append_is_deterministic(gpu):
    wl = synth.WORKLOADS["kvarn_q3_tail2048"].with_(B=1, T=256, N=64)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    gk, gv, _, _ = H.specs(wl)
    outs = []
    for _ in range(2):
        cache = H.new_cache(wl, 256, gk, gv, gpu)
        _append_chunks(cache, k, v, [256], gpu)
        outs.append(H.download(cache, "k")["codes"])
    assert np.array_equal(outs[0], outs[1])


def test_lowrank_prefill_ragged_tail(gpu):
    """A prefill-sized low-rank append (the 16-token matrix-core path) into a
    ragged batch with a precision tail: sequence b appends n tokens at its
    own position; codes follow the tie rule against the oracle's encoding of
    those tokens, and the tail ring (all newest 64 from this call) is exact."""
    Ts0, n = [0, 21, 40], 90
    wl = synth.WORKLOADS["lowrank_1bpd"].with_(B=3, T=n, N=64)
    k = synth.layer_rows(wl, 0, "k")              # [3, n, Hkv, 128]: each sequence's new tokens
    v = synth.layer_rows(wl, 0, "v")
    gk, gv, ok_, ov = H.specs(wl)
    cap = 192
    cache = H.new_cache(wl, cap, gk, gv, gpu, N=64)
    cache.n_tokens = max(Ts0)
    cache.set_seq_tokens(torch.tensor(Ts0, dtype=torch.int32, device=gpu))
    cache.append(k.to(gpu), v.to(gpu))
    torch.cuda.synchronize()
    assert cache.seq_tokens.cpu().tolist() == [t + n for t in Ts0]
    for name, x, spec in (("k", k.numpy(), ok_), ("v", v.numpy(), ov)):
        encs, buf = H.unpack(cache, name, spec, max(Ts0) + n)
        for b in range(3):
            for h in range(wl.Hkv):
                e = encs[b][h]
                rows = {key: (val[Ts0[b]:Ts0[b] + n] if val is not None else None) for key, val in e.items()}
                H.check_rotated_head(x[b, :, h, :], rows, spec, h)
        # sequence b's tokens sit at positions Ts0[b] ..; n >= 64, so every
        # ring slot holds one of this call's tokens
        rings = []
        for b in range(3):
            xb = np.concatenate([np.zeros((1, Ts0[b], wl.Hkv, 128), np.float32), x[b:b + 1]], axis=1)
            rings.append(OL.tail_ring(xb, 64))
        assert np.array_equal(buf["tail"], OL.pack_tail(np.concatenate(rings))), name


def test_lowrank_every_rank_and_width(gpu):
    """Every (rank, bits) a low-rank head can take (ranks 16, 32, 64, 128 x
    1-4 bits: rows of 2 to 64 bytes, tiled in 2- to 16-byte chunks), one kv
    head each, through the matrix-core prefill path (runs of 280 and 19
    tokens) and the one-token path: codes follow the tie rule against the
    oracle and the decode over them matches the oracle's."""
    table = tuple((r, b) for r in (16, 32, 64, 128) for b in (1, 2, 3, 4))
    wl = synth.WORKLOADS["lowrank_1bpd"].with_(B=1, Hkv=16, Hq=32, T=300, N=0, lowrank=table)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    gk, gv, ok_, ov = H.specs(wl)
    cache = H.new_cache(wl, 320, gk, gv, gpu, N=0)
    T = _append_chunks(cache, k, v, [280, 1, 19], gpu)
    encs = {}
    for name, x, spec in (("k", k.numpy(), ok_), ("v", v.numpy(), ov)):
        encs[name], _ = H.unpack(cache, name, spec, T)
        for h in range(wl.Hkv):
            H.check_rotated_head(x[0, :, h, :], encs[name][0][h], spec, h)
    q = synth.queries(wl, 0)
    out = cache.decode(q.to(gpu), wl.sm_scale).cpu().numpy().astype(np.float64)
    ref = OL.decode(q.numpy(), encs["k"], encs["v"], None, None, ok_, ov, T, 0, wl.sm_scale)
    assert np.max(np.abs(out - ref)) <= H.ATOL
