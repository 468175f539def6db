"""Pins of oracle.layer (tail ring, decode composition, transcode, plane
bytes) and oracle.budget against the pages' printed figures."""

import json
import os

import numpy as np
import pytest

from oracle import attention, budget, cobra, layer, layout
from oracle.codecs import encode_rows, decode_rows
from oracle.layer import PlaneSpec
from oracle.rounding import rbf16, rn16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _x(rng, B, T, Hkv):
    return rng.standard_normal((B, T, Hkv, 128)).astype(np.float32)


def test_tail_ring_slots():
    rng = np.random.default_rng(0)
    x = _x(rng, 1, 200, 2)
    ring = layer.tail_ring(x, 64)
    for t in range(136, 200):                   # the newest 64 tokens
        assert np.array_equal(ring[0, :, t % 64], rn16(x[0, t]))


def test_tail_covering_everything_is_f16_attention():
    rng = np.random.default_rng(1)
    B, T, Hkv, G = 1, 100, 2, 2
    x, v = _x(rng, B, T, Hkv), _x(rng, B, T, Hkv)
    q = rng.standard_normal((B, Hkv * G, 128))
    spec = PlaneSpec("q2_0")
    out = layer.decode(q, layer.encode_plane(x, spec), layer.encode_plane(v, spec),
                       layer.tail_ring(x, 128), layer.tail_ring(v, 128), spec, spec, T, 128, 0.1)
    ref = attention.attend_batch(q, rn16(x).astype(np.float64), rn16(v).astype(np.float64), 0.1)
    assert np.allclose(out, ref, rtol=0, atol=1e-13)


def test_body_plus_tail_split():
    rng = np.random.default_rng(2)
    B, T, Hkv, N = 2, 150, 1, 64
    x, v = _x(rng, B, T, Hkv), _x(rng, B, T, Hkv)
    q = rng.standard_normal((B, 3, 128))
    ks, vs = PlaneSpec("q8_0"), PlaneSpec("q4_1")
    kenc, venc = layer.encode_plane(x, ks), layer.encode_plane(v, vs)
    out = layer.decode(q, kenc, venc, layer.tail_ring(x, N), layer.tail_ring(v, N), ks, vs, T, N, 0.3)
    K = np.concatenate([decode_rows(encode_rows(x[:, :T - N], "q8_0"), "q8_0"),
                        rn16(x[:, T - N:]).astype(np.float64)], axis=1)
    V = np.concatenate([decode_rows(encode_rows(v[:, :T - N], "q4_1"), "q4_1", rounded=False),
                        rn16(v[:, T - N:]).astype(np.float64)], axis=1)
    assert np.allclose(out, attention.attend_batch(q, K, V, 0.3), rtol=0, atol=1e-13)


def test_transcode_closed_forms():
    rng = np.random.default_rng(3)
    x = _x(rng, 1, 70, 2)
    f16, q8 = PlaneSpec("f16"), PlaneSpec("q8_0")
    enc = layer.encode_plane(x, f16)
    tc = layer.transcode_plane(enc, f16, q8)
    direct = layer.encode_plane(rn16(x).astype(np.float32), q8)
    for b in range(1):
        for h in range(2):
            assert np.array_equal(tc[b][h]["codes"], direct[b][h]["codes"])
            assert np.array_equal(tc[b][h]["scales"], direct[b][h]["scales"])
    for c in ("q4_0", "q3_1"):
        s = PlaneSpec(c)
        e = layer.encode_plane(x, s)
        same = layer.transcode_plane(e, s, s)
        assert np.array_equal(same[0][1]["codes"], e[0][1]["codes"])


def _lowrank_spec(rng, Hkv):
    table = [(128, 1), (64, 2), (32, 4), (16, 4), (64, 3), (128, 1), (32, 2), (64, 3)][:Hkv]
    Ps = []
    for r, _ in table:
        Q, R = np.linalg.qr(rng.standard_normal((128, 128)))
        Ps.append(cobra.projection(Q * np.sign(np.diag(R)), r))
    return PlaneSpec(basis="lowrank", P=Ps, head_codec=["q%d_1" % b for _, b in table]), table


@pytest.mark.parametrize("codec", ["q8_0", "q3_0", "q6_1", "q1_1", "f16"])
def test_plane_bytes_roundtrip(codec):
    rng = np.random.default_rng(4)
    x = _x(rng, 2, 100, 3)
    spec = PlaneSpec(codec)
    enc = layer.encode_plane(x, spec)
    buf = layer.pack_plane(enc, spec, 128)
    R = budget.code_bits(codec) // 8
    assert buf["codes"].size == 2 * 3 * 128 * R
    back = layer.unpack_plane(buf, spec, 2, 3, 128, 100)
    key = "values" if codec == "f16" else "codes"
    for b in range(2):
        for h in range(3):
            assert np.array_equal(back[b][h][key], enc[b][h][key])


def test_lowrank_plane_bytes_roundtrip_and_sizes():
    rng = np.random.default_rng(5)
    spec, table = _lowrank_spec(rng, 8)
    x = _x(rng, 2, 64, 8)
    enc = layer.encode_plane(x, spec)
    buf = layer.pack_plane(enc, spec, 64)
    # per token over the 8 heads: 128 code bytes + 17 blocks x (scale + min)
    assert buf["codes"].size == 2 * 64 * 128
    assert buf["scales"].size == 2 * 64 * 17 and buf["mins"].size == 2 * 64 * 17
    back = layer.unpack_plane(buf, spec, 2, 8, 64, 64)
    for h in range(8):
        assert np.array_equal(back[1][h]["codes"], enc[1][h]["codes"])
        assert np.array_equal(back[1][h]["mins"], enc[1][h]["mins"])


def test_tail_bytes_roundtrip():
    rng = np.random.default_rng(6)
    ring = layer.tail_ring(_x(rng, 2, 300, 2), 128)
    assert np.array_equal(layer.unpack_tail(layer.pack_tail(ring), 2, 2, 128), ring)


def test_bf16_tail_bytes():
    """bfloat16 ring: values are the rounded inputs of the newest tokens, and
    a row's bytes are the high halves of the values' binary32 patterns."""
    rng = np.random.default_rng(8)
    x = _x(rng, 1, 130, 1)
    ring = layer.tail_ring(x, 64, fmt="bf16")
    for t in range(66, 130):
        assert np.array_equal(ring[0, 0, t % 64], rbf16(x[0, t, 0].astype(np.float64)).astype(np.float32))
    raw = layer.pack_tail(ring, fmt="bf16")
    rows = layout.untile_plane(raw, 256)
    hi = (ring[0, 0].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(rows.view(np.uint16), hi)


def test_cobra_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "cobra_worked_example.json")))
    assert budget.budget_bits(g["bpd"], g["head_dim"]) * g["heads"] == g["pair_budget_bits"]
    for k in ("uniform", "head_A", "head_B"):
        assert budget.head_code_bits(g[k]["rank"], g[k]["bits"]) == g[k]["code_bits"]
    assert g["head_A"]["code_bits"] + g["head_B"]["code_bits"] == g["pair_budget_bits"]
    # a diffuse head loses the share of directions it drops
    assert 1 - g["uniform"]["rank"] / g["head_dim"] == g["head_B_variance_lost"]["uniform"]
    assert 1 - g["head_B"]["rank"] / g["head_dim"] == g["head_B_variance_lost"]["per_head"]


def test_lowrank_table_is_one_bit_per_dim():
    rng = np.random.default_rng(7)
    _, table = _lowrank_spec(rng, 8)
    assert sum(budget.head_code_bits(r, b) for r, b in table) == 8 * budget.budget_bits(1)


def test_kld_table_consistency():
    g = json.load(open(os.path.join(GOLDEN, "kld_table.json")))
    for c, stated in g["stated_reductions_tail0_to_tail1024"].items():
        t0, t1, _ = g["median_kld"][c]
        assert abs((1 - t1 / t0) - stated) < 0.005
