"""GPU parity of kvq_dequantize (the raw-basis read-back of a plane) against
the oracle's ``attention_kv``, the fp64 cache that decode attends over.

The planes are the oracle's packed encoding uploaded to the device, so the
test isolates the read-back.  Plain planes are bit-exact against the oracle's
binary32 decode (q*d, or the single rounding of u*d + m); rotated and
low-rank planes go through a binary32 inverse transform and are compared
within a bound derived from it (sums of 128 binary32 terms: a few units in
the last place of the row's largest magnitude).  Tail rows are the binary16
ring and must match exactly.  Ragged T (not a tile multiple), T shorter than
the tail, and an empty layer are covered."""

import numpy as np
import pytest
import torch

import oracle.layer as OL
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _expected_plain(enc_planes, tail, spec, T, N):
    """attention_kv with the binary32 rounding of the plain decode."""
    B, Hkv = len(enc_planes), len(enc_planes[0])
    out = np.empty((B, T, Hkv, 128), dtype=np.float32)
    for b in range(B):
        for h in range(Hkv):
            out[b, :, h, :] = OL.dequant_head(enc_planes[b][h], spec, h, exact=False)[:T]
    if N > 0:
        for t in range(max(0, T - N), T):
            out[:, t, :, :] = tail[:, :, t % N, :].astype(np.float32)
    return out


CASES = [
    ("vbr_32layer", "q8_0", 333, 64),
    ("vbr_32layer", "q4_0", 200, 0),
    ("vbr_32layer", "q2_0", 333, 128),
    ("vbr_32layer", "q3_1", 100, 128),     # T shorter than the tail
    ("vbr_32layer", "q1_1", 257, 64),
    ("vbr_32layer", "f16", 190, 64),
    ("vbr_32layer", "q6_0", 65, 0),
    ("kvarn_q3_tail2048", "q3_0", 333, 64),
    ("kvarn_q3_tail2048", "q8_1", 129, 0),
    ("kvarn_q3_tail2048", "q5_0", 300, 128),
    ("lowrank_1bpd", None, 333, 0),
    ("lowrank_1bpd", None, 200, 64),
]


@pytest.mark.parametrize("name,codec,T,N", CASES)
def test_dequantize_matches_oracle(gpu, name, codec, T, N):
    wl = synth.WORKLOADS[name].with_(B=2, T=T, N=N)
    if name != "lowrank_1bpd":
        wl = wl.with_(Hkv=2, Hq=8)
    k = synth.layer_rows(wl, 0, "k").numpy()
    v = synth.layer_rows(wl, 0, "v").numpy()
    gk, gv, ok_, ov = H.specs(wl, kcodec=codec, vcodec=codec)
    cap = (T + 63) // 64 * 64
    cache = H.new_cache(wl, cap, gk, gv, gpu)
    for nm, x, spec in (("k", k, ok_), ("v", v, ov)):
        enc, packed, tail = H.oracle_layer_bytes(x, spec, cap, N)
        H.upload(cache, nm, packed, tail)
    cache.n_tokens = T
    worst = 0.0
    for nm, x, spec in (("k", k, ok_), ("v", v, ov)):
        enc = OL.encode_plane(x, spec)
        ring = OL.tail_ring(x, N) if N else None
        got = cache.dequantize(nm).cpu().numpy()
        torch.cuda.synchronize()
        assert got.shape == (wl.B, T, wl.Hkv, 128)
        nt = min(N, T)
        if nt:
            exp_tail = ring[:, :, [t % N for t in range(T - nt, T)], :].transpose(0, 2, 1, 3)
            assert np.array_equal(got[:, T - nt:], exp_tail.astype(np.float32)), (nm, "tail")
        if spec.basis == "plain":
            exp = _expected_plain(enc, ring, spec, T, N)
            assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), nm
        else:
            ref = OL.attention_kv(enc, ring, spec, T, N)
            scale = np.abs(ref).max(axis=-1, keepdims=True) + 1e-30
            err = np.abs(got.astype(np.float64) - ref) / scale
            worst = max(worst, float(err.max()))
            assert err.max() <= 2e-5, (nm, float(err.max()))
    print("%s %s T=%d N=%d: worst relative %.2e" % (name, codec, T, N, worst))


def test_dequantize_empty_and_after_append(gpu):
    """n_tokens == 0 writes nothing; after device appends the read-back
    equals the oracle's cache of the same rows."""
    wl = synth.WORKLOADS["gqa4_q8k_q4v_tail1024"].with_(B=1, Hkv=2, Hq=8, T=150, N=64)
    gk, gv, ok_, ov = H.specs(wl)
    cache = H.new_cache(wl, 192, gk, gv, gpu)
    out = torch.full((1, 0, 2, 128), 7.0, device=gpu)
    assert cache.dequantize("k", out=out).numel() == 0
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    cache.append(k[:, :100].to(gpu), v[:, :100].to(gpu))
    cache.append(k[:, 100:].contiguous().to(gpu), v[:, 100:].contiguous().to(gpu))
    for nm, x, spec in (("k", k.numpy(), ok_), ("v", v.numpy(), ov)):
        got = cache.dequantize(nm).cpu().numpy()
        exp = _expected_plain(OL.encode_plane(x, spec), OL.tail_ring(x, 64), spec, 150, 64)
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), nm
