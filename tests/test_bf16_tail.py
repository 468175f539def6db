"""GPU parity of the bfloat16 precision tail (the release notes' other tail
format) against the oracle.

 - device append writes the tail ring bit-exactly as the oracle's bfloat16
   ring (round to nearest even of the binary32 input), body codes unchanged;
 - decode over a cache with bfloat16 tails matches the oracle's decode over
   the same cache (plain, KVarN and low-rank bodies; T below, at and above
   the tail length), within the decode tolerance;
 - the read-back returns the bfloat16 values exactly;
 - a transcode keeps sharing the tails (same format)."""

import numpy as np
import pytest
import torch

import oracle.layer as OL
import synth
from quantized_kv_cache_kvq_amd.cache import LayerCache
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _cache(wl, capacity, gk, gv, gpu, N):
    return LayerCache(wl.B, wl.Hkv, capacity, N, gk, gv, gpu, tail_format="bf16")


def test_append_writes_bf16_ring(gpu):
    wl = synth.WORKLOADS["gqa4_q8k_q4v_tail1024"].with_(B=2, Hkv=2, Hq=8, T=400, N=128)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    gk, gv, ok_, ov = H.specs(wl)
    cache = _cache(wl, 448, gk, gv, gpu, 128)
    for a, b in ((0, 300), (300, 399), (399, 400)):
        cache.append(k[:, a:b].contiguous().to(gpu), v[:, a:b].contiguous().to(gpu))
    torch.cuda.synchronize()
    for name, x, spec in (("k", k.numpy(), ok_), ("v", v.numpy(), ov)):
        dev = H.download(cache, name)
        ring = OL.tail_ring(x, 128, fmt="bf16")
        assert np.array_equal(dev["tail"], OL.pack_tail(ring, fmt="bf16")), name
        packed = OL.pack_plane(OL.encode_plane(x, spec), spec, 448)
        assert np.array_equal(dev["codes"][: packed["codes"].size], packed["codes"]), name
        got = cache.dequantize(name).cpu().numpy()
        for t in range(400 - 128, 400):
            assert np.array_equal(got[:, t], ring[:, :, t % 128, :]), (name, t)


CASES = [("gqa4_q8k_q4v_tail1024", 1, 128), ("gqa4_q8k_q4v_tail1024", 100, 128),
         ("gqa4_q8k_q4v_tail1024", 128, 128), ("gqa4_q8k_q4v_tail1024", 700, 256),
         ("kvarn_q3_tail2048", 900, 256), ("lowrank_1bpd", 333, 64)]


@pytest.mark.parametrize("name,T,N", CASES)
def test_decode_with_bf16_tail(gpu, name, T, N):
    wl = synth.WORKLOADS[name].with_(T=T, N=N)
    if name != "lowrank_1bpd":
        wl = wl.with_(B=2, Hkv=4, Hq=16)
    else:
        wl = wl.with_(B=2)
    k = synth.layer_rows(wl, 0, "k").numpy()
    v = synth.layer_rows(wl, 0, "v").numpy()
    q = synth.queries(wl, 0)
    gk, gv, ok_, ov = H.specs(wl)
    cap = (T + 63) // 64 * 64
    cache = _cache(wl, cap, gk, gv, gpu, N)
    rings = {}
    for nm, x, spec in (("k", k, ok_), ("v", v, ov)):
        packed = OL.pack_plane(OL.encode_plane(x, spec), spec, cap)
        rings[nm] = OL.tail_ring(x, N, fmt="bf16")
        H.upload(cache, nm, packed, OL.pack_tail(rings[nm], fmt="bf16"))
    cache.n_tokens = T
    kenc, venc = OL.encode_plane(k, ok_), OL.encode_plane(v, ov)
    ref = OL.decode(q.numpy(), kenc, venc, rings["k"], rings["v"], ok_, ov, T, N, wl.sm_scale)
    bound = H.decode_bound(q.numpy(), kenc, venc, rings["k"], rings["v"], ok_, ov, T, N, wl.sm_scale,
                           tail_fmt="bf16")
    for splits in (0, 3):
        out = cache.decode(q.to(gpu), wl.sm_scale, body_splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(got - ref)))
        assert err <= H.ATOL, (name, T, N, splits, err)
        H.check_precision(got, ref, bound, "%s T=%d N=%d bf16 splits=%d" % (name, T, N, splits))
    print("%s T=%d N=%d bf16 tail: max-abs %.2e" % (name, T, N, err))


def test_transcode_keeps_bf16_tail(gpu):
    """A degrade step re-encodes the body and keeps the (shared) bfloat16
    tails: decode of the new layer equals the oracle's decode over the
    oracle's transcode of the same body with the same rings."""
    wl = synth.WORKLOADS["vbr_32layer"].with_(B=1, Hkv=2, Hq=8, T=200, N=64)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    gk, gv, oks, ovs = H.specs(wl, kcodec="f16", vcodec="f16")
    cache = _cache(wl, 256, gk, gv, gpu, 64)
    cache.append(k.to(gpu), v.to(gpu))
    dst = cache.transcode("q8_0", "q8_0")
    torch.cuda.synchronize()
    assert dst.tail_format == "bf16" and dst.bufs["k"]["tail"] is cache.bufs["k"]["tail"]
    _, _, okd, ovd = H.specs(wl, kcodec="q8_0", vcodec="q8_0")
    kn, vn = k.numpy(), v.numpy()
    kenc = OL.transcode_plane(OL.encode_plane(kn, oks), oks, okd)
    venc = OL.transcode_plane(OL.encode_plane(vn, ovs), ovs, ovd)
    q = synth.queries(wl, 0)
    ref = OL.decode(q.numpy(), kenc, venc, OL.tail_ring(kn, 64, fmt="bf16"),
                    OL.tail_ring(vn, 64, fmt="bf16"), okd, ovd, 200, 64, wl.sm_scale)
    out = dst.decode(q.to(gpu), wl.sm_scale)
    torch.cuda.synchronize()
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)))
    assert err <= H.ATOL, err
