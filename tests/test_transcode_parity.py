"""GPU parity of the layer transcode (VBR degrade step) against the oracle:
the source planes are the oracle's packed encoding, the device re-encodes
them, and the destination bytes must equal the oracle's transcode bit for
bit (decode is exact or a single binary32 rounding, encode is the block
quantiser).  The tails are untouched and shared."""

import numpy as np
import pytest
import torch

import oracle.layer as OL
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

PAIRS = [("f16", "q8_0"), ("f16", "q4_0"), ("f16", "q2_0"), ("q8_0", "q4_0"), ("q4_0", "q2_0"),
         ("q8_1", "q3_1"), ("q4_1", "q2_0"), ("q6_0", "q5_1"), ("q3_0", "q1_1"), ("q4_0", "f16"),
         ("q2_1", "q2_1")]


@pytest.mark.parametrize("src,dst", PAIRS)
@pytest.mark.parametrize("basis", ["plain", "hadamard"])
def test_transcode_bit_exact(gpu, src, dst, basis):
    name = "vbr_32layer" if basis == "plain" else "kvarn_q3_tail2048"
    wl = synth.WORKLOADS[name].with_(B=2, Hkv=2, Hq=8, T=333, N=64)
    k = synth.layer_rows(wl, 0, "k").numpy()
    v = synth.layer_rows(wl, 0, "v").numpy()
    gk, gv, ok_, ov = H.specs(wl, kcodec=src, vcodec=src)
    cache = H.new_cache(wl, 384, gk, gv, gpu)
    kenc, kp, kt = H.oracle_layer_bytes(k, ok_, 384, wl.N)
    venc, vp, vt = H.oracle_layer_bytes(v, ov, 384, wl.N)
    H.upload(cache, "k", kp, kt)
    H.upload(cache, "v", vp, vt)
    cache.n_tokens = wl.T
    out = cache.transcode(dst, dst)
    torch.cuda.synchronize()
    assert out.bufs["k"]["tail"] is cache.bufs["k"]["tail"]
    _, _, okd, ovd = H.specs(wl, kcodec=dst, vcodec=dst)
    for name_, enc, sspec, dspec in (("k", kenc, ok_, okd), ("v", venc, ov, ovd)):
        want = OL.pack_plane(OL.transcode_plane(enc, sspec, dspec), dspec, 384)
        got = H.download(out, name_)
        n = wl.B * wl.Hkv
        R = want["codes"].size // n
        for p in range(n):          # rows beyond T are not written by transcode
            rows_w = want["codes"][p * R:(p + 1) * R]
            rows_g = got["codes"][p * R:(p + 1) * R]
            Rb = R // 384
            from oracle.layout import untile_plane
            assert np.array_equal(untile_plane(rows_g, Rb)[: wl.T], untile_plane(rows_w, Rb)[: wl.T])
        if want["scales"] is not None:
            nb = want["scales"].size // (n * 384)
            sw = want["scales"].reshape(n, 384, nb)[:, : wl.T]
            sg = got["scales"].reshape(n, 384, nb)[:, : wl.T]
            assert np.array_equal(sg, sw)
        if want["mins"] is not None:
            nb = want["mins"].size // (n * 384)
            assert np.array_equal(got["mins"].reshape(n, 384, nb)[:, : wl.T],
                                  want["mins"].reshape(n, 384, nb)[:, : wl.T])


def test_transcode_then_decode(gpu):
    """f16 layer degraded to q8_0 on the device decodes like the oracle's
    q8_0 encoding of the binary16 values."""
    wl = synth.WORKLOADS["vbr_32layer"].with_(T=900, N=0)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    gk, gv, ok_, ov = H.specs(wl, kcodec="f16", vcodec="f16")
    cache = H.new_cache(wl, 1024, gk, gv, gpu, N=0)
    cache.append(k.to(gpu), v.to(gpu))
    q8 = cache.transcode("q8_0", "q8_0")
    q = synth.queries(wl, 0)
    out = q8.decode(q.to(gpu), wl.sm_scale).cpu().numpy()
    _, _, o8, _ = H.specs(wl, kcodec="q8_0", vcodec="q8_0")
    kf = k.numpy().astype(np.float16).astype(np.float32)
    vf = v.numpy().astype(np.float16).astype(np.float32)
    ref = OL.decode(q.numpy(), OL.encode_plane(kf, o8), OL.encode_plane(vf, o8), None, None,
                    o8, o8, 900, 0, wl.sm_scale)
    assert np.max(np.abs(out - ref)) <= H.ATOL
