"""The decode step replayed as a HIP graph (how the benchmark and a serving
loop drive it): every replay gives exactly the eager step's output and
cache bytes.  Replays are separated by eager work and synchronisations, and
each is checked on its own."""

import numpy as np
import pytest
import torch

import synth
from quantized_kv_cache_kvq_amd.cache import LayerCache, PlaneSpec
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _bytes(c):
    return {n: {k: (v.clone() if v is not None else None) for k, v in c.bufs[n].items()} for n in ("k", "v")}


def _same(a, b):
    for n in a:
        for k in a[n]:
            if a[n][k] is not None:
                assert torch.equal(a[n][k], b[n][k]), (n, k)


@pytest.mark.parametrize("name,N,Hq,transcode", [("gqa4_q8k_q4v_tail1024", 128, 8, False),
                                                  ("gqa4_q8k_q4v_tail1024", 0, 32, False),
                                                  ("vbr_32layer", 64, 8, True),
                                                  ("lowrank_1bpd", 0, 32, False)])
def test_graph_replays_equal_eager(gpu, name, N, Hq, transcode):
    T = 777
    wl = synth.WORKLOADS[name].with_(B=2, T=T, N=N)
    if name != "lowrank_1bpd":
        wl = wl.with_(Hkv=2, Hq=Hq)
    kc = "f16" if transcode else None
    gk, gv, _, _ = H.specs(wl, kcodec=kc, vcodec=kc)
    k = synth.layer_rows(wl, 0, "k").to(gpu)
    v = synth.layer_rows(wl, 0, "v").to(gpu)
    q = synth.queries(wl, 0).to(gpu)
    cap = (T + 63) // 64 * 64
    cache = LayerCache(wl.B, wl.Hkv, cap, N, gk, gv, gpu)
    cache.append(k[:, : T - 1].contiguous(), v[:, : T - 1].contiguous())
    kn, vn = k[:, T - 1:].contiguous(), v[:, T - 1:].contiguous()
    dst = None
    if transcode:
        dst = LayerCache(wl.B, wl.Hkv, cap, N, PlaneSpec("q8_0"), PlaneSpec("q8_0"), gpu,
                         share_tail_with=cache)
    out = torch.empty_like(q)

    def step():
        cache.n_tokens = T - 1
        cache.append_decode(kn, vn, q, wl.sm_scale, out=out)
        if dst is not None:
            cache.transcode_into(dst)

    step()
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref_cache = _bytes(cache)
    ref_dst = _bytes(dst) if dst is not None else None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.zero_()
        junk = torch.randn(1 << 16, device=gpu).sum()     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        assert torch.equal(out, ref_out), "replay %d output differs from the eager step" % r
        _same(ref_cache, _bytes(cache))
        if dst is not None:
            _same(ref_dst, _bytes(dst))
    assert np.isfinite(out.cpu().numpy()).all()
