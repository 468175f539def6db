"""The allocation-free one-call step (kvq_append_decode_noalloc) through the
C ABI against the step with a caller workspace (kvq_append_decode): two
calls in a row on one GPU, the second on a smaller layer, each leaving the
same cache bytes (bit-exact) and outputs within the parity tolerance of the
other entry point's and of the oracle; and the size limit."""

import ctypes

import numpy as np
import pytest
import torch

import oracle.layer as OL
import synth
from quantized_kv_cache_kvq_amd import lib
from quantized_kv_cache_kvq_amd.cache import _ptr, _stream
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _pair(gpu, wl, capacity):
    """Two identical device caches holding tokens 0 .. T-2 of the workload."""
    gk, gv, ok_, ov = H.specs(wl)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    caches = []
    for _ in range(2):
        c = H.new_cache(wl, capacity, gk, gv, gpu)
        c.append(k[:, : wl.T - 1].to(gpu), v[:, : wl.T - 1].to(gpu))
        caches.append(c)
    return caches, k, v, ok_, ov


@pytest.mark.parametrize("wl", [
    synth.WORKLOADS["gqa4_q8k_q4v_tail1024"].with_(T=3000, N=256),
    synth.WORKLOADS["kvarn_q3_tail2048"].with_(B=1, Hkv=2, Hq=12, T=700, N=64),
])
def test_noalloc_step_equals_workspace_step(gpu, wl):
    caches, k, v, ok_, ov = _pair(gpu, wl, (wl.T + 63) // 64 * 64)
    q = synth.queries(wl, 0)
    kn = k[:, wl.T - 1:].contiguous().to(gpu)
    vn = v[:, wl.T - 1:].contiguous().to(gpu)
    qd = q.to(gpu)
    out_ws = caches[0].append_decode(kn, vn, qd, wl.sm_scale)
    out_na = torch.empty_like(qd)
    st = _stream(gpu, None)
    # twice in a row on the scratch array: the second call must see no
    # trace of the first
    for rep in range(2):
        c = caches[1]
        c.n_tokens = wl.T - 1
        lib.append_decode_noalloc(c.desc, _ptr(kn), _ptr(vn), _ptr(qd), wl.Hq, wl.sm_scale, _ptr(out_na), st)
        c.n_tokens = wl.T
        torch.cuda.synchronize()
        for name in ("k", "v"):
            a, b = H.download(caches[0], name), H.download(caches[1], name)
            for key in ("codes", "scales", "mins", "tail"):
                if a[key] is not None:
                    assert np.array_equal(a[key], b[key]), (rep, name, key)
        got, want = out_na.cpu().numpy().astype(np.float64), out_ws.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got - want)) <= 1e-5, rep
        kenc, _ = H.unpack(caches[1], "k", ok_, wl.T)
        venc, _ = H.unpack(caches[1], "v", ov, wl.T)
        kx, vx = k.numpy(), v.numpy()
        kt = OL.tail_ring(kx, wl.N) if wl.N else None
        vt = OL.tail_ring(vx, wl.N) if wl.N else None
        ref = OL.decode(q.numpy(), kenc, venc, kt, vt, ok_, ov, wl.T, wl.N, wl.sm_scale)
        assert np.max(np.abs(got - ref)) <= H.ATOL
        H.check_precision(got, ref, H.decode_bound(q.numpy(), kenc, venc, kt, vt, ok_, ov, wl.T, wl.N,
                                                   wl.sm_scale), "noalloc %s rep %d" % (wl.name, rep))


def test_noalloc_rejects_steps_above_its_scratch(gpu):
    """512 sequences x 64 query heads need more than the fixed 16 MiB: the
    call fails before enqueueing anything (the cache is left as it was)."""
    wl = synth.WORKLOADS["gqa4_q8k_q4v_tail1024"].with_(B=512, Hq=64, T=32, N=0)
    gk, gv, _, _ = H.specs(wl)
    c = H.new_cache(wl, 64, gk, gv, gpu)
    c.n_tokens = 31
    kn = torch.ones((wl.B, 1, wl.Hkv, 128), device=gpu)
    q = torch.ones((wl.B, wl.Hq, 128), device=gpu)
    out = torch.empty_like(q)
    before = c.bufs["k"]["codes"].clone()
    with pytest.raises(lib.KvqError) as ei:
        lib.append_decode_noalloc(c.desc, _ptr(kn), _ptr(kn), _ptr(q), wl.Hq, 1.0, _ptr(out),
                                  _stream(gpu, None))
    assert ei.value.status == lib.KVQ_ERR_WORKSPACE and "16777216" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.equal(before, c.bufs["k"]["codes"])
