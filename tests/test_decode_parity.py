"""GPU parity of decode attention against the fp64 oracle run on the same
cache.  The oracle encodes the seeded inputs, the packed bytes are uploaded
into the device planes, the library decodes, and the outputs must agree
within max-abs 2e-3.  Covers every workload's basis, every compiled codec
pair, query-group sizes 1..16, ragged token counts around tile and tail
boundaries (T = 1, T < N, T = N, T = N + 1, ...), several split counts and
split-count invariance."""

import numpy as np
import pytest
import torch

import oracle.layer as OL
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _run(gpu, wl, T, N, capacity, kc=None, vc=None, splits=(0,), seed_step=0, Hq=None):
    wl = wl.with_(T=T, N=N) if Hq is None else wl.with_(T=T, N=N, Hq=Hq)
    k = synth.layer_rows(wl, 0, "k").numpy()
    v = synth.layer_rows(wl, 0, "v").numpy()
    q = synth.queries(wl, 0, step=seed_step)
    gk, gv, ok_, ov = H.specs(wl, kcodec=kc, vcodec=vc)
    cache = H.new_cache(wl, capacity, gk, gv, gpu, N=N)
    kenc, kp, kt = H.oracle_layer_bytes(k, ok_, capacity, N)
    venc, vp, vt = H.oracle_layer_bytes(v, ov, capacity, N)
    H.upload(cache, "k", kp, kt)
    H.upload(cache, "v", vp, vt)
    cache.n_tokens = T
    ref = OL.decode(q.numpy(), kenc, venc, OL.tail_ring(k, N) if N else None,
                    OL.tail_ring(v, N) if N else None, ok_, ov, T, N, wl.sm_scale)
    bound = H.decode_bound(q.numpy(), kenc, venc, OL.tail_ring(k, N) if N else None,
                           OL.tail_ring(v, N) if N else None, ok_, ov, T, N, wl.sm_scale)
    outs = []
    for s in splits:
        out = cache.decode(q.to(gpu), wl.sm_scale, body_splits=s)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        err = np.max(np.abs(got - ref))
        assert err <= H.ATOL, (wl.name, T, N, kc, vc, s, err)
        H.check_precision(got, ref, bound, "%s T=%d N=%d %s/%s splits=%d" % (wl.name, T, N, kc, vc, s))
        outs.append(got)
    return outs


@pytest.mark.parametrize("T", [1, 63, 256, 257, 700])
def test_tiny_workload(gpu, T):
    _run(gpu, synth.WORKLOADS["tiny"], T, 0, 768, splits=(0, 1, 3))


@pytest.mark.parametrize("T,N", [(1, 1024), (500, 1024), (1024, 1024), (1025, 1024),
                                 (3000, 1024), (2049, 128), (1300, 0)])
def test_gqa4_q8k_q4v(gpu, T, N):
    _run(gpu, synth.WORKLOADS["gqa4_q8k_q4v_tail1024"], T, N, 3072, splits=(0, 1, 5))


@pytest.mark.parametrize("T,N", [(900, 256), (256, 256), (1500, 0)])
def test_kvarn_q3(gpu, T, N):
    wl = synth.WORKLOADS["kvarn_q3_tail2048"].with_(B=2)
    _run(gpu, wl, T, N, 1536, splits=(0, 2))


@pytest.mark.parametrize("T", [1, 300, 777])
def test_lowrank(gpu, T):
    wl = synth.WORKLOADS["lowrank_1bpd"].with_(B=2)
    _run(gpu, wl, T, 0, 832, splits=(0, 3))


def test_lowrank_with_tail(gpu):
    wl = synth.WORKLOADS["lowrank_1bpd"].with_(B=1)
    _run(gpu, wl, 600, 128, 640)


PAIRS = [("f16", "f16"), ("q8_0", "q8_0"), ("q6_0", "q6_0"), ("q5_0", "q5_0"),
         ("q4_0", "q4_0"), ("q3_0", "q3_0"), ("q2_0", "q2_0"), ("q8_1", "q8_1"),
         ("q6_1", "q6_1"), ("q5_1", "q5_1"), ("q4_1", "q4_1"), ("q3_1", "q3_1"),
         ("q2_1", "q2_1"), ("q1_1", "q1_1"), ("q8_0", "q4_0"), ("q8_0", "q3_0"),
         ("q8_0", "q2_0"), ("q6_0", "q4_0"), ("q4_0", "q2_0"), ("q8_1", "q4_1"),
         ("f16", "q8_0"), ("f16", "q4_0")]


@pytest.mark.parametrize("kc,vc", PAIRS)
def test_codec_pairs(gpu, kc, vc):
    wl = synth.WORKLOADS["vbr_32layer"].with_(Hkv=2, Hq=8)
    _run(gpu, wl, 650, 128, 768, kc=kc, vc=vc, splits=(0, 2))


@pytest.mark.parametrize("kc,vc", [("q8_0", "q4_0"), ("q8_0", "q3_0"), ("q8_0", "q2_0"),
                                   ("q8_1", "q4_1"), ("q1_1", "q1_1")])
def test_cancelling_values_low_bit(gpu, kc, vc):
    """Value codes of at most 4 bits reach the PV matrix cores unsigned,
    with the _0 offset (or the _1 minimum) added as a separate per-block
    term.  Values that alternate in sign token by token, at the codes'
    extremes, under near-uniform weights make the output a small difference
    of large sums: it must still match the oracle within the tolerance and
    the derived bound."""
    wl = synth.WORKLOADS["vbr_32layer"].with_(Hkv=2, Hq=8, T=700, N=64)
    T, N, cap = 700, 64, 768
    rng = np.random.default_rng(11)
    k = (0.01 * rng.standard_normal((1, T, 2, 128))).astype(np.float32)
    sign = np.where(np.arange(T) % 2 == 0, 1.0, -1.0)[None, :, None, None]
    v = (sign * (1.0 + 0.001 * rng.standard_normal((1, T, 2, 128)))).astype(np.float32)
    q = synth.queries(wl, 0)
    gk, gv, ok_, ov = H.specs(wl, kcodec=kc, vcodec=vc)
    cache = H.new_cache(wl, cap, gk, gv, gpu, N=N)
    kenc, kp, kt = H.oracle_layer_bytes(k, ok_, cap, N)
    venc, vp, vt = H.oracle_layer_bytes(v, ov, cap, N)
    H.upload(cache, "k", kp, kt)
    H.upload(cache, "v", vp, vt)
    cache.n_tokens = T
    ref = OL.decode(q.numpy(), kenc, venc, OL.tail_ring(k, N), OL.tail_ring(v, N), ok_, ov, T, N,
                    wl.sm_scale)
    bound = H.decode_bound(q.numpy(), kenc, venc, OL.tail_ring(k, N), OL.tail_ring(v, N), ok_, ov,
                           T, N, wl.sm_scale)
    for splits in (0, 3):
        out = cache.decode(q.to(gpu), wl.sm_scale, body_splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got - ref)) <= H.ATOL, (vc, splits)
        H.check_precision(got, ref, bound, "cancelling values %s splits=%d" % (vc, splits))


@pytest.mark.parametrize("Hq", [2, 4, 6, 12, 16, 24])
def test_group_sizes(gpu, Hq):
    wl = synth.WORKLOADS["vbr_32layer"].with_(Hkv=2, Hq=Hq)
    _run(gpu, wl, 400, 64, 512, kc="q8_0", vc="q4_0")


def test_hadamard_group6_other_codec(gpu):
    wl = synth.WORKLOADS["kvarn_q3_tail2048"].with_(B=1)
    _run(gpu, wl, 500, 128, 512, kc="q4_0", vc="q4_0")


def test_split_count_invariance(gpu):
    outs = _run(gpu, synth.WORKLOADS["gqa4_q8k_q4v_tail1024"], 4000, 256, 4096,
                splits=(0, 1, 2, 7, 15))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-5


def test_uniform_keys_give_value_mean(gpu):
    """Identical keys: every weight equal, the output is the mean of the
    dequantised values (oracle-free property)."""
    wl = synth.WORKLOADS["gqa4_q8k_q4v_tail1024"].with_(Hkv=1, Hq=4, T=300, N=0)
    k = np.repeat(synth.layer_rows(wl, 0, "k", T=1).numpy(), 300, axis=1)
    v = synth.layer_rows(wl, 0, "v").numpy()
    gk, gv, ok_, ov = H.specs(wl)
    cache = H.new_cache(wl, 320, gk, gv, gpu, N=0)
    cache.append(torch.from_numpy(k).to(gpu), torch.from_numpy(v).to(gpu))
    out = cache.decode(synth.queries(wl, 0).to(gpu), 1.0).cpu().numpy()
    vq = OL.attention_kv(OL.encode_plane(v, ov), None, ov, 300, 0)
    assert np.max(np.abs(out[0] - vq[0, :, 0, :].mean(0))) < 1e-4


def test_workspace_reuse_across_calls_and_shapes(gpu):
    """Splits of one call are merged by whichever workgroup finishes its
    unit last, through the workspace; consecutive calls (new queries, other
    split counts, another layer shape) on one workspace must each see only
    their own partials."""
    wl = synth.WORKLOADS["gqa4_q8k_q4v_tail1024"]
    ws = None
    for T, N, Hq, splits in [(3000, 1024, 32, 0), (2049, 128, 32, 7), (700, 0, 8, 0),
                             (3000, 1024, 32, 3), (1300, 256, 16, 0)]:
        w = wl.with_(T=T, N=N, Hq=Hq)
        k = synth.layer_rows(w, 0, "k").numpy()
        v = synth.layer_rows(w, 0, "v").numpy()
        gk, gv, ok_, ov = H.specs(w)
        cache = H.new_cache(w, 3072, gk, gv, gpu, N=N)
        kenc, kp, kt = H.oracle_layer_bytes(k, ok_, 3072, N)
        venc, vp, vt = H.oracle_layer_bytes(v, ov, 3072, N)
        H.upload(cache, "k", kp, kt)
        H.upload(cache, "v", vp, vt)
        cache.n_tokens = T
        need = cache.workspace(Hq).numel()
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 1 << 24), dtype=torch.uint8, device=gpu)
        for step in range(3):
            q = synth.queries(w, 0, step=step)
            ref = OL.decode(q.numpy(), kenc, venc, OL.tail_ring(k, N) if N else None,
                            OL.tail_ring(v, N) if N else None, ok_, ov, T, N, w.sm_scale)
            out = cache.decode(q.to(gpu), w.sm_scale, body_splits=splits, ws=ws)
            torch.cuda.synchronize()
            err = np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref))
            assert err <= H.ATOL, (T, N, Hq, splits, step, err)
            assert int(ws[: 1 << 16].count_nonzero()) == 0, (T, N, Hq, splits, step)


def test_counters_left_zero_many_units(gpu):
    """Each (batch entry, kv head, head group) has its own completion
    counter (units u and u + 16 share a 4 KiB page at different words);
    with more units than pages every counter must be back at zero after a
    call and the outputs must match the oracle on repeated calls."""
    wl = synth.WORKLOADS["gqa4_q8k_q4v_tail1024"].with_(B=3, T=900, N=128)
    k = synth.layer_rows(wl, 0, "k").numpy()
    v = synth.layer_rows(wl, 0, "v").numpy()
    q = synth.queries(wl, 0)
    gk, gv, ok_, ov = H.specs(wl)
    cache = H.new_cache(wl, 960, gk, gv, gpu, N=128)
    kenc, kp, kt = H.oracle_layer_bytes(k, ok_, 960, 128)
    venc, vp, vt = H.oracle_layer_bytes(v, ov, 960, 128)
    H.upload(cache, "k", kp, kt)
    H.upload(cache, "v", vp, vt)
    cache.n_tokens = wl.T
    ref = OL.decode(q.numpy(), kenc, venc, OL.tail_ring(k, 128), OL.tail_ring(v, 128), ok_, ov,
                    wl.T, 128, wl.sm_scale)
    ws = cache.workspace(wl.Hq)
    for splits in (0, 5, 0):
        out = cache.decode(q.to(gpu), wl.sm_scale, body_splits=splits, ws=ws)
        torch.cuda.synchronize()
        assert np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)) <= H.ATOL, splits
        assert int(ws[: 1 << 16].count_nonzero()) == 0, splits


@pytest.mark.parametrize("N", [0, 128])
def test_lowrank_stale_workspace(gpu, N):
    """Only the counters at the start of a workspace must be zero: a
    workspace whose remaining bytes hold NaN patterns (0xFF) from earlier
    use must give the same low-rank decode, with and without a tail."""
    wl = synth.WORKLOADS["lowrank_1bpd"].with_(B=1, T=600, N=N)
    k = synth.layer_rows(wl, 0, "k").numpy()
    v = synth.layer_rows(wl, 0, "v").numpy()
    q = synth.queries(wl, 0)
    gk, gv, ok_, ov = H.specs(wl)
    cache = H.new_cache(wl, 640, gk, gv, gpu, N=N)
    kenc, kp, kt = H.oracle_layer_bytes(k, ok_, 640, N)
    venc, vp, vt = H.oracle_layer_bytes(v, ov, 640, N)
    H.upload(cache, "k", kp, kt)
    H.upload(cache, "v", vp, vt)
    cache.n_tokens = wl.T
    ref = OL.decode(q.numpy(), kenc, venc, OL.tail_ring(k, N) if N else None,
                    OL.tail_ring(v, N) if N else None, ok_, ov, wl.T, N, wl.sm_scale)
    need = cache.workspace(wl.Hq).numel()
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=gpu)
    ws[: 1 << 16].zero_()
    for splits in (0, 3):
        out = cache.decode(q.to(gpu), wl.sm_scale, body_splits=splits, ws=ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), splits
        assert np.max(np.abs(got - ref)) <= H.ATOL, splits
