"""GPU parity of the one-call decode step (kvq_append_decode): append one
token per sequence and decode over the cache with it.

For each case a layer holding T0 tokens (the oracle's encoding, uploaded)
takes one step; then
 - its stored bytes (codes, scales, mins, tail ring) equal the oracle's
   encoding of the T0 + 1 tokens bit for bit;
 - its output equals, bit for bit, that of a twin layer that ran the append
   and the decode as two calls, and the oracle's decode over T0 + 1 tokens
   within the decode tolerance.
Cases: the new token landing in the tail ring (T0 below, at and past the
tail length, slot wrap), no tail (the new row read by the last body split),
plain and KVarN bodies, 3/5/6-bit rows (LDS packing inside the launch),
binary16 and bfloat16 tails, a ragged batch, two head groups per kv head
(the owner workgroup of each group writes the same row), and low-rank
layers (the launch projects and quantises the new rows and the query)."""

import numpy as np
import pytest
import torch

import oracle.layer as OL
import synth
from quantized_kv_cache_kvq_amd.cache import LayerCache
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _layer(wl, cap, gk, gv, gpu, N, fmt):
    return LayerCache(wl.B, wl.Hkv, cap, N, gk, gv, gpu, tail_format=fmt)


def _upload(cache, name, x, spec, Ts, N, cap, fmt):
    B, _, Hkv, _ = x.shape
    enc = [[OL.encode_head(x[b, :Ts[b], h, :], spec, h) for h in range(Hkv)] for b in range(B)]
    tail = None
    if N > 0:
        ring = np.concatenate([OL.tail_ring(x[b:b + 1, :Ts[b]], N, fmt=fmt) for b in range(B)])
        tail = OL.pack_tail(ring, fmt=fmt)
    H.upload(cache, name, OL.pack_plane(enc, spec, cap), tail)


CASES = [
    # name, kcodec, vcodec, Hq, T0, N, tail format, ragged
    ("gqa4_q8k_q4v_tail1024", None, None, 8, 300, 128, "f16", False),
    ("gqa4_q8k_q4v_tail1024", None, None, 8, 127, 128, "f16", False),
    ("gqa4_q8k_q4v_tail1024", None, None, 8, 128, 128, "f16", False),
    ("gqa4_q8k_q4v_tail1024", None, None, 8, 0, 64, "f16", False),
    ("gqa4_q8k_q4v_tail1024", "q4_0", "q4_0", 8, 700, 0, "f16", False),
    ("gqa4_q8k_q4v_tail1024", "q6_0", "q6_0", 8, 257, 0, "f16", False),
    ("gqa4_q8k_q4v_tail1024", "q5_1", "q5_1", 8, 64, 64, "f16", False),
    ("gqa4_q8k_q4v_tail1024", "q8_0", "q3_0", 12, 333, 64, "bf16", False),
    ("kvarn_q3_tail2048", None, None, 12, 500, 128, "f16", False),
    ("vbr_32layer", "f16", "f16", 8, 190, 64, "f16", False),
    ("gqa4_q8k_q4v_tail1024", None, None, 8, 0, 128, "f16", True),
    ("gqa4_q8k_q4v_tail1024", "q4_0", "q4_0", 8, 0, 0, "f16", True),
    ("gqa4_q8k_q4v_tail1024", None, None, 32, 200, 64, "f16", False),   # two head groups
]


@pytest.mark.parametrize("name,kc,vc,Hq,T0,N,fmt,ragged", CASES)
def test_step_matches_two_calls_and_oracle(gpu, name, kc, vc, Hq, T0, N, fmt, ragged):
    B = 3 if ragged else 2
    Ts = [T0 + 90, T0 + 7, T0] if ragged else [T0] * B
    wl = synth.WORKLOADS[name].with_(B=B, Hkv=2, Hq=Hq, T=max(Ts) + 1, N=N)
    k = synth.layer_rows(wl, 0, "k").numpy()
    v = synth.layer_rows(wl, 0, "v").numpy()
    q = synth.queries(wl, 0)
    gk, gv, ok_, ov = H.specs(wl, kcodec=kc, vcodec=vc)
    cap = (max(Ts) + 1 + 63) // 64 * 64
    kn = torch.from_numpy(np.stack([k[b, Ts[b]:Ts[b] + 1] for b in range(B)])).to(gpu)
    vn = torch.from_numpy(np.stack([v[b, Ts[b]:Ts[b] + 1] for b in range(B)])).to(gpu)
    outs, caches = [], []
    for fused in (True, False):
        c = _layer(wl, cap, gk, gv, gpu, N, fmt)
        _upload(c, "k", k, ok_, Ts, N, cap, fmt)
        _upload(c, "v", v, ov, Ts, N, cap, fmt)
        c.n_tokens = max(Ts)
        if ragged:
            c.set_seq_tokens(torch.tensor(Ts, dtype=torch.int32, device=gpu))
        if fused:
            out = c.append_decode(kn, vn, q.to(gpu), wl.sm_scale)
        else:
            c.append(kn, vn)
            out = c.decode(q.to(gpu), wl.sm_scale)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        caches.append(c)
    assert np.array_equal(outs[0], outs[1]), "one-call step differs from append + decode"
    T1 = [t + 1 for t in Ts]
    for name_, x, spec in (("k", k, ok_), ("v", v, ov)):
        dev = H.download(caches[0], name_)
        if spec.basis == "hadamard":
            # rotated rows: the tie rule on the new row (equal counts here)
            encs, _ = H.unpack(caches[0], name_, spec, T1[0])
            for b in range(B):
                for h in range(2):
                    H.check_rotated_head(x[b, :T1[b], h, :], encs[b][h], spec, h)
        else:
            enc = [[OL.encode_head(x[b, :T1[b], h, :], spec, h) for h in range(2)] for b in range(B)]
            packed = OL.pack_plane(enc, spec, cap)
            assert np.array_equal(dev["codes"][: packed["codes"].size], packed["codes"]), name_
            for key in ("scales", "mins"):
                if packed.get(key) is not None:
                    assert np.array_equal(dev[key], packed[key]), (name_, key)
        if N > 0:
            ring = np.concatenate([OL.tail_ring(x[b:b + 1, :T1[b]], N, fmt=fmt) for b in range(B)])
            assert np.array_equal(dev["tail"], OL.pack_tail(ring, fmt=fmt)), name_
    ref = np.zeros(outs[0].shape)
    bound = np.zeros(outs[0].shape)
    for b in range(B):
        kb, vb = k[b:b + 1, :T1[b]], v[b:b + 1, :T1[b]]
        ke, ve = OL.encode_plane(kb, ok_), OL.encode_plane(vb, ov)
        kt = OL.tail_ring(kb, N, fmt=fmt) if N else None
        vt = OL.tail_ring(vb, N, fmt=fmt) if N else None
        ref[b] = OL.decode(q.numpy()[b:b + 1], ke, ve, kt, vt, ok_, ov, T1[b], N, wl.sm_scale)[0]
        bound[b] = H.decode_bound(q.numpy()[b:b + 1], ke, ve, kt, vt, ok_, ov, T1[b], N, wl.sm_scale,
                                  tail_fmt=fmt)[0]
    err = float(np.max(np.abs(outs[0].astype(np.float64) - ref)))
    assert err <= H.ATOL, err
    H.check_precision(outs[0], ref, bound, "%s %s/%s Hq=%d N=%d %s" % (name, kc, vc, Hq, N, fmt))


LR_CASES = [
    # Hq, T0, N, ragged
    (32, 300, 0, False),      # the new row read by the last body split
    (32, 127, 128, False),    # the new token in the tail ring, slot 127
    (32, 300, 64, False),     # ring wrapped
    (128, 200, 0, False),     # two head groups per kv head (both owners write the row)
    (32, 150, 64, True),      # ragged batch
]


@pytest.mark.parametrize("Hq,T0,N,ragged", LR_CASES)
def test_lowrank_step_one_launch(gpu, Hq, T0, N, ragged):
    """Low-rank layer: the step's launch writes the new token's projected,
    per-head-quantised rows and tail copy itself and projects the query in
    its body workgroups.  Cache bytes and output equal the append + decode
    calls bit for bit; the new rows follow the oracle under the tie rule;
    the output matches the oracle's decode."""
    B = 3 if ragged else 2
    Ts = [T0 + 40, T0 + 3, T0] if ragged else [T0] * B
    wl = synth.WORKLOADS["lowrank_1bpd"].with_(B=B, Hq=Hq, T=max(Ts) + 1, N=N)
    k = synth.layer_rows(wl, 0, "k").numpy()
    v = synth.layer_rows(wl, 0, "v").numpy()
    q = synth.queries(wl, 0)
    gk, gv, ok_, ov = H.specs(wl)
    cap = (max(Ts) + 1 + 63) // 64 * 64
    kn = torch.from_numpy(np.stack([k[b, Ts[b]:Ts[b] + 1] for b in range(B)])).to(gpu)
    vn = torch.from_numpy(np.stack([v[b, Ts[b]:Ts[b] + 1] for b in range(B)])).to(gpu)
    outs, caches = [], []
    for fused in (True, False):
        c = _layer(wl, cap, gk, gv, gpu, N, "f16")
        _upload(c, "k", k, ok_, Ts, N, cap, "f16")
        _upload(c, "v", v, ov, Ts, N, cap, "f16")
        c.n_tokens = max(Ts)
        if ragged:
            c.set_seq_tokens(torch.tensor(Ts, dtype=torch.int32, device=gpu))
        if fused:
            out = c.append_decode(kn, vn, q.to(gpu), wl.sm_scale)
        else:
            c.append(kn, vn)
            out = c.decode(q.to(gpu), wl.sm_scale)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        caches.append(c)
    assert np.array_equal(outs[0], outs[1]), "one-call step differs from append + decode"
    T1 = [t + 1 for t in Ts]
    for name_, x, spec in (("k", k, ok_), ("v", v, ov)):
        d0, d1 = H.download(caches[0], name_), H.download(caches[1], name_)
        for key in d0:
            if d0[key] is not None:
                assert np.array_equal(d0[key], d1[key]), (name_, key)
        encs, _ = H.unpack(caches[0], name_, spec, max(T1))
        mism = 0
        for b in range(B):
            for h in range(wl.Hkv):
                e = {kk: (vv[T1[b] - 1:T1[b]] if isinstance(vv, np.ndarray) else vv) for kk, vv in encs[b][h].items()}
                n, _ = H.check_rotated_head(x[b, T1[b] - 1:T1[b], h, :], e, spec, h, max_frac=1.0)
                mism += n
        assert mism <= 4, (name_, mism)
        if N > 0:
            ring = np.concatenate([OL.tail_ring(x[b:b + 1, :T1[b]], N) for b in range(B)])
            assert np.array_equal(d0["tail"], OL.pack_tail(ring)), name_
    ref = np.zeros(outs[0].shape)
    bound = np.zeros(outs[0].shape)
    for b in range(B):
        kb, vb = k[b:b + 1, :T1[b]], v[b:b + 1, :T1[b]]
        ke, ve = OL.encode_plane(kb, ok_), OL.encode_plane(vb, ov)
        kt = OL.tail_ring(kb, N) if N else None
        vt = OL.tail_ring(vb, N) if N else None
        ref[b] = OL.decode(q.numpy()[b:b + 1], ke, ve, kt, vt, ok_, ov, T1[b], N, wl.sm_scale)[0]
        bound[b] = H.decode_bound(q.numpy()[b:b + 1], ke, ve, kt, vt, ok_, ov, T1[b], N, wl.sm_scale)[0]
    err = float(np.max(np.abs(outs[0].astype(np.float64) - ref)))
    assert err <= H.ATOL, err
    H.check_precision(outs[0], ref, bound, "lowrank Hq=%d T0=%d N=%d ragged=%s" % (Hq, T0, N, ragged))
