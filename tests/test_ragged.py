"""GPU parity for ragged batches (per-sequence token counts, kvq_layer
.seq_tokens): sequences of one layer hold different numbers of tokens.

 - decode: sequence b attends over its own T_b tokens, its tail being the
   newest min(tail_len, T_b) of them; equal to the oracle's decode of that
   sequence alone (T_b = 0 gives zeros), for plain and KVarN bodies and
   split counts that leave some splits empty for the shorter sequences;
 - append: each sequence appends at its own position; codes, scales and the
   tail ring of every sequence equal the oracle's encoding of its tokens,
   and the read-back zeroes rows past a sequence's count."""

import numpy as np
import pytest
import torch

import oracle.layer as OL
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _upload_ragged(cache, name, x, spec, Ts, N, capacity):
    """Oracle bytes of a ragged plane: sequence b holds tokens [0, Ts[b])."""
    B, _, Hkv, _ = x.shape
    enc = [[OL.encode_head(x[b, :Ts[b], h, :], spec, h) for h in range(Hkv)] for b in range(B)]
    packed = OL.pack_plane(enc, spec, capacity)
    tail = None
    if N > 0:
        ring = np.concatenate([OL.tail_ring(x[b:b + 1, :Ts[b]], N) for b in range(B)])
        tail = OL.pack_tail(ring)
    H.upload(cache, name, packed, tail)
    return enc


def _oracle_out(q, kx, vx, ok_, ov, Ts, N, sm_scale):
    out = np.zeros(q.shape, dtype=np.float64)
    for b, T in enumerate(Ts):
        if T == 0:
            continue
        kb, vb = kx[b:b + 1, :T], vx[b:b + 1, :T]
        out[b] = OL.decode(q[b:b + 1], OL.encode_plane(kb, ok_), OL.encode_plane(vb, ov),
                           OL.tail_ring(kb, N) if N else None, OL.tail_ring(vb, N) if N else None,
                           ok_, ov, T, N, sm_scale)[0]
    return out


@pytest.mark.parametrize("name,Ts,N", [("gqa4_q8k_q4v_tail1024", [700, 64, 1, 0], 128),
                                       ("gqa4_q8k_q4v_tail1024", [130, 900, 257, 63], 0),
                                       ("kvarn_q3_tail2048", [600, 200, 0, 513], 128)])
def test_ragged_decode(gpu, name, Ts, N):
    T = max(Ts)
    wl = synth.WORKLOADS[name].with_(B=len(Ts), Hkv=2, Hq=8, T=T, N=N)
    kx = synth.layer_rows(wl, 0, "k").numpy()
    vx = synth.layer_rows(wl, 0, "v").numpy()
    q = synth.queries(wl, 0)
    gk, gv, ok_, ov = H.specs(wl)
    cap = (T + 63) // 64 * 64
    cache = H.new_cache(wl, cap, gk, gv, gpu, N=N)
    _upload_ragged(cache, "k", kx, ok_, Ts, N, cap)
    _upload_ragged(cache, "v", vx, ov, Ts, N, cap)
    cache.n_tokens = T
    cache.set_seq_tokens(torch.tensor(Ts, dtype=torch.int32, device=gpu))
    ref = _oracle_out(q.numpy(), kx, vx, ok_, ov, Ts, N, wl.sm_scale)
    for splits in (0, 5):
        out = cache.decode(q.to(gpu), wl.sm_scale, body_splits=splits).cpu().numpy()
        torch.cuda.synchronize()
        err = float(np.max(np.abs(out.astype(np.float64) - ref)))
        assert err <= H.ATOL, (name, Ts, N, splits, err)
        for b, Tb in enumerate(Ts):
            if Tb == 0:
                assert not np.any(out[b]), "empty sequence must give zeros"


def test_ragged_append_and_readback(gpu):
    Ts0, n = [200, 7, 0], 70
    wl = synth.WORKLOADS["gqa4_q8k_q4v_tail1024"].with_(B=3, Hkv=2, Hq=8, T=max(Ts0) + n, N=64)
    cap = 320
    full_k = synth.layer_rows(wl, 0, "k").numpy()          # stream of each sequence's tokens
    full_v = synth.layer_rows(wl, 0, "v").numpy()
    gk, gv, ok_, ov = H.specs(wl)
    cache = H.new_cache(wl, cap, gk, gv, gpu, N=64)
    _upload_ragged(cache, "k", full_k, ok_, Ts0, 64, cap)
    _upload_ragged(cache, "v", full_v, ov, Ts0, 64, cap)
    cache.n_tokens = max(Ts0)
    cache.set_seq_tokens(torch.tensor(Ts0, dtype=torch.int32, device=gpu))
    # the next n tokens of every sequence, appended in two calls
    for a, c in ((0, n - 1), (n - 1, n)):
        kn = np.stack([full_k[b, Ts0[b] + a: Ts0[b] + c] for b in range(3)])
        vn = np.stack([full_v[b, Ts0[b] + a: Ts0[b] + c] for b in range(3)])
        cache.append(torch.from_numpy(kn).to(gpu), torch.from_numpy(vn).to(gpu))
    torch.cuda.synchronize()
    Ts = [t + n for t in Ts0]
    assert cache.seq_tokens.cpu().tolist() == Ts and cache.n_tokens == max(Ts)
    for name, x, spec in (("k", full_k, ok_), ("v", full_v, ov)):
        dev = H.download(cache, name)
        enc = [[OL.encode_head(x[b, :Ts[b], h, :], spec, h) for h in range(2)] for b in range(3)]
        packed = OL.pack_plane(enc, spec, cap)
        ring = np.concatenate([OL.tail_ring(x[b:b + 1, :Ts[b]], 64) for b in range(3)])
        per = cap * OL.head_row_bytes(spec, 0)
        for b in range(3):
            for h in range(2):
                i = b * 2 + h
                R = OL.head_row_bytes(spec, h)
                got = OL.untile_plane(dev["codes"][i * per:(i + 1) * per], R)[:Ts[b]]
                exp = OL.untile_plane(packed["codes"][i * per:(i + 1) * per], R)[:Ts[b]]
                assert np.array_equal(got, exp), (name, b, h)
        nb = OL.head_nblk(spec, 0)
        for b in range(3):
            for h in range(2):
                i = b * 2 + h
                sl = slice(i * cap * nb, i * cap * nb + Ts[b] * nb)
                assert np.array_equal(dev["scales"][sl], packed["scales"][sl]), (name, b, h)
        assert np.array_equal(dev["tail"], OL.pack_tail(ring)), name
        back = cache.dequantize(name).cpu().numpy()
        for b in range(3):
            assert not np.any(back[b, Ts[b]:]), "rows past a sequence's count are zero"
    q = synth.queries(wl, 0)
    ref = _oracle_out(q.numpy(), full_k, full_v, ok_, ov, Ts, 64, wl.sm_scale)
    out = cache.decode(q.to(gpu), wl.sm_scale).cpu().numpy()
    assert float(np.max(np.abs(out.astype(np.float64) - ref))) <= H.ATOL
