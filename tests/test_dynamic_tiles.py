"""GPU parity of decode splits long enough that waves claim their tiles at
run time (at least 4 tiles per wave): one body split over a few thousand
tokens, so each wave's share depends on when its data arrive; the output
must still match the oracle's decode within the decode tolerance, for a
plain q8_0/q4_0 body with a binary16 tail, a KVarN q3_0 body (six query
heads per kv head) and a low-rank body, and repeated launches must agree to
well below that tolerance."""

import numpy as np
import pytest

import oracle.layer as OL
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T,N,Hq", [("gqa4_q8k_q4v_tail1024", 2600, 128, 8),
                                         ("kvarn_q3_tail2048", 2300, 64, 12),
                                         ("lowrank_1bpd", 2200, 0, None)])
def test_long_split_matches_oracle(gpu, name, T, N, Hq):
    wl = synth.WORKLOADS[name].with_(B=1, T=T, N=N)
    if Hq:
        wl = wl.with_(Hkv=2, Hq=Hq)
    k = synth.layer_rows(wl, 0, "k").numpy()
    v = synth.layer_rows(wl, 0, "v").numpy()
    q = synth.queries(wl, 0)
    gk, gv, ok_, ov = H.specs(wl)
    cap = (T + 63) // 64 * 64
    cache = H.new_cache(wl, cap, gk, gv, gpu, N=N)
    for nm, x, spec in (("k", k, ok_), ("v", v, ov)):
        tail = OL.pack_tail(OL.tail_ring(x, N)) if N else None
        H.upload(cache, nm, OL.pack_plane(OL.encode_plane(x, spec), spec, cap), tail)
    cache.n_tokens = T
    ref = OL.decode(q.numpy(), OL.encode_plane(k, ok_), OL.encode_plane(v, ov),
                    OL.tail_ring(k, N) if N else None, OL.tail_ring(v, N) if N else None,
                    ok_, ov, T, N, wl.sm_scale)
    body_tiles = (T - N + 63) // 64
    assert body_tiles >= 4 * 8, "the split must give every wave at least 4 tiles"
    outs = []
    for _ in range(3):
        out = cache.decode(q.to(gpu), wl.sm_scale, body_splits=1).cpu().numpy().astype(np.float64)
        outs.append(out)
        err = float(np.max(np.abs(out - ref)))
        assert err <= H.ATOL, (name, err)
    spread = max(float(np.max(np.abs(o - outs[0]))) for o in outs)
    assert spread <= 1e-5, spread
