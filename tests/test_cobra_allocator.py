"""KV-COBRA per-head rank/bit allocation (host calibration step in libkvq)
against the oracle: the exact optimum (dynamic programming over the
budget, pinned by brute force), the continuous relaxation (weak duality)
and the rounding gap a greedy fill can leave; the oracle's plain C1/C2
reading of the explainer; and the explainer's statements: the two-head
worked example's split, C2 settling within five rounds, and the
calibration taking under 200 ms for a 256-head model (LLaMA-3.1-8B has
8 kv heads x 32 layers)."""

import itertools
import random
import time

import numpy as np
import pytest

from oracle import allocator as A
from quantized_kv_cache_kvq_amd import lib

RANKS = list(range(16, 129, 16))
BITS = list(range(1, 9))


@pytest.fixture(scope="module")
def L():
    return lib.load()


def _spectrum(rng, kind):
    j = np.arange(1, 129, dtype=np.float64)
    if kind == 0:
        lam = j ** -rng.choice([0.25, 0.5, 1.0, 2.0, 3.0])
    elif kind == 1:
        k = rng.integers(4, 64)
        lam = np.concatenate([np.full(k, 1.0), np.full(128 - k, rng.uniform(1e-4, 1e-2))])
    else:
        lam = np.sort(rng.exponential(1.0, 128))[::-1]
    return lam * rng.lognormal(0.0, 1.0)


def test_worked_example(L):
    """Two heads at 1 bpd (256 bits): head A keeps 99% of its variance in 16
    directions, head B is flat.  The explainer's per-head split: A at rank
    16 x 4 bits, B at rank 96 x 2 bits."""
    lamA = np.concatenate([np.full(16, 0.99 / 16), np.full(112, 0.01 / 112)])
    lamB = np.full(128, 1.0 / 128)
    tot, alloc = A.optimum([lamA, lamB], RANKS, BITS, 256)
    assert alloc == [(16, 4), (96, 2)]
    got, rounds, lt = lib.cobra_allocate(np.stack([lamA, lamB]), RANKS, BITS, 256)
    assert got == [(16, 4), (96, 2)] and rounds <= 5 and abs(lt - tot) < 1e-12
    # the uniform setting it improves on: rank 32 x 4 bits for both
    uni = A.head_error(lamA, 32, 4) + A.head_error(lamB, 32, 4)
    assert tot < uni
    # B's lost variance: 75% at rank 32, 25% at rank 96
    assert abs(lamB[32:].sum() - 0.75) < 1e-12 and abs(lamB[96:].sum() - 0.25) < 1e-12


def test_oracle_optimum_is_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(30):
        H = int(rng.integers(1, 4))
        ranks = sorted(rng.choice(RANKS, size=3, replace=False).tolist())
        bits = sorted(rng.choice(BITS, size=3, replace=False).tolist())
        sp = [_spectrum(rng, int(rng.integers(0, 3))) for _ in range(H)]
        budget = int(rng.integers(min(ranks) * min(bits) * H, max(ranks) * max(bits) * H + 1))
        best = None
        for combo in itertools.product(itertools.product(ranks, bits), repeat=H):
            if sum(r * b for r, b in combo) <= budget:
                e = sum(A.head_error(l, r, b) for l, (r, b) in zip(sp, combo))
                best = e if best is None else min(best, e)
        tot, alloc = A.optimum(sp, ranks, bits, budget)
        assert sum(r * b for r, b in alloc) <= budget
        assert abs(tot - best) <= 1e-12 * max(1.0, best)
        # C1 alone: the best pair of one head at a budget is brute force too
        lam, B = sp[0], budget
        c1 = A.best_in_head(lam, ranks, bits, B)
        bf = min(((A.head_error(lam, r, b), r * b) for r in ranks for b in bits if r * b <= B), default=None)
        assert (c1 is None and bf is None) or abs(c1[1] - bf[0]) < 1e-15


def test_oracle_c1_and_plain_c2():
    """C1 (each head's best error at every budget) against brute force over
    the candidates; the plain C1/C2 reading of the explainer never beats
    the exact optimum and respects the budget; the relaxation bound sits
    below the optimum (weak duality)."""
    rng = np.random.default_rng(4)
    for _ in range(20):
        H = int(rng.integers(1, 6))
        sp = [_spectrum(rng, int(rng.integers(0, 3))) for _ in range(H)]
        budget = int(rng.integers(16 * H, 128 * 8 * H + 1))
        errs, pick = A.c1_curve(sp[0], RANKS, BITS, 1024)
        for c in range(0, 1025, 37):
            bf = [A.head_error(sp[0], r, b) for r in RANKS for b in BITS if r * b <= c]
            assert (not bf and pick[c] is None) or errs[c] == min(bf)
        tot, _ = A.optimum(sp, RANKS, BITS, budget)
        alloc, wt, _ = A.water_fill_plain(sp, RANKS, BITS, budget)
        assert sum(r * b for r, b in alloc) <= budget and wt >= tot - 1e-12 * tot
        lb, mu = A.lagrangian_bound(sp, RANKS, BITS, budget)
        assert lb <= tot * (1 + 1e-12) + 1e-15 and mu >= 0.0
        assert wt <= lb + A.rounding_gap(sp, RANKS, BITS, mu) + 1e-9 * tot


def _check_against_optimum(sp, budget):
    """The library's allocation against the oracle: within the budget, never
    below the exact optimum, and within the relaxation's rounding gap of
    the relaxation's optimum (what a greedy that fills heads by error
    removed per bit is guaranteed to reach; exchange rounds only lower it)."""
    alloc, rounds, lt = lib.cobra_allocate(np.stack(sp), RANKS, BITS, budget)
    assert sum(r * b for r, b in alloc) <= budget
    assert abs(lt - sum(A.head_error(l, r, b) for l, (r, b) in zip(sp, alloc))) <= 1e-12 * max(1.0, lt)
    tot, _ = A.optimum(sp, RANKS, BITS, budget)
    lb, mu = A.lagrangian_bound(sp, RANKS, BITS, budget)
    assert lt >= tot - 1e-12 * max(1.0, tot)
    assert lt <= lb + A.rounding_gap(sp, RANKS, BITS, mu) + 1e-9 * max(1.0, tot)
    return (lt / tot - 1.0 if tot > 0 else 0.0), rounds, alloc


def test_library_against_exact_optimum(L):
    """1-8 heads, coarse candidates (8 ranks x 8 bit widths), budgets from
    the cheapest to the richest: every case passes the relaxation bound and
    settles within five exchange rounds; as a regression guard on these
    seeded cases, at least 90% reach the exact optimum and none is more
    than 12% above it (measured: 95% exact, worst 11.0%, 99th percentile
    3%)."""
    rng = np.random.default_rng(11)
    gaps = []
    for _ in range(280):
        H = int(rng.integers(1, 9))
        sp = [_spectrum(rng, int(rng.integers(0, 3))) for _ in range(H)]
        budget = int(rng.integers(16 * H, 128 * 8 * H + 1))
        gap, rounds, _ = _check_against_optimum(sp, budget)
        assert rounds <= 5
        gaps.append(gap)
    gaps = np.array(gaps)
    print("exact in %d of %d, worst gap %.4g" % ((gaps <= 1e-12).sum(), len(gaps), gaps.max()))
    assert (gaps <= 1e-12).mean() >= 0.90 and gaps.max() <= 0.12


@pytest.mark.parametrize("bpd", [0.5, 1, 2, 4])
def test_256_heads_rounds_and_time(L, bpd):
    """A 256-head model (8 kv heads x 32 layers): under 200 ms and at most
    five C2 rounds (the explainer's figures), within 0.1% of the exact
    optimum."""
    rng = np.random.default_rng(5)
    H = 256
    sp = [_spectrum(rng, int(rng.integers(0, 3))) for _ in range(H)]
    budget = int(bpd * 128 * H)
    t = time.perf_counter()
    alloc, rounds, lt = lib.cobra_allocate(np.stack(sp), RANKS, BITS, budget)
    dt = time.perf_counter() - t
    assert rounds <= 5 and dt < 0.2, (rounds, dt)
    gap, _, _ = _check_against_optimum(sp, budget)
    assert gap <= 1e-3
    # heads differ: the allocation spreads across ranks and bit widths
    assert len({r for r, _ in alloc}) > 1 and len({b for _, b in alloc}) > 1


def test_invalid_and_infeasible(L):
    sp = np.ones((2, 128))
    with pytest.raises(lib.KvqError):
        lib.cobra_allocate(sp, RANKS, BITS, 16)           # below 2 x 16 x 1 bits
    with pytest.raises(lib.KvqError):
        lib.cobra_allocate(-sp, RANKS, BITS, 1024)        # negative variances


@pytest.mark.gpu
def test_allocation_drives_lowrank_decode(gpu):
    """Calibrate spectra from the low-rank workload's own keys, allocate at
    1 bpd over the ranks and bit widths the decode kernel supports, and run
    the resulting per-head table through append + decode against the
    oracle."""
    import torch
    import oracle.cobra
    import oracle.layer as OL
    import synth
    from quantized_kv_cache_kvq_amd import calib
    from quantized_kv_cache_kvq_amd.cache import PlaneSpec
    from tests import helpers as H

    wl = synth.WORKLOADS["lowrank_1bpd"].with_(B=1, T=700)
    kcal = synth.layer_rows(wl.with_(T=4096), 0, "k")[0]          # [T, Hkv, 128]
    sp = calib.head_spectra(kcal).numpy()
    alloc, rounds, _ = lib.cobra_allocate(sp, [16, 32, 64, 128], [1, 2, 3, 4], 128 * wl.Hkv)
    assert rounds <= 5 and sum(r * b for r, b in alloc) <= 128 * wl.Hkv
    wl = wl.with_(lowrank=tuple(alloc))
    gk, gv, ok_, ov = H.specs(wl)
    cache = H.new_cache(wl, 768, gk, gv, gpu)
    k = synth.layer_rows(wl, 0, "k")
    v = synth.layer_rows(wl, 0, "v")
    cache.append(k.to(gpu), v.to(gpu))
    q = synth.queries(wl, 0)
    out = cache.decode(q.to(gpu), wl.sm_scale).cpu().numpy()
    kenc, _ = H.unpack(cache, "k", ok_, wl.T)
    venc, _ = H.unpack(cache, "v", ov, wl.T)
    for h in range(wl.Hkv):
        H.check_rotated_head(k.numpy()[0, :, h], kenc[0][h], ok_, h)
    ref = OL.decode(q.numpy(), kenc, venc, None, None, ok_, ov, wl.T, 0, wl.sm_scale)
    assert np.max(np.abs(out - ref)) <= H.ATOL
    print("allocation", alloc)
