"""Per-head rank / bit allocation (KV-COBRA), written plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: the KV-COBRA explainer.  A head keeps its top r directions (the rest
of their variance is lost) and stores each kept coordinate with b bits; the
rounding noise falls about 4x per extra bit (C1 description).  A head costs
r*b bits per token; the heads share a total budget (bits per dimension
times 128 times the number of heads, "Where the bits actually go").  C1
chooses (r, b) inside a head, C2 moves budget between heads until each sits
at the same marginal error.

Reading of the error model (the pages give the rule, not the constant): the
stored coordinates are flattened by the fused Hadamard rotation, so each
kept direction carries the mean kept variance and a b-bit uniform quantiser
over a 4-sigma range adds noise (range / (2^b - 1))^2 / 12 per coordinate:

    E_h(r, b) = sum_{j > r} lambda_hj + (4/3) / (2^b - 1)^2 * sum_{j <= r} lambda_hj

With this constant the explainer's two-head worked example (1 bpd, head A
holding 99% of its variance in 16 directions, head B flat) comes out at its
printed split, rank 16 x 4 bits and rank 96 x 2 bits (tests pin it).

The allocation problem is then plainly: minimise sum_h E_h(r_h, b_h) over
the candidate (r, b) pairs subject to sum_h r_h b_h <= budget.  The oracle
solves it exactly by dynamic programming over the budget (pinned by brute
force), bounds it from below by the continuous relaxation (weak duality),
and writes C1 / C2 out plainly from the explainer's words (each head's best
error at every budget; bits go where they remove the most error, then
moves between heads until none helps).  The library's allocation is checked
against the optimum and the relaxation, not against a copy of its loop.
"""

import numpy as np

GAMMA = 4.0 / 3.0


def head_error(lam, r, b, gamma=GAMMA):
    lam = np.asarray(lam, np.float64)
    return float(lam[r:].sum() + gamma / (2.0 ** b - 1.0) ** 2 * lam[:r].sum())


def options(lam, ranks, bits, gamma=GAMMA):
    """(cost r*b, error, r, b) for every candidate pair of one head."""
    return [(r * b, head_error(lam, r, b, gamma), r, b) for r in ranks for b in bits]


def best_in_head(lam, ranks, bits, budget, gamma=GAMMA):
    """C1 alone: the best (r, b) of one head within `budget` bits (None if
    no candidate fits)."""
    fit = [o for o in options(lam, ranks, bits, gamma) if o[0] <= budget]
    return min(fit, key=lambda o: (o[1], o[0])) if fit else None


def optimum(spectra, ranks, bits, budget, gamma=GAMMA):
    """Exact minimum of the total error: DP over heads and budget (in units
    of the gcd of the costs).  Returns (total error, [(r, b) per head])."""
    from math import gcd
    from functools import reduce

    opts = [options(lam, ranks, bits, gamma) for lam in spectra]
    unit = reduce(gcd, [o[0] for ho in opts for o in ho])
    nb = budget // unit
    INF = float("inf")
    best = np.full(nb + 1, INF)
    best[0] = 0.0
    choice = []
    for ho in opts:
        nxt = np.full(nb + 1, INF)
        arg = np.full(nb + 1, -1, dtype=np.int64)
        for k, (c, e, _, _) in enumerate(ho):
            cu = c // unit
            if cu > nb:
                continue
            cand = np.full(nb + 1, INF)
            cand[cu:] = best[: nb + 1 - cu] + e
            better = cand < nxt
            nxt[better] = cand[better]
            arg[better] = k
        choice.append(arg)
        best = nxt
    end = int(np.argmin(best))
    total = float(best[end])
    alloc = []
    for h in range(len(opts) - 1, -1, -1):
        k = int(choice[h][end])
        c, _, r, b = opts[h][k]
        alloc.append((r, b))
        end -= c // unit
    return total, alloc[::-1]


def c1_curve(lam, ranks, bits, max_cost, gamma=GAMMA):
    """C1 for one head, written as its definition: F(c) = the smallest error
    of any candidate (r, b) with r*b <= c, for c = 0 .. max_cost (inf where
    no candidate fits).  Returns (errors [max_cost+1], choice [(r, b) or
    None])."""
    errs = [float("inf")] * (max_cost + 1)
    pick = [None] * (max_cost + 1)
    for c in range(max_cost + 1):
        for r in ranks:
            for b in bits:
                if r * b <= c:
                    e = head_error(lam, r, b, gamma)
                    if e < errs[c]:
                        errs[c], pick[c] = e, (r, b)
    return errs, pick


def _candidates(spectra, ranks, bits, gamma):
    costs = np.array([r * b for r in ranks for b in bits], np.float64)
    errs = np.array([[head_error(l, r, b, gamma) for r in ranks for b in bits] for l in spectra])
    return costs, errs


def lagrangian_bound(spectra, ranks, bits, budget, gamma=GAMMA):
    """A lower bound on the optimum by weak duality: for any mu >= 0,
    g(mu) = sum_h min_(r,b) [E_h(r, b) + mu r b] - mu * budget <= the
    optimum.  g is concave and piecewise linear; its maximum sits at mu = 0
    or at a mu where some head's minimiser changes, mu = (E_a - E_b) /
    (c_b - c_a) for two candidates a, b of one head.  The sorted breakpoints
    are searched by ternary search (g at sorted points rises, then falls).
    Returns (max g, the maximising mu): the continuous relaxation's optimum
    and its multiplier."""
    costs, errs = _candidates(spectra, ranks, bits, gamma)
    mus = [np.zeros(1)]
    dc = costs[None, :] - costs[:, None]            # c_j - c_i
    for e in errs:
        de = e[:, None] - e[None, :]                # E_i - E_j
        ok = (dc > 0) & (de > 0)
        mus.append(de[ok] / dc[ok])
    mus = np.unique(np.concatenate(mus))

    def g(k):
        m = mus[k]
        return float((errs + m * costs[None, :]).min(axis=1).sum() - m * budget)

    lo, hi = 0, len(mus) - 1
    while hi - lo > 3:
        m1, m2 = lo + (hi - lo) // 3, hi - (hi - lo) // 3
        if g(m1) < g(m2):
            lo = m1 + 1
        else:
            hi = m2
    k = max(range(lo, hi + 1), key=g)
    return g(k), float(mus[k])


def rounding_gap(spectra, ranks, bits, mu, gamma=GAMMA):
    """How far rounding the relaxation can cost: at the multiplier mu, heads
    with several minimisers of E + mu * cost are the ones the relaxation may
    split between two candidates; the sum over them of (largest - smallest
    error among their minimisers).  A greedy that fills heads in order of
    error removed per bit, stopping when the next step does not fit, ends
    at most this far above the relaxation's optimum."""
    costs, errs = _candidates(spectra, ranks, bits, gamma)
    gap = 0.0
    for e in errs:
        val = e + mu * costs
        m = val.min()
        tie = np.abs(val - m) <= 1e-12 * max(1.0, abs(m)) + 1e-15
        if tie.sum() > 1:
            gap += float(e[tie].max() - e[tie].min())
    return gap


def water_fill_plain(spectra, ranks, bits, budget, gamma=GAMMA, max_rounds=50):
    """C1 / C2 as the explainer words them.  C1: each head's best error at
    every budget (c1_curve).  C2: start every head at its cheapest fitting
    budget, then, while bits remain, give the next bits to the head where
    they remove the most error per bit (any larger budget of that head that
    fits); then, in rounds, move bits from one head to another whenever
    that lowers the total, until a round changes nothing.  Returns
    (allocation [(r, b)], total error, rounds) or None when even the
    cheapest candidates exceed the budget."""
    H = len(spectra)
    maxc = max(r * b for r in ranks for b in bits)
    curves = [c1_curve(l, ranks, bits, maxc, gamma) for l in spectra]
    level = []
    for F, _ in curves:
        c = next(c for c in range(maxc + 1) if F[c] < float("inf"))
        level.append(c)
    if sum(level) > budget:
        return None
    spare = budget - sum(level)
    while True:
        pick = None
        for h, (F, _) in enumerate(curves):
            for c in range(level[h] + 1, min(maxc, level[h] + spare) + 1):
                gain = (F[level[h]] - F[c]) / (c - level[h])
                if gain > 0 and (pick is None or gain > pick[0]):
                    pick = (gain, h, c)
        if pick is None:
            break
        _, h, c = pick
        spare -= c - level[h]
        level[h] = c
    rounds = 0
    while rounds < max_rounds:
        moved = False
        for i in range(H):
            for j in range(H):
                if i == j:
                    continue
                Fi, Fj = curves[i][0], curves[j][0]
                best = None
                for ci in range(level[i] + 1):
                    if Fi[ci] == float("inf"):
                        continue
                    cj = min(maxc, level[j] + spare + (level[i] - ci))
                    d = (Fi[ci] - Fi[level[i]]) + (Fj[cj] - Fj[level[j]])
                    if d < -1e-12 * (Fi[level[i]] + Fj[level[j]]) and (best is None or d < best[0]):
                        best = (d, ci, cj)
                if best is not None:
                    _, ci, cj = best
                    spare += (level[i] - ci) - (cj - level[j])
                    level[i], level[j] = ci, cj
                    moved = True
        if not moved:
            break
        rounds += 1
    alloc = [curves[h][1][level[h]] for h in range(H)]
    total = sum(head_error(l, r, b, gamma) for l, (r, b) in zip(spectra, alloc))
    return alloc, total, rounds
