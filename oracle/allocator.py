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
solves it exactly by dynamic programming over the budget; the library's C1/C2
iteration is checked against that optimum.
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


def _errors(lam, ranks, bits, gamma):
    """Candidate list in the library's construction order (rank-major),
    errors summed the same way (running prefix sums)."""
    pre = [0.0]
    for x in np.asarray(lam, np.float64):
        pre.append(pre[-1] + float(x))
    out = []
    for r in ranks:
        for b in bits:
            q = 2.0 ** b - 1.0
            out.append((r * b, (pre[128] - pre[r]) + gamma / (q * q) * pre[r], r, b))
    return out


def _hull(opts):
    """Lower convex hull of (cost, error) over the efficient candidates."""
    o = sorted(opts)
    front = []
    for x in o:
        if not front or x[1] < front[-1][1]:
            if front and front[-1][0] == x[0]:
                front[-1] = x
            else:
                front.append(x)
    hull = []
    for x in front:
        while len(hull) >= 2:
            a, c = hull[-2], hull[-1]
            if (c[1] - a[1]) * (x[0] - a[0]) >= (x[1] - a[1]) * (c[0] - a[0]):
                hull.pop()
            else:
                break
        hull.append(x)
    return hull


def water_fill(spectra, ranks, bits, budget, gamma=GAMMA, max_rounds=64):
    """The C1 / C2 steps as described: C1 reduces each head to its efficient
    (bits, error) pairs; C2 gives bits, step by step, to the head whose next
    step removes the most error per bit, then exchanges bits between heads
    (one head moves down, another takes the freed bits) in rounds until no
    exchange lowers the total error.  Returns (allocation, rounds, total
    error, fits)."""
    H = len(spectra)
    opts = [_errors(l, ranks, bits, gamma) for l in spectra]
    hulls = [_hull(o) for o in opts]
    pos = [0] * H
    used = sum(h[0][0] for h in hulls)
    if used > budget:
        return None, 0, None, False
    while True:
        best, gain = -1, 0.0
        for h in range(H):
            if pos[h] + 1 >= len(hulls[h]):
                continue
            a, c = hulls[h][pos[h]], hulls[h][pos[h] + 1]
            if used + c[0] - a[0] > budget:
                continue
            g = (a[1] - c[1]) / float(c[0] - a[0])
            if g > gain:
                gain, best = g, h
        if best < 0:
            break
        used += hulls[best][pos[best] + 1][0] - hulls[best][pos[best]][0]
        pos[best] += 1
    cur = [hulls[h][pos[h]] for h in range(H)]
    # best candidate of each head at or below every cost (first of the
    # cost-sorted list achieving the smallest error so far)
    maxc = max(o[0] for ho in opts for o in ho)
    table = []
    for ho in opts:
        s = sorted(ho)
        row, k, best_o = [None] * (maxc + 1), 0, None
        for c in range(maxc + 1):
            while k < len(s) and s[k][0] <= c:
                if best_o is None or not (best_o[1] <= s[k][1]):
                    best_o = s[k]
                k += 1
            row[c] = best_o
        table.append(row)
    rounds = 0
    for _ in range(max_rounds):
        changed = False
        for i in range(H):
            best_delta, bj, bi_o, bj_o = -1e-15, -1, None, None
            slack = budget - used
            for di in opts[i]:
                if di[0] > cur[i][0] + slack:
                    continue
                room = slack + cur[i][0] - di[0]
                d_i = di[1] - cur[i][1]
                if d_i < best_delta:
                    best_delta, bj, bi_o, bj_o = d_i, i, di, di
                for j in range(H):
                    if j == i:
                        continue
                    uj = table[j][min(cur[j][0] + room, maxc)]
                    if uj is None:
                        continue
                    d = d_i + (uj[1] - cur[j][1])
                    if d < best_delta:
                        best_delta, bj, bi_o, bj_o = d, j, di, uj
            if bj >= 0:
                used += bi_o[0] - cur[i][0]
                cur[i] = bi_o
                if bj != i:
                    used += bj_o[0] - cur[bj][0]
                    cur[bj] = bj_o
                changed = True
        if not changed:
            break
        rounds += 1
    total = 0.0
    for x in cur:
        total += x[1]
    return [(x[2], x[3]) for x in cur], rounds, total, True
