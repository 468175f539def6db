"""VBR budget controller, written plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: the VBR announcement thread (opening posts).  The cache stays at 16
bits while it fits; as the session grows, layers move down a codec ladder
one at a time, in a per-layer order found by profiling, never below a floor
codec (--vbr-floor), so that the whole cache fits a VRAM budget
(--vbr-vram).  The reply on injected KV: any added KV can push a degrade.

Reading (the pages give no algorithm): one degrade step moves one layer one
rung down the ladder; the next layer to move is the one at the highest rung
still above the floor, ties broken by the degrade order; layers never move
back up.  Bytes of the cache: every layer's K and V rows (codes plus binary16
scales, plus mins for _1 codecs) for every token of every (batch, kv head),
plus the binary16 tail of each plane.
"""

from .budget import row_total_bytes


def cache_bytes(ladder, level, n_tokens, batch, n_kv_heads, tail_len):
    total = 0
    for lv in level:
        codec = ladder[lv]
        total += 2 * batch * n_kv_heads * n_tokens * row_total_bytes(codec)
        if tail_len > 0:
            total += 2 * batch * n_kv_heads * tail_len * 2 * 128
    return total


def plan(ladder, floor, order, level, n_tokens, batch, n_kv_heads, tail_len, budget):
    """Returns (fits, new levels, steps) with steps = [(layer, from, to), ...]."""
    level = list(level)
    steps = []
    while cache_bytes(ladder, level, n_tokens, batch, n_kv_heads, tail_len) > budget:
        candidates = [l for l in order if level[l] < floor]
        if not candidates:
            return False, level, steps
        best = min(level[l] for l in candidates)
        layer = next(l for l in order if level[l] == best and level[l] < floor)
        steps.append((layer, ladder[level[layer]], ladder[level[layer] + 1]))
        level[layer] += 1
    return True, level, steps
