// VBR budget controller: which layers to move to which codec so the cache
// fits a byte budget as the session grows (host-only policy over the layer
// transcode kernel).
//
// The VBR announcement thread (opening posts) describes the behaviour: the
// cache stays at 16 bits while it fits, then layers move down a codec
// ladder one at a time in a profiled per-layer order (all layers at 16 bits
// up to a context size, then mixes of 16-bit and lower-bit layers), never
// below a floor codec (--vbr-floor), within
// a VRAM budget (--vbr-vram); any added KV, injected or generated, can push a
// degrade (the reply on injected KV).  Reading taken here: a degrade moves
// one layer one rung; the next layer to move is the one at the highest rung
// still above the floor, ties broken by the degrade order; a session never
// moves a layer back up (the raw values are gone).
#include <string.h>

#include "kvq_common.hpp"
#include "kvq_internal.hpp"

namespace {

bool ladder_codec_ok(int c) { return c >= KVQ_F16 && c <= KVQ_Q1_1; }

// Bytes of one token of one kv head in a codec: codes + scales (+ mins).
long long row_total(int codec) {
  using namespace kvq;
  if (codec_family(codec) == FAM_F16) return 2 * D;
  const long long side = (codec_family(codec) == FAM_0 ? 2 : 4) * (D / 32);
  return (long long)row_bytes(codec, D) + side;
}

}  // namespace

extern "C" {

long long kvq_vbr_bytes(const kvq_vbr_policy *pol, const int32_t *level, int32_t n_tokens) {
  if (!pol || !level || n_tokens < 0) return -1;
  const long long per_tok_heads = (long long)pol->batch * pol->n_kv_heads;
  long long total = 0;
  for (int l = 0; l < pol->n_layers; ++l) {
    const int lv = level[l];
    if (lv < 0 || lv >= pol->ladder_len) return -1;
    const int c = pol->ladder[lv];
    total += 2 * per_tok_heads * n_tokens * row_total(c);                  // K and V
    if (pol->tail_len > 0) total += 2 * per_tok_heads * pol->tail_len * (2LL * 128);
  }
  return total;
}

kvq_status kvq_vbr_plan(const kvq_vbr_policy *pol, int32_t n_tokens, int32_t *level,
                        int32_t *steps, int32_t max_steps, int32_t *n_steps) {
  if (n_steps) *n_steps = 0;
  if (!pol || !level || !pol->ladder || !pol->order || (max_steps > 0 && !steps))
    return kvq::api_fail(KVQ_ERR_INVALID_ARG, "vbr plan: NULL policy, level, ladder, order or steps");
  if (pol->n_layers < 1 || pol->ladder_len < 1 || pol->floor < 0 ||
      pol->floor >= pol->ladder_len || pol->batch < 1 || pol->n_kv_heads < 1 ||
      pol->tail_len < 0 || n_tokens < 0 || pol->budget_bytes < 0)
    return kvq::api_fail(KVQ_ERR_INVALID_ARG, "vbr plan: bad shape, floor, budget or token count");
  for (int i = 0; i < pol->ladder_len; ++i)
    if (!ladder_codec_ok(pol->ladder[i])) return kvq::api_fail(KVQ_ERR_INVALID_ARG, "vbr plan: ladder entry is not a kvq_codec");
  // order must be a permutation of the layers
  unsigned char seen[4096];
  if (pol->n_layers > 4096) return kvq::api_fail(KVQ_ERR_INVALID_ARG, "vbr plan: more than 4096 layers");
  memset(seen, 0, sizeof seen);
  for (int i = 0; i < pol->n_layers; ++i) {
    const int l = pol->order[i];
    if (l < 0 || l >= pol->n_layers || seen[l])
      return kvq::api_fail(KVQ_ERR_INVALID_ARG, "vbr plan: order is not a permutation of the layers");
    seen[l] = 1;
    if (level[l] < 0 || level[l] >= pol->ladder_len)
      return kvq::api_fail(KVQ_ERR_INVALID_ARG, "vbr plan: level outside the ladder");
  }
  int done = 0;
  for (;;) {
    if (kvq_vbr_bytes(pol, level, n_tokens) <= pol->budget_bytes) {
      if (n_steps) *n_steps = done;
      return kvq::api_ok();
    }
    // highest rung (smallest level) above the floor, first in degrade order
    int pick = -1;
    for (int i = 0; i < pol->n_layers; ++i) {
      const int l = pol->order[i];
      if (level[l] < pol->floor && (pick < 0 || level[l] < level[pick])) pick = l;
    }
    if (pick < 0) {
      if (n_steps) *n_steps = done;
      return kvq::api_fail(KVQ_ERR_CAPACITY, "vbr plan: budget exceeded with every layer at the floor");
    }
    if (done >= max_steps) {
      if (n_steps) *n_steps = done;
      return kvq::api_fail(KVQ_ERR_WORKSPACE, "vbr plan: steps array too short");
    }
    steps[3 * done] = pick;
    steps[3 * done + 1] = pol->ladder[level[pick]];
    steps[3 * done + 2] = pol->ladder[level[pick] + 1];
    ++level[pick];
    ++done;
  }
}

}  // extern "C"

// ------------------------------------------------ KV-COBRA allocation ------
//
// KV-COBRA explainer: a head keeps its top r directions (their dropped
// variance is lost outright) and stores the kept coordinates with b bits,
// whose rounding noise falls about 4x per extra bit; C1 chooses (r, b) in a
// head, C2 moves budget between heads until each sits at the same marginal
// error (water-filling: a bit goes where it removes the most error), and
// the paper's C2 settles within five rounds.  Error model (the reading the
// tests pin with the explainer's worked example): with the kept directions
// flattened by the fused Hadamard rotation, a b-bit uniform quantiser over a
// 4-sigma range adds gamma / (2^b - 1)^2 of the kept variance, gamma = 4/3.
//
// C1: every head's candidate pairs, reduced to the lower convex hull of
// (bits, error).  C2: start every head at its cheapest hull point, then give
// hull steps to the head with the largest error drop per bit while the
// budget lasts; then rounds of exchanges over all candidate pairs (a donor
// head moves down, the freed bits and any slack let another head move up)
// until no exchange lowers the total error.
#include <algorithm>
#include <cmath>
#include <vector>

namespace {

struct CobraOpt {
  long long cost;
  double err;
  int r, b;
};

// total order: cost, then error, then rank, then bits
bool cobra_less(const CobraOpt &x, const CobraOpt &y) {
  if (x.cost != y.cost) return x.cost < y.cost;
  if (x.err != y.err) return x.err < y.err;
  if (x.r != y.r) return x.r < y.r;
  return x.b < y.b;
}

}  // namespace

extern "C" kvq_status kvq_cobra_allocate(const double *spectra, int32_t n_heads, const int32_t *ranks,
                                         int32_t n_ranks, const int32_t *bits, int32_t n_bits,
                                         long long budget_bits, double gamma, int32_t *out_rank,
                                         int32_t *out_bits, int32_t *rounds, double *total_error) {
  if (!spectra || !ranks || !bits || !out_rank || !out_bits || n_heads < 1 || n_ranks < 1 ||
      n_bits < 1 || budget_bits < 0 || !(gamma > 0.0))
    return kvq::api_fail(KVQ_ERR_INVALID_ARG, "cobra allocate: bad arguments");
  for (int i = 0; i < n_ranks; ++i)
    if (ranks[i] < 1 || ranks[i] > 128)
      return kvq::api_fail(KVQ_ERR_INVALID_ARG, "cobra allocate: ranks must be in [1, 128]");
  for (int i = 0; i < n_bits; ++i)
    if (bits[i] < 1 || bits[i] > 16)
      return kvq::api_fail(KVQ_ERR_INVALID_ARG, "cobra allocate: bits must be in [1, 16]");
  const int H = n_heads;
  std::vector<std::vector<CobraOpt>> opt(H), hull(H), front(H);
  for (int h = 0; h < H; ++h) {
    const double *lam = spectra + (long long)h * 128;
    double pre[129];
    pre[0] = 0.0;
    for (int j = 0; j < 128; ++j) {
      if (!(lam[j] >= 0.0))
        return kvq::api_fail(KVQ_ERR_INVALID_ARG, "cobra allocate: spectra must be non-negative");
      pre[j + 1] = pre[j] + lam[j];
    }
    for (int i = 0; i < n_ranks; ++i)
      for (int k = 0; k < n_bits; ++k) {
        const int r = ranks[i], b = bits[k];
        const double q = std::ldexp(1.0, b) - 1.0;
        opt[h].push_back({(long long)r * b, (pre[128] - pre[r]) + gamma / (q * q) * pre[r], r, b});
      }
    std::vector<CobraOpt> o = opt[h];
    std::sort(o.begin(), o.end(), cobra_less);
    // efficient frontier, then lower convex hull
    std::vector<CobraOpt> f;
    for (const auto &x : o)
      if (f.empty() || x.err < f.back().err) {
        if (!f.empty() && f.back().cost == x.cost) f.back() = x;
        else f.push_back(x);
      }
    front[h] = f;
    for (const auto &x : f) {
      while (hull[h].size() >= 2) {
        const CobraOpt &a = hull[h][hull[h].size() - 2], &c = hull[h].back();
        // drop c if it lies on or above the segment a -> x
        if ((c.err - a.err) * (x.cost - a.cost) >= (x.err - a.err) * (c.cost - a.cost)) hull[h].pop_back();
        else break;
      }
      hull[h].push_back(x);
    }
  }
  // C2 greedy on the hulls
  std::vector<int> pos(H, 0);
  long long used = 0;
  for (int h = 0; h < H; ++h) used += hull[h][0].cost;
  if (used > budget_bits)
    return kvq::api_fail(KVQ_ERR_CAPACITY, "cobra allocate: budget below every head's cheapest pair");
  for (;;) {
    int best = -1;
    double gain = 0.0;
    for (int h = 0; h < H; ++h) {
      if (pos[h] + 1 >= (int)hull[h].size()) continue;
      const CobraOpt &a = hull[h][pos[h]], &c = hull[h][pos[h] + 1];
      if (used + c.cost - a.cost > budget_bits) continue;
      const double g = (a.err - c.err) / (double)(c.cost - a.cost);
      if (g > gain) { gain = g; best = h; }
    }
    if (best < 0) break;
    used += hull[best][pos[best] + 1].cost - hull[best][pos[best]].cost;
    ++pos[best];
  }
  std::vector<CobraOpt> cur(H);
  for (int h = 0; h < H; ++h) cur[h] = hull[h][pos[h]];
  // exchange rounds over the full candidate sets: per head, candidates by
  // cost with the best error at or below each cost (a receiver's best
  // move for given room is one binary search)
  std::vector<std::vector<CobraOpt>> by_cost(H), pref(H);
  for (int h = 0; h < H; ++h) {
    by_cost[h] = opt[h];
    std::sort(by_cost[h].begin(), by_cost[h].end(), cobra_less);
    pref[h] = by_cost[h];
    for (size_t k = 1; k < pref[h].size(); ++k)
      if (pref[h][k - 1].err <= pref[h][k].err) pref[h][k] = pref[h][k - 1];
  }
  auto best_within = [&](int h, long long max_cost, CobraOpt &out) {
    const auto &v = by_cost[h];
    size_t lo = 0, hi = v.size();             // first index with cost > max_cost
    while (lo < hi) {
      const size_t mid = (lo + hi) / 2;
      if (v[mid].cost <= max_cost) lo = mid + 1; else hi = mid;
    }
    if (lo == 0) return false;
    out = pref[h][lo - 1];
    return true;
  };
  // Receivers' gains by extra bits: gtab[j][x] = the error head j sheds
  // with x more bits (its best candidate within cur[j].cost + x); b1/b2: the
  // two heads with the largest gain at each x.  A donor's move then finds
  // its best receiver in one lookup.
  long long maxc = 0;
  for (int h = 0; h < H; ++h) maxc = std::max(maxc, by_cost[h].back().cost);
  const size_t W = (size_t)maxc + 1;
  std::vector<double> gtab((size_t)H * W);
  std::vector<int> b1(W), b2(W);
  auto fill_row = [&](int j) {
    const auto &v = by_cost[j];
    size_t k = 0;
    double best = cur[j].err;
    for (size_t x = 0; x < W; ++x) {
      const long long lim = cur[j].cost + (long long)x;
      while (k < v.size() && v[k].cost <= lim) best = std::min(best, v[k++].err);
      gtab[(size_t)j * W + x] = cur[j].err - best;
    }
  };
  auto fill_top = [&]() {
    for (size_t x = 0; x < W; ++x) {
      int f = -1, s2 = -1;
      for (int j = 0; j < H; ++j) {
        const double g = gtab[(size_t)j * W + x];
        if (f < 0 || g > gtab[(size_t)f * W + x]) { s2 = f; f = j; }
        else if (s2 < 0 || g > gtab[(size_t)s2 * W + x]) s2 = j;
      }
      b1[x] = f;
      b2[x] = s2;
    }
  };
  for (int j = 0; j < H; ++j) fill_row(j);
  fill_top();
  int nround = 0;
  for (int it = 0; it < 64; ++it) {
    bool changed = false;
    for (int i = 0; i < H; ++i) {
      double best_delta = -1e-15;
      int bj = -1;
      long long broom = 0;
      CobraOpt bi_opt{};
      const long long slack = budget_bits - used;
      for (const auto &di : opt[i]) {
        if (di.cost > cur[i].cost + slack) continue;
        const long long room = std::min(slack + cur[i].cost - di.cost, maxc);   // bits others may take
        const double d_i = di.err - cur[i].err;
        if (d_i < best_delta) { best_delta = d_i; bj = i; bi_opt = di; }
        const int j = b1[room] != i ? b1[room] : b2[room];
        if (j < 0) continue;
        const double d = d_i - gtab[(size_t)j * W + room];
        if (d < best_delta) { best_delta = d; bj = j; bi_opt = di; broom = room; }
      }
      if (bj >= 0) {
        CobraOpt bj_opt = bi_opt;
        if (bj != i && !best_within(bj, cur[bj].cost + broom, bj_opt)) continue;
        used += bi_opt.cost - cur[i].cost;
        cur[i] = bi_opt;
        fill_row(i);
        if (bj != i) {
          used += bj_opt.cost - cur[bj].cost;
          cur[bj] = bj_opt;
          fill_row(bj);
        }
        fill_top();
        changed = true;
      }
    }
    // Several donors for one receiver: a head moving up to a better
    // candidate of its efficient frontier that does not fit is funded by
    // downgrading other heads, the
    // cheapest downgrade first (least error added per bit freed; a donor
    // may step down more than once), when it gains more than they lose.
    // Pairwise exchanges alone miss these.
    {
      struct Step {
        double rate;
        int h;
        CobraOpt d;
      };
      auto worse = [](const Step &x, const Step &y) { return x.rate > y.rate; };   // min-heap
      // each head's cheapest single downgrade from a candidate
      auto step_from = [&](int i, const CobraOpt &from, Step &st) {
        CobraOpt d;
        if (from.cost == 0 || !best_within(i, from.cost - 1, d)) return false;
        st = {(d.err - from.err) / (double)(from.cost - d.cost), i, d};
        return true;
      };
      std::vector<Step> base;
      auto rebuild = [&]() {
        base.clear();
        for (int i = 0; i < H; ++i) {
          Step st;
          if (step_from(i, cur[i], st)) base.push_back(st);
        }
      };
      rebuild();
      std::vector<CobraOpt> tent(H);
      std::vector<char> touched(H);
      std::vector<Step> heap;
      for (int j = 0; j < H && !base.empty(); ++j) {
        bool moved = false;
        double mrate = -1.0;                     // cheapest downgrade per bit of the other heads
        for (const auto &st : base)
          if (st.h != j && (mrate < 0.0 || st.rate < mrate)) mrate = st.rate;
        if (mrate < 0.0) continue;
        for (const auto &upv : front[j]) {
          if (upv.cost <= cur[j].cost || !(upv.err < cur[j].err)) continue;
          long long need = upv.cost - cur[j].cost - (budget_bits - used);
          if (need <= 0) continue;               // fits: the pairwise pass takes such moves
          const double gain = cur[j].err - upv.err;
          if (gain <= mrate * (double)need) continue;
          double loss = 0.0;
          heap.clear();
          for (const auto &st : base)
            if (st.h != j) heap.push_back(st);
          std::make_heap(heap.begin(), heap.end(), worse);
          for (int i = 0; i < H; ++i) { tent[i] = cur[i]; touched[i] = 0; }
          while (need > 0 && loss < gain && !heap.empty()) {
            std::pop_heap(heap.begin(), heap.end(), worse);
            const Step st = heap.back();
            heap.pop_back();
            loss += st.d.err - tent[st.h].err;
            need -= tent[st.h].cost - st.d.cost;
            tent[st.h] = st.d;
            touched[st.h] = 1;
            Step nx;
            if (step_from(st.h, tent[st.h], nx)) {
              heap.push_back(nx);
              std::push_heap(heap.begin(), heap.end(), worse);
            }
          }
          if (need > 0 || !(loss < gain * (1.0 - 1e-12))) continue;
          for (int i = 0; i < H; ++i)
            if (touched[i]) {
              used += tent[i].cost - cur[i].cost;
              cur[i] = tent[i];
            }
          used += upv.cost - cur[j].cost;
          cur[j] = upv;
          changed = moved = true;
          break;
        }
        if (moved) {
          rebuild();
          for (int h = 0; h < H; ++h) fill_row(h);
          fill_top();
        }
      }
    }
    if (!changed) break;
    ++nround;
  }
  double tot = 0.0;
  for (int h = 0; h < H; ++h) {
    out_rank[h] = cur[h].r;
    out_bits[h] = cur[h].b;
    tot += cur[h].err;
  }
  if (rounds) *rounds = nround;
  if (total_error) *total_error = tot;
  return kvq::api_ok();
}
