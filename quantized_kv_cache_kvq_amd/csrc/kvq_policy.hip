// VBR budget controller: which layers to move to which codec so the cache
// fits a byte budget as the session grows (host-only policy over the layer
// transcode kernel).
//
// The VBR announcement thread (opening posts) describes the behaviour: the
// cache stays at 16 bits while it fits, then layers move down a codec
// ladder one at a time in a profiled per-layer order ("F16 until 18k, then
// F16/T8 mixes, and so on"), never below a floor codec (--vbr-floor), within
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
