// C ABI of libkvq.so: argument checks, plans and dispatch to the kernels.
// Every check runs on the host before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kvq_common.hpp"
#include "kvq_internal.hpp"

using namespace kvq;

namespace {

thread_local char g_err[512] = "";

kvq_status fail(kvq_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

kvq_status ok() {
  g_err[0] = '\0';
  return KVQ_OK;
}

kvq_status hip_fail(hipError_t e, const char *what) {
  return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool codec_ok(int c) { return c >= 0 && c < KVQ_NUM_CODECS; }

// Checks one plane of a layer; `name` is "k" or "v".
kvq_status check_plane(const kvq_layer &L, const kvq_plane &p, const char *name) {
  if (p.basis < KVQ_BASIS_PLAIN || p.basis > KVQ_BASIS_LOWRANK)
    return fail(KVQ_ERR_INVALID_ARG, "%s.basis %d is not a kvq_basis", name, p.basis);
  if (p.codes == nullptr) return fail(KVQ_ERR_INVALID_ARG, "%s.codes is NULL", name);
  if (L.tail_len > 0 && p.tail == nullptr)
    return fail(KVQ_ERR_INVALID_ARG, "%s.tail is NULL with tail_len %d", name, L.tail_len);
  bool any_q = false, any_1 = false;
  if (p.basis == KVQ_BASIS_LOWRANK) {
    if (L.n_kv_heads > KVQ_MAX_LOWRANK_HEADS)
      return fail(KVQ_ERR_UNSUPPORTED, "low-rank planes support at most %d kv heads",
                  KVQ_MAX_LOWRANK_HEADS);
    if (!p.proj || !p.rank || !p.head_codec)
      return fail(KVQ_ERR_INVALID_ARG, "%s: low-rank plane needs proj, rank and head_codec", name);
    for (int h = 0; h < L.n_kv_heads; ++h) {
      const int r = p.rank[h], c = p.head_codec[h];
      if (!(r == 16 || r == 32 || r == 64 || r == 128))
        return fail(KVQ_ERR_INVALID_ARG, "%s.rank[%d] = %d (must be 16, 32, 64 or 128)", name, h, r);
      if (!codec_ok(c) || c == KVQ_F16)
        return fail(KVQ_ERR_INVALID_ARG, "%s.head_codec[%d] = %d is not a block codec", name, h, c);
      any_q = true;
      any_1 = any_1 || codec_family(c) == FAM_1;
    }
  } else {
    if (!codec_ok(p.codec))
      return fail(KVQ_ERR_INVALID_ARG, "%s.codec %d is not a kvq_codec", name, p.codec);
    any_q = p.codec != KVQ_F16;
    any_1 = codec_family(p.codec) == FAM_1;
    if (p.basis == KVQ_BASIS_HADAMARD && p.w == nullptr)
      return fail(KVQ_ERR_INVALID_ARG, "%s.w is NULL for the Hadamard basis", name);
  }
  if (any_q && p.scales == nullptr) return fail(KVQ_ERR_INVALID_ARG, "%s.scales is NULL", name);
  if (any_1 && p.mins == nullptr) return fail(KVQ_ERR_INVALID_ARG, "%s.mins is NULL", name);
  return KVQ_OK;
}

kvq_status check_layer(const kvq_layer *L) {
  if (!L) return fail(KVQ_ERR_INVALID_ARG, "layer is NULL");
  if (L->head_dim != KVQ_HEAD_DIM)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d (only %d is supported)", L->head_dim, KVQ_HEAD_DIM);
  if (L->batch < 1 || L->n_kv_heads < 1)
    return fail(KVQ_ERR_INVALID_ARG, "batch %d and n_kv_heads %d must be >= 1", L->batch, L->n_kv_heads);
  if (L->capacity < 0 || L->capacity % KVQ_TILE_TOKENS)
    return fail(KVQ_ERR_INVALID_ARG, "capacity %d must be a non-negative multiple of %d",
                L->capacity, KVQ_TILE_TOKENS);
  if (L->tail_len < 0 || L->tail_len % KVQ_TILE_TOKENS)
    return fail(KVQ_ERR_INVALID_ARG, "tail_len %d must be a non-negative multiple of %d",
                L->tail_len, KVQ_TILE_TOKENS);
  if (L->capacity > KVQ_MAX_CAPACITY || L->tail_len > KVQ_MAX_CAPACITY)
    return fail(KVQ_ERR_INVALID_ARG, "capacity %d / tail_len %d above KVQ_MAX_CAPACITY %d (32-bit in-plane offsets)",
                L->capacity, L->tail_len, KVQ_MAX_CAPACITY);
  if (L->tail_format != KVQ_TAIL_F16 && L->tail_format != KVQ_TAIL_BF16)
    return fail(KVQ_ERR_INVALID_ARG, "tail_format %d is not a kvq_tail_format", L->tail_format);
  if (L->n_tokens < 0 || L->n_tokens > L->capacity)
    return fail(KVQ_ERR_INVALID_ARG, "n_tokens %d outside [0, capacity %d]", L->n_tokens, L->capacity);
  kvq_status s = check_plane(*L, L->k, "k");
  if (s != KVQ_OK) return s;
  s = check_plane(*L, L->v, "v");
  if (s != KVQ_OK) return s;
  if ((L->k.basis == KVQ_BASIS_LOWRANK) != (L->v.basis == KVQ_BASIS_LOWRANK))
    return fail(KVQ_ERR_UNSUPPORTED, "K and V must both or neither use the low-rank basis");
  if (L->k.basis == KVQ_BASIS_LOWRANK) {
    for (int h = 0; h < L->n_kv_heads; ++h)
      if (L->k.rank[h] != L->v.rank[h] || L->k.head_codec[h] != L->v.head_codec[h])
        return fail(KVQ_ERR_UNSUPPORTED, "low-rank head %d: K and V must share rank and codec", h);
  }
  return KVQ_OK;
}

PlaneArgs plane_args(const kvq_layer &L, const kvq_plane &p) {
  PlaneArgs a;
  memset(&a, 0, sizeof a);
  a.codes = reinterpret_cast<uint8_t *>(p.codes);
  a.scales = p.scales;
  a.mins = p.mins;
  a.tail = p.tail;
  a.w = p.w;
  a.proj = p.proj;
  a.codec = p.codec;
  a.basis = p.basis;
  a.hkv = L.n_kv_heads;
  a.capacity = L.capacity;
  a.tail_len = L.tail_len;
  a.tail_bf16 = L.tail_format == KVQ_TAIL_BF16;
  if (p.basis == KVQ_BASIS_LOWRANK) {
    int rows = 0, blks = 0;
    for (int h = 0; h < L.n_kv_heads; ++h) {
      a.hcodec[h] = (int8_t)p.head_codec[h];
      a.hrank[h] = (int16_t)p.rank[h];
      a.hrow_before[h] = rows;
      a.hblk_before[h] = blks;
      rows += row_bytes(p.head_codec[h], p.rank[h]);
      blks += p.rank[h] / block_len(p.rank[h]);
    }
    a.row_all = rows;
    a.blk_all = blks;
    a.codec = -1;
  }
  return a;
}

void plane_sizes(const kvq_layer &L, const kvq_plane &p, size_t &codes, size_t &scales,
                 size_t &mins, size_t &tail) {
  codes = scales = mins = 0;
  const size_t cap = (size_t)L.capacity;
  if (p.basis == KVQ_BASIS_LOWRANK) {
    for (int h = 0; h < L.n_kv_heads; ++h) {
      const int r = p.rank[h], c = p.head_codec[h];
      codes += cap * row_bytes(c, r);
      scales += cap * (r / block_len(r)) * 2;
      if (codec_family(c) == FAM_1) mins += cap * (r / block_len(r)) * 2;
    }
    codes *= L.batch;
    scales *= L.batch;
    mins *= L.batch;
  } else {
    const size_t planes = (size_t)L.batch * L.n_kv_heads;
    codes = planes * cap * row_bytes(p.codec, KVQ_HEAD_DIM);
    if (p.codec != KVQ_F16) scales = planes * cap * (KVQ_HEAD_DIM / 32) * 2;
    if (codec_family(p.codec) == FAM_1) mins = scales;
  }
  tail = (size_t)L.batch * L.n_kv_heads * L.tail_len * 2 * KVQ_HEAD_DIM;
}

int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int MAX_BODY_SPLITS = 1024;
constexpr int MAX_TAIL_SPLITS = 64;
constexpr int TAIL_TT = 64;
constexpr int TAIL_TILES_PER_SPLIT = DECODE_WG_WAVES;
// Fixed cost of one wave tile in the split planner, in bytes of streaming
// (about one loaded memory round trip per tile at the per-wave rate seen on
// MI355X).
constexpr double PLAN_TILE_COST = 16384.0;

// Relative decode time of a low-rank head's body per tile, by bits (1..4)
// and rank (16, 32, 64, 128): measured on MI355X as the kernel time of a
// layer whose eight heads all share that (rank, bits), 8 sequences of 128k
// tokens, less the fixed per-launch part (~10 us).  Other pairs:
// rank-proportional.
double lowrank_tile_cost(int codec, int rank) {
  static const double cost[4][4] = {{74, 79, 121, 219}, {77, 78, 120, 227}, {106, 104, 169, 338}, {76, 81, 137, 263}};
  const int bits = codec_bits(codec);
  const int ri = rank == 16 ? 0 : rank == 32 ? 1 : rank == 64 ? 2 : rank == 128 ? 3 : -1;
  if (codec_family(codec) == FAM_1 && bits >= 1 && bits <= 4 && ri >= 0) return cost[bits - 1][ri];
  return 30.0 + 0.7 * rank;
}

// Body bytes per token of a layer (codes, scales, mins of K and V; the mean
// over kv heads for low rank).
double body_token_bytes(const kvq_layer &L) {
  double sum = 0.0;
  for (const kvq_plane *p : {&L.k, &L.v}) {
    if (p->basis == KVQ_BASIS_LOWRANK) {
      double t = 0.0;
      for (int h = 0; h < L.n_kv_heads; ++h) {
        const int r = p->rank[h], c = p->head_codec[h], nb = r / block_len(r);
        t += row_bytes(c, r) + nb * 2 * (codec_family(c) == FAM_1 ? 2 : 1);
      }
      sum += t / L.n_kv_heads;
    } else {
      const int c = p->codec;
      sum += row_bytes(c, KVQ_HEAD_DIM) +
             (c == KVQ_F16 ? 0 : (KVQ_HEAD_DIM / 32) * 2 * (codec_family(c) == FAM_1 ? 2 : 1));
    }
  }
  return sum;
}

int max_splits(const kvq_layer &L) {
  const int tt = decode_tile_tokens(L.k.codec, L.v.codec, L.k.basis);
  int body = (L.capacity + tt - 1) / tt;
  if (body > MAX_BODY_SPLITS) body = MAX_BODY_SPLITS;
  int tail = (L.tail_len + TAIL_TT - 1) / TAIL_TT;
  if (tail > MAX_TAIL_SPLITS) tail = MAX_TAIL_SPLITS;
  return (body > 0 ? body : 1) + tail;
}

struct WsLayout {
  size_t cnt, part, total;
};

// Workspace: split-completion counters (fixed size and place, zero between
// calls), then the split partials.
WsLayout ws_layout(const kvq_layer &L, int Hq, int S) {
  WsLayout w;
  const size_t bh = (size_t)L.batch * Hq;
  w.cnt = 0;
  w.part = align256(DECODE_CNT_BYTES);
  w.total = w.part + align256(bh * (size_t)S * PSTRIDE * sizeof(float));
  return w;
}

}  // namespace

namespace kvq {
// Status setters for the other host translation units (detail for
// kvq_last_error).
kvq_status api_fail(kvq_status s, const char *detail) { return fail(s, "%s", detail); }
kvq_status api_ok() { return ok(); }
}  // namespace kvq

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

#ifndef KVQ_SOURCE_HASH
#define KVQ_SOURCE_HASH "unknown"
#endif
const char *kvq_source_hash(void) { return KVQ_SOURCE_HASH; }

const char *kvq_last_error(void) { return g_err; }

const char *kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARG: return "KVQ_ERR_INVALID_ARG";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_CAPACITY: return "KVQ_ERR_CAPACITY";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP";
  }
  return "KVQ_ERR_UNKNOWN";
}

kvq_status kvq_plane_bytes(const kvq_layer *layer, int32_t which, size_t *codes_bytes,
                           size_t *scales_bytes, size_t *mins_bytes, size_t *tail_bytes) {
  kvq_status s = check_layer(layer);
  if (s != KVQ_OK && s != KVQ_ERR_INVALID_ARG) return s;
  if (!layer) return s;
  // sizes only need shapes, codecs and (low rank) the host tables
  if (which != 0 && which != 1) return fail(KVQ_ERR_INVALID_ARG, "which must be 0 (K) or 1 (V)");
  const kvq_plane &p = which ? layer->v : layer->k;
  if (layer->head_dim != KVQ_HEAD_DIM || layer->batch < 1 || layer->n_kv_heads < 1 ||
      layer->capacity < 0 || layer->capacity % KVQ_TILE_TOKENS || layer->tail_len < 0 ||
      layer->tail_len % KVQ_TILE_TOKENS)
    return fail(KVQ_ERR_INVALID_ARG, "bad layer shape");
  if (p.basis == KVQ_BASIS_LOWRANK) {
    if (!p.rank || !p.head_codec || layer->n_kv_heads > KVQ_MAX_LOWRANK_HEADS)
      return fail(KVQ_ERR_INVALID_ARG, "low-rank plane needs rank and head_codec tables");
    for (int h = 0; h < layer->n_kv_heads; ++h) {
      const int r = p.rank[h], c = p.head_codec[h];
      if (!(r == 16 || r == 32 || r == 64 || r == 128) || !codec_ok(c) || c == KVQ_F16)
        return fail(KVQ_ERR_INVALID_ARG, "low-rank head %d: bad rank %d or codec %d", h, r, c);
    }
  } else if (!codec_ok(p.codec)) {
    return fail(KVQ_ERR_INVALID_ARG, "codec %d is not a kvq_codec", p.codec);
  }
  size_t c, sc, m, t;
  plane_sizes(*layer, p, c, sc, m, t);
  if (codes_bytes) *codes_bytes = c;
  if (scales_bytes) *scales_bytes = sc;
  if (mins_bytes) *mins_bytes = m;
  if (tail_bytes) *tail_bytes = t;
  return ok();
}

kvq_status kvq_quantize_append(const kvq_layer *layer, const float *k_new, const float *v_new,
                               int32_t n_new, void *stream) {
  kvq_status s = check_layer(layer);
  if (s != KVQ_OK) return s;
  if (!k_new || !v_new) return fail(KVQ_ERR_INVALID_ARG, "k_new / v_new is NULL");
  if (n_new < 1) return fail(KVQ_ERR_INVALID_ARG, "n_new %d must be >= 1", n_new);
  if ((long long)layer->n_tokens + n_new > layer->capacity)
    return fail(KVQ_ERR_CAPACITY, "n_tokens %d + n_new %d exceeds capacity %d", layer->n_tokens,
                n_new, layer->capacity);
  if ((long long)layer->batch * n_new * layer->n_kv_heads * 2 > 0x7fffffffLL)
    return fail(KVQ_ERR_UNSUPPORTED, "append too large for one launch; split n_new");
  const PlaneArgs kp = plane_args(*layer, layer->k), vp = plane_args(*layer, layer->v);
  hipError_t e = launch_append(kp, vp, k_new, v_new, layer->batch, n_new, layer->n_tokens,
                               layer->seq_tokens,
                               reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

kvq_status kvq_dequantize(const kvq_layer *layer, int32_t which, float *out, void *stream) {
  kvq_status s = check_layer(layer);
  if (s != KVQ_OK) return s;
  if (which != 0 && which != 1) return fail(KVQ_ERR_INVALID_ARG, "which must be 0 (K) or 1 (V)");
  if (layer->n_tokens == 0) return ok();
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out is NULL");
  if ((long long)layer->batch * layer->n_kv_heads > 65535LL * 65535LL || layer->batch > 65535 ||
      layer->n_kv_heads > 65535)
    return fail(KVQ_ERR_UNSUPPORTED, "batch or n_kv_heads above 65535");
  const PlaneArgs p = plane_args(*layer, which ? layer->v : layer->k);
  hipError_t e = launch_dequant(p, layer->batch, layer->n_tokens, layer->seq_tokens, out,
                                reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return ok();
}

kvq_status kvq_transcode_layer(const kvq_layer *src, const kvq_layer *dst, void *stream) {
  kvq_status s = check_layer(src);
  if (s != KVQ_OK) return s;
  s = check_layer(dst);
  if (s != KVQ_OK) return s;
  if (src->batch != dst->batch || src->n_kv_heads != dst->n_kv_heads ||
      src->capacity != dst->capacity || src->tail_len != dst->tail_len ||
      src->n_tokens != dst->n_tokens || src->tail_format != dst->tail_format)
    return fail(KVQ_ERR_INVALID_ARG, "src and dst layers differ in shape or n_tokens");
  if (src->k.basis != dst->k.basis || src->v.basis != dst->v.basis)
    return fail(KVQ_ERR_INVALID_ARG, "transcode keeps the basis: src and dst bases differ");
  if (src->k.basis == KVQ_BASIS_LOWRANK || src->v.basis == KVQ_BASIS_LOWRANK)
    return fail(KVQ_ERR_UNSUPPORTED, "transcode of low-rank planes is not supported");
  if (src->k.codes == dst->k.codes || src->v.codes == dst->v.codes)
    return fail(KVQ_ERR_INVALID_ARG, "transcode is out of place: src and dst codes alias");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int which = 0; which < 2; ++which) {
    const kvq_plane &ps = which ? src->v : src->k;
    const kvq_plane &pd = which ? dst->v : dst->k;
    hipError_t e = launch_transcode(plane_args(*src, ps), plane_args(*dst, pd), src->batch,
                                    src->n_tokens, st);
    if (e != hipSuccess) return hip_fail(e, "transcode launch");
  }
  return ok();
}

size_t kvq_decode_workspace_bytes(const kvq_layer *layer, int32_t n_q_heads) {
  if (!layer || n_q_heads < 1 || layer->batch < 1) return 0;
  if (layer->capacity < 0 || layer->tail_len < 0) return 0;
  return ws_layout(*layer, n_q_heads, max_splits(*layer)).total;
}

}  // extern "C"

namespace {

// Decode of `layer` (already validated).  Fused step: k_new / v_new non-null
// and layer.n_tokens already counting the new token (the kernel writes it);
// seq_add is added to every seq_tokens entry.
// check_only: run every check, launch nothing.
kvq_status decode_impl(const kvq_layer &L, const float *q, int32_t n_q_heads, float sm_scale,
                       float *out, void *ws, size_t ws_bytes, int32_t body_splits, void *stream,
                       const float *k_new, const float *v_new, int seq_add, bool check_only = false) {
  if (!q || !out) return fail(KVQ_ERR_INVALID_ARG, "q / out is NULL");
  if (n_q_heads < 1 || n_q_heads % L.n_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "n_q_heads %d must be a positive multiple of n_kv_heads %d",
                n_q_heads, L.n_kv_heads);
  if (L.n_tokens < 1) return fail(KVQ_ERR_INVALID_ARG, "decode needs n_tokens >= 1");
  if (body_splits < 0) return fail(KVQ_ERR_INVALID_ARG, "body_splits %d < 0", body_splits);
  if (L.k.basis != L.v.basis)
    return fail(KVQ_ERR_UNSUPPORTED, "decode needs K and V in the same basis");

  DecodePlan P;
  P.B = L.batch;
  P.Hkv = L.n_kv_heads;
  P.Hq = n_q_heads;
  P.G = n_q_heads / L.n_kv_heads;
  P.HG = decode_head_group(P.G);
  P.NHG = P.G / P.HG;
  P.T = L.n_tokens;
  P.tail_tokens = L.tail_len < P.T ? L.tail_len : P.T;
  P.body_tokens = P.T - P.tail_tokens;
  if (L.k.basis == KVQ_BASIS_LOWRANK) {
    for (int h = 0; h < L.n_kv_heads; ++h)
      if (!decode_lowrank_supported(L.k.head_codec[h], L.k.rank[h]))
        return fail(KVQ_ERR_UNSUPPORTED, "low-rank head %d: codec %d at rank %d not supported by decode",
                    h, L.k.head_codec[h], L.k.rank[h]);
  } else if (!decode_pair_supported(L.k.codec, L.v.codec, P.HG)) {
    return fail(KVQ_ERR_UNSUPPORTED, "decode of K codec %d with V codec %d (group %d) not supported",
                L.k.codec, L.v.codec, P.HG);
  }
  P.tt_body = decode_tile_tokens(L.k.codec, L.v.codec, L.k.basis);
  const int units = P.B * P.Hkv * P.NHG;
  const int tail_tiles = (P.tail_tokens + TAIL_TT - 1) / TAIL_TT;
  const int body_tiles = (P.body_tokens + P.tt_body - 1) / P.tt_body;
  int tail_want = tail_tiles > 0 ? (tail_tiles + TAIL_TILES_PER_SPLIT - 1) / TAIL_TILES_PER_SPLIT : 0;
  if (tail_want > MAX_TAIL_SPLITS) tail_want = MAX_TAIL_SPLITS;
  int body_want = body_tiles > 0 ? 1 : 0;
  if (body_tiles > 0 && body_splits > 0) {
    body_want = body_splits;
  } else if (body_tiles > 0) {
    // One round of workgroups (the resident workgroups of all CUs hold the
    // whole grid), split between body and tail so that the slowest wave is
    // as fast as possible.  Wave w of a split takes tiles w, w + 8, ...; a
    // wave's time is modelled as its tile count times (a fixed per-tile
    // cost, mostly one memory round trip, + the tile's bytes).  A binary16
    // tail tile holds 2.5x the bytes of a q8/q4 body tile, so one tail
    // split per unit would make the tail wave the slowest.  Ties keep the
    // fewest tail splits.
    const int per_unit = (DECODE_WG_PER_CU * device_cus()) / units;
    const double cb = PLAN_TILE_COST + (double)P.tt_body * body_token_bytes(L);
    const double ct = PLAN_TILE_COST + (double)TAIL_TT * 2 * 2 * KVQ_HEAD_DIM;
    int st_hi = tail_tiles < MAX_TAIL_SPLITS ? tail_tiles : MAX_TAIL_SPLITS;
    if (st_hi > per_unit - 1) st_hi = per_unit - 1;
    const int st_lo = tail_tiles > 0 ? 1 : 0;
    if (st_hi < st_lo) st_hi = st_lo;
    double best = -1.0;
    for (int st = st_lo; st <= st_hi; ++st) {
      int sb = per_unit - st;
      if (sb < 1) sb = 1;
      if (sb > body_tiles) sb = body_tiles;
      const int tpb = (body_tiles + sb - 1) / sb;
      const int tpt = st > 0 ? (tail_tiles + st - 1) / st : 0;
      const double wb = (double)((tpb + DECODE_WG_WAVES - 1) / DECODE_WG_WAVES) * cb;
      const double wt = (double)((tpt + DECODE_WG_WAVES - 1) / DECODE_WG_WAVES) * ct;
      const double cost = wb > wt ? wb : wt;
      if (best < 0.0 || cost < best) {
        best = cost;
        body_want = (body_tiles + tpb - 1) / tpb;
        tail_want = st;
      }
    }
  }
  if (tail_tiles > 0) {
    P.tiles_per_split_tail = (tail_tiles + tail_want - 1) / tail_want;
    P.S_tail = (tail_tiles + P.tiles_per_split_tail - 1) / P.tiles_per_split_tail;
  } else {
    P.tiles_per_split_tail = 1;
    P.S_tail = 0;
  }
  if (body_tiles > 0) {
    int want = body_want;
    if (want > MAX_BODY_SPLITS) want = MAX_BODY_SPLITS;
    if (want > body_tiles) want = body_tiles;
    if (want < 1) want = 1;
    P.tiles_per_split_body = (body_tiles + want - 1) / want;
    P.S_body = (body_tiles + P.tiles_per_split_body - 1) / P.tiles_per_split_body;
  } else {
    P.tiles_per_split_body = 1;
    P.S_body = 0;
  }
  // Low rank: a tile's decode time depends on the head's (rank, bits), so
  // the body workgroups of a batch entry are shared out over its kv heads in
  // proportion to that time (largest remainder); explicit body_splits keep
  // one count for every head.
  int16_t lr_sb[KVQ_MAX_LOWRANK_HEADS] = {0}, lr_tp[KVQ_MAX_LOWRANK_HEADS] = {0};
  if (L.k.basis == KVQ_BASIS_LOWRANK && body_tiles > 0) {
    const int H = L.n_kv_heads;
    int sh[KVQ_MAX_LOWRANK_HEADS];
    if (body_splits > 0) {
      for (int h = 0; h < H; ++h) sh[h] = P.S_body;
    } else {
      int slots = (DECODE_WG_PER_CU * device_cus()) / (P.B * P.NHG) - H * P.S_tail;
      if (slots < H) slots = H;
      double w[KVQ_MAX_LOWRANK_HEADS], frac[KVQ_MAX_LOWRANK_HEADS], sum = 0.0;
      for (int h = 0; h < H; ++h) sum += (w[h] = lowrank_tile_cost(L.k.head_codec[h], L.k.rank[h]));
      int used = 0;
      for (int h = 0; h < H; ++h) {
        const double e = slots * w[h] / sum;
        sh[h] = (int)e;
        frac[h] = e - sh[h];
        if (sh[h] < 1) {
          sh[h] = 1;
          frac[h] = -1.0;
        }
        used += sh[h];
      }
      while (used < slots) {
        int best = -1;
        for (int h = 0; h < H; ++h)
          if (frac[h] >= 0.0 && (best < 0 || frac[h] > frac[best])) best = h;
        if (best < 0) break;
        ++sh[best];
        frac[best] = -1.0;
        ++used;
      }
    }
    int smax = 1;
    for (int h = 0; h < H; ++h) {
      int want = sh[h];
      if (want > MAX_BODY_SPLITS) want = MAX_BODY_SPLITS;
      if (want > body_tiles) want = body_tiles;
      if (want < 1) want = 1;
      const int tps = (body_tiles + want - 1) / want;
      lr_tp[h] = (int16_t)tps;
      lr_sb[h] = (int16_t)((body_tiles + tps - 1) / tps);
      if (lr_sb[h] > smax) smax = lr_sb[h];
    }
    P.S_body = smax;
  }
  P.S_total = P.S_body + P.S_tail;

  const WsLayout W = ws_layout(L, n_q_heads, P.S_total);
  if (!ws) return fail(KVQ_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < W.total)
    return fail(KVQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, W.total);
  if ((long long)P.Hkv * P.NHG > 65535 || P.B > 65535)
    return fail(KVQ_ERR_UNSUPPORTED, "grid too large (kv heads x head groups or batch above 65535)");
  if (units > DECODE_MAX_UNITS)
    return fail(KVQ_ERR_UNSUPPORTED, "batch x kv heads x head groups = %d above %d", units,
                DECODE_MAX_UNITS);

  if (check_only) return KVQ_OK;
  uint8_t *wsb = reinterpret_cast<uint8_t *>(ws);
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.k = plane_args(L, L.k);
  a.v = plane_args(L, L.v);
  a.part = reinterpret_cast<float *>(wsb + W.part);
  a.out = out;
  a.cnt = reinterpret_cast<unsigned *>(wsb + W.cnt);
  a.seq = L.seq_tokens;
  a.seq_add = seq_add;
  a.k_new = k_new;
  a.v_new = v_new;
  a.T = P.T;
  a.N = L.tail_len;
  a.B = P.B;
  a.Hkv = P.Hkv;
  a.Hq = P.Hq;
  a.G = P.G;
  a.HG = P.HG;
  a.NHG = P.NHG;
  a.body_tokens = P.body_tokens;
  a.tail_tokens = P.tail_tokens;
  a.S_body = P.S_body;
  a.S_tail = P.S_tail;
  a.S_total = P.S_total;
  a.tps_body = P.tiles_per_split_body;
  a.tps_tail = P.tiles_per_split_tail;
  a.tt_body = P.tt_body;
  a.lr_body_all = 0;
  for (int h = 0; h < KVQ_MAX_LOWRANK_HEADS; ++h) {
    a.lr_sbody[h] = lr_sb[h];
    a.lr_tps[h] = lr_tp[h];
    a.lr_first[h] = (int16_t)a.lr_body_all;
    if (h < L.n_kv_heads) a.lr_body_all += lr_sb[h];
  }
  hipError_t e = launch_decode(a, q, sm_scale, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention_splits(const kvq_layer *layer, const float *q, int32_t n_q_heads,
                                       float sm_scale, float *out, void *ws, size_t ws_bytes,
                                       int32_t body_splits, void *stream) {
  kvq_status s = check_layer(layer);
  if (s != KVQ_OK) return s;
  return decode_impl(*layer, q, n_q_heads, sm_scale, out, ws, ws_bytes, body_splits, stream,
                     nullptr, nullptr, 0);
}

}  // extern "C"

namespace {

// One decode step (append + decode) on a given workspace; check_only runs
// every check and launches nothing.
kvq_status append_decode_impl(const kvq_layer *layer, const float *k_new, const float *v_new,
                              const float *q, int32_t n_q_heads, float sm_scale, float *out, void *ws,
                              size_t ws_bytes, void *stream, bool check_only) {
  kvq_status s = check_layer(layer);
  if (s != KVQ_OK) return s;
  if (!k_new || !v_new) return fail(KVQ_ERR_INVALID_ARG, "k_new / v_new is NULL");
  if ((long long)layer->n_tokens + 1 > layer->capacity)
    return fail(KVQ_ERR_CAPACITY, "n_tokens %d + 1 exceeds capacity %d", layer->n_tokens,
                layer->capacity);
  kvq_layer after = *layer;
  after.n_tokens = layer->n_tokens + 1;
  // one launch: the workgroup whose tiles hold the new token writes its K
  // and V rows (every head group's owner the same bytes) before reading
  return decode_impl(after, q, n_q_heads, sm_scale, out, ws, ws_bytes, 0, stream, k_new, v_new, 1,
                     check_only);
}

// Scratch of the allocation-free step: the decode workspace (completion
// counters and split partials) in a fixed device array.  Each
// GPU the library runs on holds its own copy for the life of the process;
// host code reaches it only through the address hipGetSymbolAddress gives
// on that device.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

__global__ void zero_words_kernel(uint32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct ScratchDev {
  void *ptr = nullptr;   // device address of `scratch` on this device
  bool armed = false;    // completion counters cleared
};
constexpr int SCRATCH_MAX_DEVICES = 64;
ScratchDev g_scratch[SCRATCH_MAX_DEVICES];
std::mutex g_scratch_mu;

}  // namespace

extern "C" {

kvq_status kvq_append_decode(const kvq_layer *layer, const float *k_new, const float *v_new,
                             const float *q, int32_t n_q_heads, float sm_scale, float *out,
                             void *ws, size_t ws_bytes, void *stream) {
  return append_decode_impl(layer, k_new, v_new, q, n_q_heads, sm_scale, out, ws, ws_bytes, stream,
                            false);
}

kvq_status kvq_append_decode_noalloc(const kvq_layer *layer, const float *k_new, const float *v_new,
                                     const float *q, int32_t n_q_heads, float sm_scale, float *out,
                                     void *stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(KVQ_ERR_UNSUPPORTED, "device %d above the %d the allocation-free step tracks", dev,
                SCRATCH_MAX_DEVICES);
  void *ptr = nullptr;
  bool armed = false;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev].ptr) {
      void *p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      g_scratch[dev].ptr = p;
    }
    ptr = g_scratch[dev].ptr;
    armed = g_scratch[dev].armed;
  }
  kvq_status s = append_decode_impl(layer, k_new, v_new, q, n_q_heads, sm_scale, out, ptr,
                                    NOALLOC_SCRATCH_BYTES, stream, true);
  if (s == KVQ_ERR_WORKSPACE) {
    char detail[512];
    snprintf(detail, sizeof detail, "%s", g_err);
    return fail(KVQ_ERR_WORKSPACE, "kvq_append_decode_noalloc: the layer needs more scratch than the "
                "fixed %zu bytes (%s); use kvq_append_decode with a workspace", NOALLOC_SCRATCH_BYTES,
                detail);
  }
  if (s != KVQ_OK) return s;
  if (!armed) {
    // the completion counters start at zero; every completed step leaves
    // them zero again
    const int n = (int)(DECODE_CNT_BYTES / sizeof(uint32_t));
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<uint32_t *>(ptr), n);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scratch counter clear");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    g_scratch[dev].armed = true;
  }
  return append_decode_impl(layer, k_new, v_new, q, n_q_heads, sm_scale, out, ptr, NOALLOC_SCRATCH_BYTES,
                            stream, false);
}

kvq_status kvq_decode_attention(const kvq_layer *layer, const float *q, int32_t n_q_heads,
                                float sm_scale, float *out, void *ws, size_t ws_bytes,
                                void *stream) {
  return kvq_decode_attention_splits(layer, q, n_q_heads, sm_scale, out, ws, ws_bytes, 0, stream);
}

kvq_status kvq_timing_begin(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20))
    return fail(KVQ_ERR_INVALID_ARG, "timing capacity %d outside [1, 1<<20]", capacity);
  hipError_t e = kvq::timing_begin(capacity);
  return e == hipSuccess ? ok() : hip_fail(e, "kvq_timing_begin");
}

kvq_status kvq_timing_durations(float *ms_each, int32_t capacity, int32_t *count) {
  if (!ms_each || !count || capacity < 0)
    return fail(KVQ_ERR_INVALID_ARG, "ms_each and count must be non-NULL, capacity >= 0");
  int n = 0;
  hipError_t e = kvq::timing_durations(ms_each, capacity, &n);
  *count = n;
  return e == hipSuccess ? ok() : hip_fail(e, "kvq_timing_durations");
}

kvq_status kvq_timing_end(double *total_ms, int32_t *count) {
  int n = 0;
  hipError_t e = kvq::timing_end(total_ms, &n);
  if (count) *count = n;
  return e == hipSuccess ? ok() : hip_fail(e, "kvq_timing_end");
}

}  // extern "C"
