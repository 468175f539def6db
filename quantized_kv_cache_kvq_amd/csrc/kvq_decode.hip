// Decode attention over the packed cache: query pre-transforms, the launch
// of the split-K decode kernel (kvq_decode_impl.hpp, kvq_decode_q.hpp) and
// its event-timing hook.
//
// The computation (forum thread on decode bandwidth, second post): scores
// s_t = sm_scale <q, k_t>, softmax over t, output sum_t p_t v_t; the cache is
// read once per step, so the step is bound by HBM bandwidth (same thread,
// first post).  One launch does all of it: workgroups own context splits of
// a (batch entry, kv head, head group), write (m, l, o) partials, and the
// workgroup that finishes a unit last merges the splits (M = max m_s,
// L = sum l_s 2^(m_s - M), o = sum o_s 2^(m_s - M) / L) after taking body
// partials back to the raw basis (inverse Hadamard and 1/w for KVarN, P_h
// for low rank).
#include <vector>

#include "kvq_decode_impl.hpp"

namespace kvq {

// --------------------------------------------------- query pre-transforms --

// KVarN query: q' = H (q / w_k) / 128, scaled into the log2 domain; plain
// bodies with _1 keys only get the scaling.  Also the per-32-block sums of q'
// for _1 keys.  One wave per (batch entry, query head).
__global__ __launch_bounds__(64) void query_prep_kernel(const float *__restrict__ q,
                                                        const float *__restrict__ wk, int Hq,
                                                        int G, int hadamard, float scale,
                                                        float *__restrict__ qw,
                                                        float *__restrict__ qsum) {
  const int bh = blockIdx.x;
  const int h = bh % Hq;
  const int g = h / G;
  const int lane = threadIdx.x;
  float2 x = reinterpret_cast<const float2 *>(q + (long long)bh * D)[lane];
  if (hadamard) {
    const float *w = wk + (long long)g * D;
    float a = x.x / w[2 * lane], b = x.y / w[2 * lane + 1];
    float s0 = a + b, d0 = a - b;
    a = s0;
    b = d0;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      float pa = __shfl_xor(a, m, 64), pb = __shfl_xor(b, m, 64);
      bool upper = (lane & m) != 0;
      a = upper ? (pa - a) : (a + pa);
      b = upper ? (pb - b) : (b + pb);
    }
    x.x = a * (1.f / 128.f);
    x.y = b * (1.f / 128.f);
  }
  x.x *= scale;
  x.y *= scale;
  reinterpret_cast<float2 *>(qw + (long long)bh * D)[lane] = x;
  float sblk = x.x + x.y;
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) sblk += __shfl_xor(sblk, o, 64);
  if ((lane & 15) == 0) qsum[(long long)bh * 4 + lane / 16] = sblk;
}

// Low-rank query projection q_low = P_g^T q on the matrix cores, scaled into
// the log2 domain, plus per-block sums.  For kv head g the queries of its
// G heads over all batch entries form M = B*G rows; the product
// [M x 128] x [128 x r_g] runs as 16x16x4 fp32 MFMA tiles (fp32 inputs keep
// the binary16 entries of P and the binary32 queries exact in the products).
// One wave computes a 16-row by L-column tile (L = min(32, r_g): one block).
__global__ __launch_bounds__(64) void lowrank_query_kernel(const float *__restrict__ q,
                                                           PlaneArgs kp, int B, int Hq, int G,
                                                           float scale, float *__restrict__ qw,
                                                           float *__restrict__ qsum) {
  const int g = blockIdx.z;
  const int r = kp.hrank[g];
  const int L = r < 32 ? r : 32;
  const int jb = blockIdx.y;                 // block index along the rank
  if (jb * L >= r) return;
  const int m0 = blockIdx.x * 16;
  const int M = B * G;
  const int lane = threadIdx.x;
  const int i_a = lane & 15, k_a = lane >> 4;
  const uint16_t *P = kp.proj + (long long)g * D * D;

  const int ma = m0 + i_a;
  const float *qrow = nullptr;
  if (ma < M) qrow = q + ((long long)(ma / G) * Hq + g * G + ma % G) * D;

  // every load is issued before the products: the lane's 32 query values
  // once, then per 16-column tile its 32 entries of P
  float qa[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) qa[i] = qrow ? qrow[4 * i + k_a] : 0.f;
  float rowsum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int ct = 0; ct < L / 16; ++ct) {
    const int n0 = jb * L + ct * 16;
    uint16_t pb[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) pb[i] = P[(long long)(4 * i + k_a) * D + n0 + i_a];
    floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 4; ++i)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i], f16_bits_to_f32(pb[i]), c, 0, 0, 0);
    // D[i][j]: lane holds rows 4*(lane/16) + rr, column lane % 16
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int m = m0 + 4 * (lane >> 4) + rr;
      const float v = c[rr] * scale;
      if (m < M) qw[((long long)(m / G) * Hq + g * G + m % G) * D + n0 + (lane & 15)] = v;
      rowsum[rr] += v;
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    float v = rowsum[rr];
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int m = m0 + 4 * (lane >> 4) + rr;
    if ((lane & 15) == 0 && m < M) qsum[((long long)(m / G) * Hq + g * G + m % G) * 4 + jb] = v;
  }
}

// --------------------------------------------------------------- launcher --

int decode_tile_tokens(int kcodec, int vcodec, int basis) {
  (void)kcodec; (void)vcodec; (void)basis;
  return 64;   // one wave tile; a split owns whole multiples of it
}

int decode_head_group(int G) {
  const int cands[] = {8, 6, 4, 2, 1};
  for (int c : cands)
    if (G % c == 0) return c;
  return 1;
}

extern template hipError_t launch_decode_hg<1>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_hg<2>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_hg<4>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_hg<6>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_hg<8>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);

bool decode_lowrank_supported(int codec, int rank) { return decode_lowrank_supported_impl(codec, rank); }

bool decode_pair_supported(int kc, int vc, int hg) {
  if (!(hg == 1 || hg == 2 || hg == 4 || hg == 6 || hg == 8)) return false;
#define KVQ_PAIR_CHECK(K, V) if (kc == K && vc == V) return true;
  KVQ_DECODE_PAIRS(KVQ_PAIR_CHECK)
#undef KVQ_PAIR_CHECK
  return false;
}

// Optional event timing of the split-K decode kernel: one start/stop pair
// per decode call, stamped by that kernel's own dispatch.
namespace {
struct Timing {
  std::vector<hipEvent_t> ev;  // 2 per slot
  int used = 0;
  bool on = false;
};
Timing g_timing;
}  // namespace

void timing_next(hipEvent_t *ev0, hipEvent_t *ev1) {
  Timing &T = g_timing;
  const bool free = T.on && 2 * T.used < (int)T.ev.size();
  *ev0 = free ? T.ev[2 * T.used] : nullptr;
  *ev1 = free ? T.ev[2 * T.used + 1] : nullptr;
}

void timing_commit() {
  Timing &T = g_timing;
  if (T.on && 2 * T.used < (int)T.ev.size()) ++T.used;
}

hipError_t timing_begin(int capacity) {
  (void)timing_end(nullptr, nullptr);
  Timing &T = g_timing;
  T.ev.assign(2 * (size_t)capacity, nullptr);
  for (auto &e : T.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      e = nullptr;
      (void)timing_end(nullptr, nullptr);
      return r;
    }
  }
  T.used = 0;
  T.on = true;
  return hipSuccess;
}

hipError_t timing_end(double *total_ms, int *count) {
  Timing &T = g_timing;
  double sum = 0.0;
  hipError_t err = hipSuccess;
  for (int i = 0; i < T.used; ++i) {
    float ms = 0.f;
    hipError_t r = hipEventSynchronize(T.ev[2 * i + 1]);
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, T.ev[2 * i], T.ev[2 * i + 1]);
    if (r != hipSuccess && err == hipSuccess) err = r;
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (count) *count = T.used;
  for (auto e : T.ev)
    if (e) (void)hipEventDestroy(e);
  T.ev.clear();
  T.used = 0;
  T.on = false;
  return err;
}

hipError_t launch_decode(const DecodeArgs &args, const float *q, float sm_scale, float *qw,
                         float *qsum, float *out, hipStream_t stream, bool prep, bool need_qsum) {
  DecodeArgs a = args;
  const float scale2 = sm_scale * LOG2E;
  if (a.k.basis == KVQ_BASIS_LOWRANK) {
    dim3 g((a.B * a.G + 15) / 16, 4, a.Hkv);
    hipLaunchKernelGGL(lowrank_query_kernel, g, dim3(64), 0, stream, q, a.k, a.B, a.Hq, a.G,
                       scale2, qw, qsum);
    a.q_body = qw;
    a.qsum = qsum;
    a.scale_body = 1.f;
  } else if (prep) {
    hipLaunchKernelGGL(query_prep_kernel, dim3(a.B * a.Hq), dim3(64), 0, stream, q, a.k.w, a.Hq,
                       a.G, a.k.basis == KVQ_BASIS_HADAMARD ? 1 : 0, scale2, qw, qsum);
    a.q_body = qw;
    a.qsum = qsum;
    a.scale_body = 1.f;
  } else {
    a.q_body = q;
    a.qsum = qsum;
    a.scale_body = scale2;
  }
  (void)need_qsum;
  a.q_tail = q;
  a.scale_tail = scale2;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  hipError_t r;
  hipEvent_t ev0, ev1;
  timing_next(&ev0, &ev1);
  switch (a.HG) {
    case 1: r = launch_decode_hg<1>(a, stream, ev0, ev1); break;
    case 2: r = launch_decode_hg<2>(a, stream, ev0, ev1); break;
    case 4: r = launch_decode_hg<4>(a, stream, ev0, ev1); break;
    case 6: r = launch_decode_hg<6>(a, stream, ev0, ev1); break;
    case 8: r = launch_decode_hg<8>(a, stream, ev0, ev1); break;
    default: r = hipErrorNotSupported;
  }
  if (r != hipSuccess) return r;
  if (ev0) timing_commit();
  (void)out;   // merged into a.out by each unit's last workgroup
  return hipGetLastError();
}

}  // namespace kvq
