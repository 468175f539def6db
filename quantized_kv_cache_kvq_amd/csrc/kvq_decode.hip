// Decode attention over the packed cache: split-K flash-decode with the
// dequantisation done in registers.
//
// The computation (forum thread on decode bandwidth, second post): scores
// s_t = sm_scale <q, k_t>, softmax over t, output sum_t p_t v_t.  The cache
// is read once per step, so the kernel is bound by HBM bandwidth (same
// thread, first post).  Design for gfx950:
//
//  * Grid: one 256-thread workgroup per (batch entry, kv head, head group of
//    HG query heads sharing it, context split).  Splits cover the quantised
//    body and the binary16 precision tail; each writes an (m, l, o) partial.
//  * QK, token per thread: the 64-token tiled row layout makes "thread t
//    loads token t's row" a run of fully coalesced 16-byte loads (a wave
//    reads 1 KB contiguous per instruction).  The codes are unpacked in
//    registers; the HG query vectors are wave-uniform, so the compiler keeps
//    them in scalar registers and every multiply-add takes one from there.
//    Block scales are folded in once per 32-block: s += d_j * sum_i q_i c_i
//    (+ m_j * sum_i q_i for _1 codes).
//  * Online softmax in the log2 domain (scores pre-multiplied by log2 e);
//    the tile maximum is a wave shuffle reduction plus one LDS exchange.
//  * PV: the value tile is staged raw (packed) in LDS with the p*d_j
//    weights; thread (slot, group) then owns 8 output channels and walks the
//    tile's tokens, unpacking its 8 codes per token and accumulating HG x 8
//    outputs.  A cross-slot reduction through LDS closes each split.
//  * A second kernel combines the splits: M = max m_s, L = sum l_s 2^(m_s-M),
//    o = sum o_s 2^(m_s-M) / L, after taking body partials back to the raw
//    basis (inverse Hadamard and 1/w for KVarN, P_h for low rank).
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

  float rowsum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int ct = 0; ct < L / 16; ++ct) {
    const int n0 = jb * L + ct * 16;
    floatx4 c = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < D; k0 += 4) {
      const float av = qrow ? qrow[k0 + k_a] : 0.f;
      const float bv = f16_bits_to_f32(P[(long long)(k0 + k_a) * D + n0 + i_a]);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, c, 0, 0, 0);
    }
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

// ---------------------------------------------------------------- combine --

// One 256-thread workgroup per (batch entry, query head).  Split weights
// 2^(m_s - M) are computed once (thread per split), the outputs are summed
// by 4 split-groups x 64 channel pairs, then one wave takes the body sum
// back to the raw basis and writes the normalised result.
constexpr int CMB_MAX_SPLITS = 1024 + 64;

__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a, float *__restrict__ out) {
  __shared__ float wts[CMB_MAX_SPLITS];
  __shared__ float red[4][2][D];
  __shared__ float sred[2][8];
  __shared__ float olow[D];
  const int bh = blockIdx.x;
  const int h = bh % a.Hq;
  const int g = h / a.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *pr = a.part + (long long)bh * a.S_total * PSTRIDE;

  // segment maxima (body: splits [0, S_body), tail: [S_body, S_total))
  float mb = NEG_INF, mt = NEG_INF;
  for (int s = tid; s < a.S_total; s += 256) {
    const float m = pr[(long long)s * PSTRIDE];
    if (s < a.S_body) mb = fmaxf(mb, m); else mt = fmaxf(mt, m);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mb = fmaxf(mb, __shfl_xor(mb, o, 64));
    mt = fmaxf(mt, __shfl_xor(mt, o, 64));
  }
  if (lane == 0) { sred[0][wave] = mb; sred[1][wave] = mt; }
  __syncthreads();
  const float Mb = fmaxf(fmaxf(sred[0][0], sred[0][1]), fmaxf(sred[0][2], sred[0][3]));
  const float Mt = fmaxf(fmaxf(sred[1][0], sred[1][1]), fmaxf(sred[1][2], sred[1][3]));
  __syncthreads();

  // split weights and segment sums of l
  float lb = 0.f, lt = 0.f;
  for (int s = tid; s < a.S_total; s += 256) {
    const float *p = pr + (long long)s * PSTRIDE;
    const float Mseg = s < a.S_body ? Mb : Mt;
    const float w = p[0] == NEG_INF ? 0.f : exp2f(p[0] - Mseg);
    wts[s] = w;
    if (s < a.S_body) lb = fmaf(w, p[1], lb); else lt = fmaf(w, p[1], lt);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lb += __shfl_xor(lb, o, 64);
    lt += __shfl_xor(lt, o, 64);
  }
  if (lane == 0) { sred[0][4 + wave] = lb; sred[1][4 + wave] = lt; }
  __syncthreads();
  const float Lb = sred[0][4] + sred[0][5] + sred[0][6] + sred[0][7];
  const float Lt = sred[1][4] + sred[1][5] + sred[1][6] + sred[1][7];

  // weighted sums of the partial outputs: wave w takes splits w, w + 4, ...
  float ob0 = 0.f, ob1 = 0.f, ot0 = 0.f, ot1 = 0.f;
  for (int s = wave; s < a.S_total; s += 4) {
    const float2 v = *reinterpret_cast<const float2 *>(pr + (long long)s * PSTRIDE + 4 + 2 * lane);
    const float w = wts[s];
    if (s < a.S_body) { ob0 = fmaf(w, v.x, ob0); ob1 = fmaf(w, v.y, ob1); }
    else { ot0 = fmaf(w, v.x, ot0); ot1 = fmaf(w, v.y, ot1); }
  }
  red[wave][0][2 * lane] = ob0;
  red[wave][0][2 * lane + 1] = ob1;
  red[wave][1][2 * lane] = ot0;
  red[wave][1][2 * lane + 1] = ot1;
  __syncthreads();
  if (wave != 0) return;
  ob0 = red[0][0][2 * lane] + red[1][0][2 * lane] + red[2][0][2 * lane] + red[3][0][2 * lane];
  ob1 = red[0][0][2 * lane + 1] + red[1][0][2 * lane + 1] + red[2][0][2 * lane + 1] + red[3][0][2 * lane + 1];
  ot0 = red[0][1][2 * lane] + red[1][1][2 * lane] + red[2][1][2 * lane] + red[3][1][2 * lane];
  ot1 = red[0][1][2 * lane + 1] + red[1][1][2 * lane + 1] + red[2][1][2 * lane + 1] + red[3][1][2 * lane + 1];

  // body partial back to the raw basis
  const int nv = a.v.basis == KVQ_BASIS_LOWRANK ? a.v.hrank[g] : D;
  if (a.S_body > 0) {
    if (a.v.basis == KVQ_BASIS_HADAMARD) {
      float x0 = ob0, x1 = ob1;
      float s0 = x0 + x1, d0 = x0 - x1;
      x0 = s0;
      x1 = d0;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        float p0 = __shfl_xor(x0, m, 64), p1 = __shfl_xor(x1, m, 64);
        bool upper = (lane & m) != 0;
        x0 = upper ? (p0 - x0) : (x0 + p0);
        x1 = upper ? (p1 - x1) : (x1 + p1);
      }
      const float *w = a.v.w + (long long)g * D;
      ob0 = x0 * (1.f / 128.f) / w[2 * lane];
      ob1 = x1 * (1.f / 128.f) / w[2 * lane + 1];
    } else if (a.v.basis == KVQ_BASIS_LOWRANK) {
      olow[2 * lane] = 2 * lane < nv ? ob0 : 0.f;
      olow[2 * lane + 1] = 2 * lane + 1 < nv ? ob1 : 0.f;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint16_t *P = a.v.proj + (long long)g * D * D;
      float y0 = 0.f, y1 = 0.f;
      for (int k = 0; k < nv; ++k) {
        y0 = fmaf(f16_bits_to_f32(P[(long long)(2 * lane) * D + k]), olow[k], y0);
        y1 = fmaf(f16_bits_to_f32(P[(long long)(2 * lane + 1) * D + k]), olow[k], y1);
      }
      ob0 = y0;
      ob1 = y1;
    }
  }

  const float M = fmaxf(Mb, Mt);
  const float wb = Mb == NEG_INF ? 0.f : exp2f(Mb - M);
  const float wt = Mt == NEG_INF ? 0.f : exp2f(Mt - M);
  const float inv = 1.f / (wb * Lb + wt * Lt);
  float2 o;
  o.x = (wb * ob0 + wt * ot0) * inv;
  o.y = (wb * ob1 + wt * ot1) * inv;
  reinterpret_cast<float2 *>(out + (long long)bh * D)[lane] = o;
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
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(a.B * a.Hq), dim3(256), 0, stream, a, out);
  return hipGetLastError();
}

}  // namespace kvq
