// Device implementation of the split-K decode kernel (see kvq_decode.hip for
// the design notes).  Included by the per-head-group instantiation units.
#pragma once

#include "kvq_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {

constexpr int WG = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_huge_valf();

template <int A, int B> struct cmax { static constexpr int value = A > B ? A : B; };

// ------------------------------------------------------------- unpacking --

// Field of BITS bits at compile-time bit offset `bit` of a register array.
template <int BITS, bool SIGNED, int NW>
__device__ __forceinline__ int field(const uint32_t (&w)[NW], int bit) {
  const int wi = bit >> 5, sh = bit & 31;
  uint32_t lo = w[wi] >> sh;
  if (sh + BITS > 32) lo |= w[wi + 1] << (32 - sh);
  if (SIGNED) return ((int32_t)(lo << (32 - BITS))) >> (32 - BITS);
  return (int)(lo & ((1u << BITS) - 1u));
}

template <int NW>
__device__ __forceinline__ float half_at(const uint32_t (&w)[NW], int e) {
  const uint32_t bitsv = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
  return f16_bits_to_f32((uint16_t)bitsv);
}

// Load chunks [K0, K1) of a token row (R bytes, C-byte chunks) of a tiled
// plane into words; words[i] = row bytes [K0*C + 4i, K0*C + 4i + 4).
template <int R, int C, int K0, int K1, int NW>
__device__ __forceinline__ void load_row(const uint8_t *__restrict__ plane, long long t,
                                         bool valid, uint32_t (&w)[NW]) {
#pragma unroll
  for (int i = 0; i < NW; ++i) w[i] = 0u;
  if (!valid) return;
#pragma unroll
  for (int k = K0; k < K1; ++k) {
    const uint8_t *p = plane + tiled_offset(t, k, R, C);
    const int o = (k - K0) * C;   // byte offset inside words
    if constexpr (C == 16) {
      const uint4 v = *reinterpret_cast<const uint4 *>(p);
      w[o / 4 + 0] = v.x; w[o / 4 + 1] = v.y; w[o / 4 + 2] = v.z; w[o / 4 + 3] = v.w;
    } else if constexpr (C == 8) {
      const uint2 v = *reinterpret_cast<const uint2 *>(p);
      w[o / 4 + 0] = v.x; w[o / 4 + 1] = v.y;
    } else if constexpr (C == 4) {
      w[o / 4] = *reinterpret_cast<const uint32_t *>(p);
    } else if constexpr (C == 2) {
      w[o / 4] |= (uint32_t)(*reinterpret_cast<const uint16_t *>(p)) << (8 * (o % 4));
    } else {
      w[o / 4] |= (uint32_t)(*p) << (8 * (o % 4));
    }
  }
}

// Per-token binary16 side values (scales or mins) of NB blocks.
template <int NB>
__device__ __forceinline__ void load_side(const uint16_t *__restrict__ p, bool valid, float (&v)[NB > 0 ? NB : 1]) {
  if constexpr (NB == 0) {
    v[0] = 1.f;
  } else if constexpr (NB == 4) {
    uint2 r = valid ? *reinterpret_cast<const uint2 *>(p) : make_uint2(0u, 0u);
    v[0] = f16_bits_to_f32(r.x & 0xFFFF); v[1] = f16_bits_to_f32(r.x >> 16);
    v[2] = f16_bits_to_f32(r.y & 0xFFFF); v[3] = f16_bits_to_f32(r.y >> 16);
  } else if constexpr (NB == 2) {
    uint32_t r = valid ? *reinterpret_cast<const uint32_t *>(p) : 0u;
    v[0] = f16_bits_to_f32(r & 0xFFFF); v[1] = f16_bits_to_f32(r >> 16);
  } else {
#pragma unroll
    for (int j = 0; j < NB; ++j) v[j] = valid ? f16_bits_to_f32(p[j]) : 0.f;
  }
}

// --------------------------------------------------------- configuration --

template <int HG_, int KC_, int VC_, int NK_, int NV_, int TT_>
struct Cfg {
  static constexpr int HG = HG_, KC = KC_, VC = VC_, NK = NK_, NV = NV_, TT = TT_;
  static constexpr int TPT = WG / TT;                       // threads per token in QK
  static constexpr int KBITS = codec_bits(KC), KFAM = codec_family(KC);
  static constexpr int VBITS = codec_bits(VC), VFAM = codec_family(VC);
  static constexpr int RK = row_bytes(KC, NK), CK = chunk_bytes(RK);
  static constexpr int RV = row_bytes(VC, NV), CV = chunk_bytes(RV);
  static constexpr int LK = KFAM == FAM_F16 ? 32 : block_len(NK);
  static constexpr int LV = VFAM == FAM_F16 ? NV : block_len(NV);
  static constexpr int NBK = KFAM == FAM_F16 ? 0 : NK / LK;
  static constexpr int NBV = VFAM == FAM_F16 ? 1 : NV / LV;
  static constexpr int PITCH = ((RV + 15) / 16) * 16 + 16;  // LDS row pitch of V
  static constexpr int HGP = (HG + 3) / 4 * 4;
  static constexpr int NGV = NV / 8;                        // 8-channel groups
  static constexpr int NSLOT = WG / NGV;
  static constexpr int LDS_V = TT * PITCH;
  static constexpr int LDS_PD = TT * NBV * HGP * 4;
  static constexpr int LDS_RED = NSLOT * (NV + 4) * 4;
  static constexpr int LDS_MAIN = (cmax<LDS_V + LDS_PD, LDS_RED>::value + 15) / 16 * 16;
  static constexpr int LDS_MISC = 4 * 8 * 4 + TT * 8 * 4 + WG * 4;   // wave maxima, QK halves, sums
  static constexpr int LDS_BYTES = LDS_MAIN + LDS_MISC;
};

constexpr int tile_tokens_for(int kc, int vc) {
  return (kc == KVQ_F16 || vc == KVQ_F16) ? 128 : 256;
}

// ----------------------------------------------------------------- QK ----

// Partial score of the channels [d0, d1) of one token for HG heads.
template <class C, int PART>
__device__ __forceinline__ void qk_part(const uint8_t *__restrict__ kplane,
                                        const uint16_t *__restrict__ ksc,
                                        const uint16_t *__restrict__ kmn, long long t, bool valid,
                                        const float *__restrict__ q, int qstride,
                                        const float *__restrict__ qs, float (&s)[C::HG]) {
  constexpr int EB = C::KFAM == FAM_F16 ? 16 : C::KBITS;      // bits per element
  constexpr int d0 = PART * C::NK / C::TPT, d1 = (PART + 1) * C::NK / C::TPT;
  constexpr int byte0 = d0 * EB / 8, byte1 = (d1 * EB + 7) / 8;
  constexpr int K0a = byte0 / C::CK;
  constexpr int K0 = (C::CK < 4) ? 0 : K0a;
  constexpr int K1 = (byte1 + C::CK - 1) / C::CK;
  constexpr int NW = ((K1 - K0) * C::CK + 3) / 4;
  uint32_t w[NW];
  load_row<C::RK, C::CK, K0, K1, NW>(kplane, t, valid, w);
  float dk[C::NBK > 0 ? C::NBK : 1], mk[C::NBK > 0 ? C::NBK : 1];
  load_side<C::NBK>(ksc + t * C::NBK, valid, dk);
  if constexpr (C::KFAM == FAM_1) load_side<C::NBK>(kmn + t * C::NBK, valid, mk);
#pragma unroll
  for (int h = 0; h < C::HG; ++h) s[h] = 0.f;
#pragma unroll
  for (int j = d0 / C::LK; j < d1 / C::LK; ++j) {
    float a[C::HG];
#pragma unroll
    for (int h = 0; h < C::HG; ++h) a[h] = 0.f;
#pragma unroll
    for (int i = 0; i < C::LK; ++i) {
      const int e = j * C::LK + i;
      const int bit = e * EB - 8 * K0 * C::CK;
      float v;
      if constexpr (C::KFAM == FAM_F16) v = half_at(w, bit / 16);
      else v = (float)field<C::KBITS, C::KFAM == FAM_0>(w, bit);
#pragma unroll
      for (int h = 0; h < C::HG; ++h) a[h] = fmaf(q[h * qstride + e], v, a[h]);
    }
#pragma unroll
    for (int h = 0; h < C::HG; ++h) {
      if constexpr (C::KFAM == FAM_F16) {
        s[h] += a[h];
      } else {
        s[h] = fmaf(dk[j], a[h], s[h]);
        if constexpr (C::KFAM == FAM_1) s[h] = fmaf(mk[j], qs[h * 4 + j], s[h]);
      }
    }
  }
}

// ------------------------------------------------------- one split range --

struct SplitIO {
  const uint8_t *kcodes; const uint16_t *ksc; const uint16_t *kmn;
  const uint8_t *vcodes; const uint16_t *vsc; const uint16_t *vmn;
  const float *q; int qstride; const float *qs; float scale;
  long long t_begin, t_end;    // token range (plane coordinates)
  float *part;                 // partial row of head 0 of the group
  long long part_head_stride;  // floats between consecutive heads' partials
};

template <class C>
__device__ void attend_range(const SplitIO &io, uint8_t *lds) {
  constexpr int HG = C::HG;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  uint8_t *vlds = lds;
  float *pdlds = reinterpret_cast<float *>(lds + C::LDS_V);
  float *wmax = reinterpret_cast<float *>(lds + C::LDS_MAIN);
  float *half = wmax + 4 * 8;
  float *sums = half + C::TT * 8;

  const int tt = tid % C::TT;          // token of this thread inside the tile (QK)
  const int part = tid / C::TT;
  const int gi = tid % C::NGV;         // PV: channel group and slot
  const int slot = tid / C::NGV;
  const int jv_g = (gi * 8) / C::LV;

  float m_run[HG], l_lane[HG], acc[HG][8];
  float pm[C::NBV][HG];
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    m_run[h] = NEG_INF;
    l_lane[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[h][k] = 0.f;
#pragma unroll
    for (int j = 0; j < C::NBV; ++j) pm[j][h] = 0.f;
  }

  for (long long t0 = io.t_begin; t0 < io.t_end; t0 += C::TT) {
    const long long t = t0 + tt;
    const bool valid = t < io.t_end;

    // ---- QK
    float s[HG];
    if (part == 0)
      qk_part<C, 0>(io.kcodes, io.ksc, io.kmn, t, valid, io.q, io.qstride, io.qs, s);
    else if constexpr (C::TPT > 1)
      qk_part<C, 1>(io.kcodes, io.ksc, io.kmn, t, valid, io.q, io.qstride, io.qs, s);
    if constexpr (C::TPT > 1) {
      if (part == 1) {
#pragma unroll
        for (int h = 0; h < HG; ++h) half[tt * 8 + h] = s[h];
      }
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int h = 0; h < HG; ++h) s[h] += half[tt * 8 + h];
      }
    }
    const bool owner = part == 0 && valid;
#pragma unroll
    for (int h = 0; h < HG; ++h) s[h] = owner ? s[h] * io.scale : NEG_INF;

    // ---- tile maximum
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      float mx = s[h];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      if (lane == 0) wmax[wave * 8 + h] = mx;
    }

    // ---- stage the V tile (raw codes) while the maxima settle
    {
      constexpr int NKV = C::RV / C::CV;
      constexpr int K0 = 0;
      const int kb = part * ((NKV + C::TPT - 1) / C::TPT);
      const int ke = (part + 1) * ((NKV + C::TPT - 1) / C::TPT) < NKV
                         ? (part + 1) * ((NKV + C::TPT - 1) / C::TPT) : NKV;
      (void)K0;
      uint8_t *row = vlds + tt * C::PITCH;
      for (int k = kb; k < ke; ++k) {
        const uint8_t *p = io.vcodes + tiled_offset(t, k, C::RV, C::CV);
        if constexpr (C::CV == 16) {
          uint4 v = valid ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
          *reinterpret_cast<uint4 *>(row + k * 16) = v;
        } else if constexpr (C::CV == 8) {
          uint2 v = valid ? *reinterpret_cast<const uint2 *>(p) : make_uint2(0, 0);
          *reinterpret_cast<uint2 *>(row + k * 8) = v;
        } else if constexpr (C::CV == 4) {
          *reinterpret_cast<uint32_t *>(row + k * 4) = valid ? *reinterpret_cast<const uint32_t *>(p) : 0u;
        } else if constexpr (C::CV == 2) {
          *reinterpret_cast<uint16_t *>(row + k * 2) = valid ? *reinterpret_cast<const uint16_t *>(p) : (uint16_t)0;
        } else {
          row[k] = valid ? *p : (uint8_t)0;
        }
      }
    }
    __syncthreads();

    float alpha[HG], mnew[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      float mx = fmaxf(fmaxf(wmax[h], wmax[8 + h]), fmaxf(wmax[16 + h], wmax[24 + h]));
      mnew[h] = fmaxf(m_run[h], mx);
      alpha[h] = (m_run[h] == NEG_INF) ? 0.f : exp2f(m_run[h] - mnew[h]);
      m_run[h] = mnew[h];
    }

    // ---- probabilities and p * d_j weights of the value blocks
    if (part == 0) {
      float dv[C::NBV], mv[C::NBV];
      if constexpr (C::VFAM == FAM_F16) {
        dv[0] = 1.f;
      } else {
        load_side<C::NBV>(io.vsc + t * C::NBV, valid, dv);
        if constexpr (C::VFAM == FAM_1) load_side<C::NBV>(io.vmn + t * C::NBV, valid, mv);
      }
      float p[HG];
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        p[h] = (s[h] == NEG_INF) ? 0.f : exp2f(s[h] - mnew[h]);
        l_lane[h] = fmaf(l_lane[h], alpha[h], p[h]);
      }
#pragma unroll
      for (int j = 0; j < C::NBV; ++j) {
        float *dst = pdlds + (tt * C::NBV + j) * C::HGP;
#pragma unroll
        for (int h = 0; h < HG; ++h) {
          dst[h] = valid ? p[h] * dv[j] : 0.f;
          if constexpr (C::VFAM == FAM_1) pm[j][h] = fmaf(pm[j][h], alpha[h], valid ? p[h] * mv[j] : 0.f);
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        l_lane[h] *= alpha[h];
#pragma unroll
        for (int j = 0; j < C::NBV; ++j) pm[j][h] *= alpha[h];
      }
    }
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[h][k] *= alpha[h];
    __syncthreads();

    // ---- PV: 8 channels of group gi, tokens slot, slot + NSLOT, ...
    for (int u = slot; u < C::TT; u += C::NSLOT) {
      const uint8_t *row = vlds + u * C::PITCH;
      float val[8];
      if constexpr (C::VFAM == FAM_F16) {
        const uint4 r = *reinterpret_cast<const uint4 *>(row + gi * 16);
        const uint32_t ww[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 8; ++k)
          val[k] = f16_bits_to_f32((uint16_t)((ww[k >> 1] >> (16 * (k & 1))) & 0xFFFFu));
      } else {
        constexpr int VB = C::VBITS;
        const int bit0 = gi * 8 * VB;
        const uint32_t *rw = reinterpret_cast<const uint32_t *>(row);
        const uint32_t lo = rw[bit0 >> 5];
        const uint32_t hi = rw[(bit0 >> 5) + 1];
        const int sh = bit0 & 31;
        uint32_t a[2];
        a[0] = sh ? ((lo >> sh) | (hi << (32 - sh))) : lo;
        a[1] = sh ? (hi >> sh) : hi;
#pragma unroll
        for (int k = 0; k < 8; ++k) val[k] = (float)field<VB, C::VFAM == FAM_0>(a, k * VB);
      }
      const float *pd = pdlds + (u * C::NBV + jv_g) * C::HGP;
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const float wgt = pd[h];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] = fmaf(wgt, val[k], acc[h][k]);
      }
    }
    __syncthreads();
  }

  // ---- close the split: l and pm summed over threads, acc over slots
  float *red = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    float l = l_lane[h];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (lane == 0) sums[wave * 64 + h] = l;
#pragma unroll
    for (int j = 0; j < C::NBV; ++j) {
      float v = pm[j][h];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      if (lane == 0) sums[wave * 64 + 8 + j * 8 + h] = v;
    }
  }
  for (int h = 0; h < HG; ++h) {
#pragma unroll
    for (int k = 0; k < 8; ++k) red[slot * (C::NV + 4) + gi * 8 + k] = acc[h][k];
    __syncthreads();
    float *dst = io.part + h * io.part_head_stride;
    for (int c = tid; c < C::NV; c += WG) {
      float o = 0.f;
      for (int sl = 0; sl < C::NSLOT; ++sl) o += red[sl * (C::NV + 4) + c];
      if constexpr (C::VFAM == FAM_1) {
        const int j = c / C::LV;
        o += sums[0 * 64 + 8 + j * 8 + h] + sums[1 * 64 + 8 + j * 8 + h] +
             sums[2 * 64 + 8 + j * 8 + h] + sums[3 * 64 + 8 + j * 8 + h];
      }
      dst[4 + c] = o;
    }
    if (tid == 0) {
      dst[0] = m_run[h];
      dst[1] = sums[h] + sums[64 + h] + sums[128 + h] + sums[192 + h];
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- kernels ----

__device__ inline void split_io_common(const DecodeArgs &a, int &b, int &kvh, int &hg, int &s) {
  int id = blockIdx.x;
  s = id % a.S_total;
  id /= a.S_total;
  hg = id % a.NHG;
  id /= a.NHG;
  kvh = id % a.Hkv;
  b = id / a.Hkv;
}

template <class C>
__device__ void run_body(const DecodeArgs &a, int b, int kvh, int hg, int s, uint8_t *lds) {
  const HeadGeom gk = head_geom(a.k, b, kvh), gv = head_geom(a.v, b, kvh);
  const int head0 = kvh * a.G + hg * C::HG;
  SplitIO io;
  io.kcodes = a.k.codes + gk.codes_off;
  io.ksc = a.k.scales ? a.k.scales + gk.scales_off : nullptr;
  io.kmn = a.k.mins ? a.k.mins + gk.scales_off : nullptr;
  io.vcodes = a.v.codes + gv.codes_off;
  io.vsc = a.v.scales ? a.v.scales + gv.scales_off : nullptr;
  io.vmn = a.v.mins ? a.v.mins + gv.scales_off : nullptr;
  io.q = a.q_body + ((long long)b * a.Hq + head0) * D;
  io.qstride = D;
  io.qs = a.qsum + ((long long)b * a.Hq + head0) * 4;
  io.scale = a.scale_body;
  const long long tpb = (long long)a.tps_body * C::TT;
  io.t_begin = (long long)s * tpb;
  io.t_end = io.t_begin + tpb < a.body_tokens ? io.t_begin + tpb : a.body_tokens;
  io.part = a.part + (((long long)b * a.Hq + head0) * a.S_total + s) * PSTRIDE;
  io.part_head_stride = (long long)a.S_total * PSTRIDE;
  attend_range<C>(io, lds);
}

template <int HG>
__device__ void run_tail(const DecodeArgs &a, int b, int kvh, int hg, int s, uint8_t *lds) {
  using C = Cfg<HG, KVQ_F16, KVQ_F16, D, D, 128>;
  const long long plane = (long long)b * a.Hkv + kvh;
  const int head0 = kvh * a.G + hg * HG;
  const int st = s - a.S_body;
  SplitIO io;
  io.kcodes = reinterpret_cast<const uint8_t *>(a.k.tail) + plane * a.k.tail_len * (2 * D);
  io.vcodes = reinterpret_cast<const uint8_t *>(a.v.tail) + plane * a.v.tail_len * (2 * D);
  io.ksc = io.kmn = io.vsc = io.vmn = nullptr;
  io.q = a.q_tail + ((long long)b * a.Hq + head0) * D;
  io.qstride = D;
  io.qs = nullptr;
  io.scale = a.scale_tail;
  const long long tps = (long long)a.tps_tail * C::TT;
  io.t_begin = (long long)st * tps;
  io.t_end = io.t_begin + tps < a.tail_tokens ? io.t_begin + tps : a.tail_tokens;
  io.part = a.part + (((long long)b * a.Hq + head0) * a.S_total + s) * PSTRIDE;
  io.part_head_stride = (long long)a.S_total * PSTRIDE;
  attend_range<C>(io, lds);
}

// Plain / KVarN body with fixed codecs + binary16 tail.
template <int HG, int KC, int VC>
__global__ __launch_bounds__(WG) void decode_kernel(DecodeArgs a) {
  using CB = Cfg<HG, KC, VC, D, D, tile_tokens_for(KC, VC)>;
  using CT = Cfg<HG, KVQ_F16, KVQ_F16, D, D, 128>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[cmax<CB::LDS_BYTES, CT::LDS_BYTES>::value];
  int b, kvh, hg, s;
  split_io_common(a, b, kvh, hg, s);
  if (s < a.S_body) run_body<CB>(a, b, kvh, hg, s, lds);
  else run_tail<HG>(a, b, kvh, hg, s, lds);
}

// Low-rank body: per-head (codec, rank) chosen at run time among the
// supported set; + binary16 tail.
#define KVQ_LR_CASES(X)                                                                  \
  X(KVQ_Q1_1, 16) X(KVQ_Q1_1, 32) X(KVQ_Q1_1, 64) X(KVQ_Q1_1, 128)                       \
  X(KVQ_Q2_1, 16) X(KVQ_Q2_1, 32) X(KVQ_Q2_1, 64) X(KVQ_Q2_1, 128)                       \
  X(KVQ_Q3_1, 16) X(KVQ_Q3_1, 32) X(KVQ_Q3_1, 64) X(KVQ_Q3_1, 128)                       \
  X(KVQ_Q4_1, 16) X(KVQ_Q4_1, 32) X(KVQ_Q4_1, 64) X(KVQ_Q4_1, 128)

template <int HG>
struct LrLds {
  static constexpr int bytes = cmax<cmax<Cfg<HG, KVQ_Q4_1, KVQ_Q4_1, 128, 128, 256>::LDS_BYTES,
                                         Cfg<HG, KVQ_Q3_1, KVQ_Q3_1, 128, 128, 256>::LDS_BYTES>::value,
                                    Cfg<HG, KVQ_F16, KVQ_F16, D, D, 128>::LDS_BYTES>::value;
};

template <int HG>
__global__ __launch_bounds__(WG) void decode_lowrank_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LrLds<HG>::bytes];
  int b, kvh, hg, s;
  split_io_common(a, b, kvh, hg, s);
  if (s >= a.S_body) {
    run_tail<HG>(a, b, kvh, hg, s, lds);
    return;
  }
  const int codec = a.k.hcodec[kvh], rank = a.k.hrank[kvh];
#define KVQ_LR_DISPATCH(CC, RR)                                                           \
  if (codec == CC && rank == RR) {                                                        \
    run_body<Cfg<HG, CC, CC, RR, RR, 256>>(a, b, kvh, hg, s, lds);                        \
    return;                                                                               \
  }
  KVQ_LR_CASES(KVQ_LR_DISPATCH)
#undef KVQ_LR_DISPATCH
}

inline bool decode_lowrank_supported_impl(int codec, int rank) {
#define KVQ_LR_CHECK(CC, RR) if (codec == CC && rank == RR) return true;
  KVQ_LR_CASES(KVQ_LR_CHECK)
#undef KVQ_LR_CHECK
  return false;
}


// (K codec, V codec) pairs with a compiled decode path, per head group.
#define KVQ_DECODE_PAIRS(X)                                                                \
  X(KVQ_F16, KVQ_F16) X(KVQ_Q8_0, KVQ_Q8_0) X(KVQ_Q6_0, KVQ_Q6_0) X(KVQ_Q5_0, KVQ_Q5_0)    \
  X(KVQ_Q4_0, KVQ_Q4_0) X(KVQ_Q3_0, KVQ_Q3_0) X(KVQ_Q2_0, KVQ_Q2_0) X(KVQ_Q8_1, KVQ_Q8_1)  \
  X(KVQ_Q6_1, KVQ_Q6_1) X(KVQ_Q5_1, KVQ_Q5_1) X(KVQ_Q4_1, KVQ_Q4_1) X(KVQ_Q3_1, KVQ_Q3_1)  \
  X(KVQ_Q2_1, KVQ_Q2_1) X(KVQ_Q1_1, KVQ_Q1_1) X(KVQ_Q8_0, KVQ_Q4_0) X(KVQ_Q8_0, KVQ_Q3_0)  \
  X(KVQ_Q8_0, KVQ_Q2_0) X(KVQ_Q6_0, KVQ_Q4_0) X(KVQ_Q4_0, KVQ_Q2_0) X(KVQ_Q8_1, KVQ_Q4_1)  \
  X(KVQ_F16, KVQ_Q8_0) X(KVQ_F16, KVQ_Q4_0)

template <int HG>
hipError_t launch_decode_hg(const DecodeArgs &a, dim3 grid, hipStream_t st) {
  if (a.k.basis == KVQ_BASIS_LOWRANK) {
    hipLaunchKernelGGL(decode_lowrank_kernel<HG>, grid, dim3(WG), 0, st, a);
    return hipGetLastError();
  }
  const int kc = a.k.codec, vc = a.v.codec;
#define KVQ_LAUNCH_PAIR(K, V)                                                               \
  if (kc == K && vc == V) {                                                                 \
    hipLaunchKernelGGL((decode_kernel<HG, K, V>), grid, dim3(WG), 0, st, a);                \
    return hipGetLastError();                                                               \
  }
  KVQ_DECODE_PAIRS(KVQ_LAUNCH_PAIR)
#undef KVQ_LAUNCH_PAIR
  return hipErrorNotSupported;
}

}  // namespace kvq
