// Device implementation of the split-K decode kernel (design notes in
// kvq_decode.hip).  Included by the per-head-group instantiation units.
//
// Work decomposition: a 256-thread workgroup owns one context split of one
// (batch entry, kv head, group of HG <= 8 query heads).  Its four waves are
// independent flash-decoders: each walks its own 64-token tiles of the split
// with its own running max, sum and output accumulators, so the main loop
// has no workgroup barrier.  The four wave states are merged through LDS
// once, at the end of the split.
//
// Per 64-token tile, one wave does:
//   QK on the matrix cores: v_mfma_f32_16x16x32_f16 with the query as the A
//     operand (rows = query heads) and 16 tokens x 32 channels of codes as
//     the B operand.  Codes are small integers, exact in binary16; the
//     binary32 query is split into hi + lo binary16 parts (two MFMAs into
//     one accumulator), after a per-head power-of-two rescale, which keeps
//     ~22 significant bits.  Block scales are applied to the fp32 results:
//     s = sum_j d_j * C_j (+ m_j * sum(q over block j) for _1 codes).
//   Online softmax in the log2 domain (DPP row reductions).
//   PV on the vector units: value rows are staged raw in LDS with the
//     p * d_j weights; lane (slot, group) owns 8 output channels.
// The next tile's code loads are issued while the current tile is still
// being computed (one tile of register prefetch).
#pragma once

#include "kvq_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {

constexpr int WG = 256;
constexpr int NWAVE = WG / 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_huge_valf();

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

template <int A, int B> struct cmax { static constexpr int value = A > B ? A : B; };

union H8 {
  half8 h;
  uint32_t u[4];
};

// ------------------------------------------------------------ DPP helpers --

// All-reduce over the 16 lanes of a DPP row (lanes 16r .. 16r+15).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xF, 0xF, false)));
  return x;
}

__device__ __forceinline__ float row_sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ float read_lane(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

// Per-token binary16 side values (scales or mins) of NB blocks.
template <int NB>
__device__ __forceinline__ void load_side(const uint16_t *__restrict__ p, bool valid,
                                          float (&v)[NB > 0 ? NB : 1]) {
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

template <int HG_, int KC_, int VC_, int NK_, int NV_>
struct Cfg {
  static constexpr int HG = HG_, KC = KC_, VC = VC_, NK = NK_, NV = NV_;
  static constexpr int KBITS = codec_bits(KC), KFAM = codec_family(KC);
  static constexpr int VBITS = codec_bits(VC), VFAM = codec_family(VC);
  static constexpr int RK = row_bytes(KC, NK), CK = chunk_bytes(RK);
  static constexpr int RV = row_bytes(VC, NV), CV = chunk_bytes(RV);
  static constexpr int NKB = NK < 32 ? 1 : NK / 32;          // 32-channel MFMA k-blocks
  static constexpr int NBK = KFAM == FAM_F16 ? 0 : NK / block_len(NK);
  static constexpr int LV = VFAM == FAM_F16 ? NV : block_len(NV);
  static constexpr int NBV = VFAM == FAM_F16 ? 1 : NV / LV;
  static constexpr int NGRP = (HG + 3) / 4;                  // 16-lane row groups with heads
  static constexpr int HGP = (HG + 3) / 4 * 4;
  static constexpr int PITCH = ((RV + 15) / 16) * 16 + 16;   // LDS row pitch of V
  static constexpr int NGV = NV / 8;                         // 8-channel groups of PV
  static constexpr int NSLOT = 64 / NGV;
  // LDS per wave: V rows, p*d weights, per-head query scalars
  static constexpr int W_V = 64 * PITCH;
  static constexpr int W_PD = 64 * NBV * HGP * 4;
  static constexpr int W_Q = 8 * 4 + 8 * 4 * 4;              // inverse scales, block sums
  static constexpr int W_BYTES = (W_V + W_PD + W_Q + 15) / 16 * 16;
  static constexpr int MERGE = NWAVE * HG * (NV + 4) * 4;
  static constexpr int LDS_BYTES = cmax<NWAVE * W_BYTES, MERGE>::value;
};

// ------------------------------------------------ QK operand preparation --

// Raw codes of (k-block j, k-group kg) of one token: the 8 channels
// 32j + 8kg .. +7 of its row.  f16 rows give 8 binary16 values (16 bytes).
template <class C>
struct KRaw {
  uint32_t u[C::KFAM == FAM_F16 ? 4 : 2];
};

template <class C>
__device__ __forceinline__ void k_load(const uint8_t *__restrict__ plane, long long t, int j,
                                       int kg, bool valid, KRaw<C> &r) {
  constexpr int b = C::KBITS, R = C::RK, CC = C::CK;
  const int e0 = 32 * j + 8 * kg;
  const bool in = valid && e0 < C::NK;
  if constexpr (C::KFAM == FAM_F16) {
    const int byte = 2 * e0;
    if (in) {
      const uint4 v = *reinterpret_cast<const uint4 *>(plane + tiled_offset(t, byte / CC, R, CC) + byte % CC);
      r.u[0] = v.x; r.u[1] = v.y; r.u[2] = v.z; r.u[3] = v.w;
    } else {
      r.u[0] = r.u[1] = r.u[2] = r.u[3] = 0u;
    }
  } else if constexpr (b == 8) {
    const int byte = e0;
    if (in) {
      const uint2 v = *reinterpret_cast<const uint2 *>(plane + tiled_offset(t, byte / CC, R, CC) + byte % CC);
      r.u[0] = v.x; r.u[1] = v.y;
    } else {
      r.u[0] = r.u[1] = 0u;
    }
  } else if constexpr (b == 4) {
    const int byte = e0 / 2;
    r.u[0] = in ? *reinterpret_cast<const uint32_t *>(plane + tiled_offset(t, byte / CC, R, CC) + byte % CC) : 0u;
    r.u[1] = 0u;
  } else if constexpr (b == 2) {
    const int byte = e0 / 4;
    r.u[0] = in ? (uint32_t)*reinterpret_cast<const uint16_t *>(plane + tiled_offset(t, byte / CC, R, CC) + byte % CC) : 0u;
    r.u[1] = 0u;
  } else if constexpr (b == 1) {
    const int byte = e0 / 8;
    r.u[0] = in ? (uint32_t)plane[tiled_offset(t, byte / CC, R, CC) + byte % CC] : 0u;
    r.u[1] = 0u;
  } else {
    // 3, 5, 6 bits: 8 codes are `b` whole bytes starting at byte e0*b/8
    uint64_t w = 0;
    if (in) {
      const int byte0 = e0 * b / 8;
#pragma unroll
      for (int i = 0; i < b; ++i) {
        const int byte = byte0 + i;
        w |= (uint64_t)plane[tiled_offset(t, byte / CC, R, CC) + byte % CC] << (8 * i);
      }
    }
    r.u[0] = (uint32_t)w;
    r.u[1] = (uint32_t)(w >> 32);
  }
}

// Exact binary16 values of the 8 codes (signed for _0, unsigned for _1).
template <class C>
__device__ __forceinline__ half8 k_convert(const KRaw<C> &r) {
  constexpr int b = C::KBITS;
  H8 o;
  if constexpr (C::KFAM == FAM_F16) {
    o.u[0] = r.u[0]; o.u[1] = r.u[1]; o.u[2] = r.u[2]; o.u[3] = r.u[3];
    return o.h;
  } else {
    // each code becomes u = code + off in [0, 2^b), binary16 1024 + u is
    // built from its bits (0x6400 | u), then 1024 + off is subtracted exactly
    constexpr uint32_t off = C::KFAM == FAM_0 ? (1u << (b - 1)) : 0u;
    const _Float16 bias = (_Float16)(-(1024.f + (float)off));
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    const half2v bias2 = {bias, bias};
    if constexpr (b == 8) {
      const uint32_t x0 = r.u[0] ^ (C::KFAM == FAM_0 ? 0x80808080u : 0u);
      const uint32_t x1 = r.u[1] ^ (C::KFAM == FAM_0 ? 0x80808080u : 0u);
      const uint32_t c64 = 0x64646464u;
      o.u[0] = __builtin_amdgcn_perm(c64, x0, 0x04010400u);
      o.u[1] = __builtin_amdgcn_perm(c64, x0, 0x04030402u);
      o.u[2] = __builtin_amdgcn_perm(c64, x1, 0x04010400u);
      o.u[3] = __builtin_amdgcn_perm(c64, x1, 0x04030402u);
    } else if constexpr (b == 4) {
      const uint32_t x = r.u[0] ^ (C::KFAM == FAM_0 ? 0x88888888u : 0u);
      const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
      o.u[0] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x64006400u;
      o.u[1] = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x64006400u;
      o.u[2] = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x64006400u;
      o.u[3] = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x64006400u;
    } else {
      const uint64_t w = (uint64_t)r.u[0] | ((uint64_t)r.u[1] << 32);
      constexpr uint32_t m = (1u << b) - 1u;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t u0 = ((uint32_t)(w >> (2 * p * b)) + off) & m;
        const uint32_t u1 = ((uint32_t)(w >> ((2 * p + 1) * b)) + off) & m;
        o.u[p] = (u0 | (u1 << 16)) | 0x64006400u;
      }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      half2v v = __builtin_bit_cast(half2v, o.u[p]);
      v = v + bias2;
      o.u[p] = __builtin_bit_cast(uint32_t, v);
    }
    return o.h;
  }
}

// ------------------------------------------------------- one split range --

struct SplitIO {
  const uint8_t *kcodes; const uint16_t *ksc; const uint16_t *kmn;
  const uint8_t *vcodes; const uint16_t *vsc; const uint16_t *vmn;
  const float *q;              // HG query rows (stride 128), raw binary32
  float scale;                 // multiplier into the log2 domain
  long long t_begin, t_end;    // token range (plane coordinates), t_begin % 64 == 0
  float *part;                 // partial row of head 0 of the group
  long long part_head_stride;  // floats between consecutive heads' partials
};

template <class C>
__device__ void attend_range(const SplitIO &io, uint8_t *lds) {
  constexpr int HG = C::HG;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  uint8_t *wl = lds + wave * C::W_BYTES;
  uint8_t *vlds = wl;
  float *pdlds = reinterpret_cast<float *>(wl + C::W_V);
  float *qinv = reinterpret_cast<float *>(wl + C::W_V + C::W_PD);   // [8]
  float *qsum = qinv + 8;                                            // [8][4]

  const int n = lane & 15, g = lane >> 4;   // QK layout: token column, row group
  const int gi = lane % C::NGV, slot = lane / C::NGV;   // PV layout
  const int jv_g = (gi * 8) / C::LV;

  // ---- query operands: row i = lane % 16 is head i (< HG), k-group = lane / 16
  half8 qa_hi[C::NKB], qa_lo[C::NKB];
  {
    const int i = n, kg = g;
    float v[C::NKB][8];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < C::NKB; ++j) {
      const int e0 = 32 * j + 8 * kg;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = i < HG && e0 + e < C::NK;
        v[j][e] = ok ? io.q[i * D + e0 + e] * io.scale : 0.f;
        amax = fmaxf(amax, fabsf(v[j][e]));
      }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    int ex = 0;
    if (amax > 0.f) (void)frexpf(amax, &ex);
    const int sh = 14 - ex;                       // |q * 2^sh| < 2^14
    const float up = ldexpf(1.f, sh);
#pragma unroll
    for (int j = 0; j < C::NKB; ++j) {
      H8 hi, lo;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = v[j][e] * up;
        const _Float16 h = (_Float16)x;
        hi.h[e] = h;
        lo.h[e] = (_Float16)(x - (float)h);
        s += v[j][e];
      }
      qa_hi[j] = hi.h;
      qa_lo[j] = lo.h;
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (g == 0 && i < HG && C::KFAM == FAM_1) qsum[i * 4 + j] = s;
    }
    if (g == 0 && i < HG) qinv[i] = ldexpf(1.f, -sh);
  }
  wave_sync_lds();

  // per-lane copies for the QK layout (heads 4g + r)
  float inv_r[4], qs_r[4][C::NKB];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g + r;
    inv_r[r] = h < HG ? qinv[h] : 0.f;
#pragma unroll
    for (int j = 0; j < C::NKB; ++j) qs_r[r][j] = (C::KFAM == FAM_1 && h < HG) ? qsum[h * 4 + j] : 0.f;
  }

  float m_run[4], l_lane[4];
  float acc[HG][8];
  float pm[C::NBV][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = NEG_INF;
    l_lane[r] = 0.f;
#pragma unroll
    for (int j = 0; j < C::NBV; ++j) pm[j][r] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[h][k] = 0.f;

  // this wave's tiles: t_begin + 64 * (wave + NWAVE * i)
  const long long first = io.t_begin + 64LL * wave;
  const long long stride = 64LL * NWAVE;

  // One full tile of register prefetch: while tile i is computed, every
  // load of tile i+1 is in flight (K operands and scales of its 4 N-tiles,
  // the lane's V row and the V scales its p*d weights need).
  KRaw<C> kr[4][C::NKB];
  uint2 ksr[4], kmr[4], vsr[4], vmr[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) ksr[nt] = kmr[nt] = vsr[nt] = vmr[nt] = make_uint2(0u, 0u);
  constexpr int NVCH = C::RV / C::CV;
  constexpr int NVW = (C::RV + 3) / 4;
  uint32_t vw[NVW];

  auto side_raw = [&](const uint16_t *base, long long t, bool valid, int nb) -> uint2 {
    if (!valid) return make_uint2(0u, 0u);
    const uint16_t *p = base + t * nb;
    if (nb == 4) return *reinterpret_cast<const uint2 *>(p);
    if (nb == 2) return make_uint2(*reinterpret_cast<const uint32_t *>(p), 0u);
    return make_uint2((uint32_t)*p, 0u);
  };
  auto load_k_nt = [&](long long t0, int nt) {
    const long long t = t0 + 16 * nt + n;
    const bool valid = t < io.t_end;
#pragma unroll
    for (int j = 0; j < C::NKB; ++j) k_load<C>(io.kcodes, t, j, g, valid, kr[nt][j]);
    if constexpr (C::KFAM != FAM_F16) ksr[nt] = side_raw(io.ksc, t, valid, C::NBK);
    if constexpr (C::KFAM == FAM_1) kmr[nt] = side_raw(io.kmn, t, valid, C::NBK);
  };
  auto load_v = [&](long long t0) {
    const long long t = t0 + lane;
    const bool valid = t < io.t_end;
#pragma unroll
    for (int k = 0; k < NVW; ++k) vw[k] = 0u;
    if (valid) {
#pragma unroll
      for (int k = 0; k < NVCH; ++k) {
        const uint8_t *p = io.vcodes + tiled_offset(t, k, C::RV, C::CV);
        if constexpr (C::CV == 16) {
          const uint4 v = *reinterpret_cast<const uint4 *>(p);
          vw[4 * k] = v.x; vw[4 * k + 1] = v.y; vw[4 * k + 2] = v.z; vw[4 * k + 3] = v.w;
        } else if constexpr (C::CV == 8) {
          const uint2 v = *reinterpret_cast<const uint2 *>(p);
          vw[2 * k] = v.x; vw[2 * k + 1] = v.y;
        } else if constexpr (C::CV == 4) {
          vw[k] = *reinterpret_cast<const uint32_t *>(p);
        } else if constexpr (C::CV == 2) {
          vw[k / 2] |= (uint32_t)(*reinterpret_cast<const uint16_t *>(p)) << (16 * (k & 1));
        } else {
          vw[k / 4] |= (uint32_t)(*p) << (8 * (k & 3));
        }
      }
    }
    if constexpr (C::VFAM != FAM_F16) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const long long tv = t0 + 16 * nt + n;
        const bool ok = tv < io.t_end;
        vsr[nt] = side_raw(io.vsc, tv, ok, C::NBV);
        if constexpr (C::VFAM == FAM_1) vmr[nt] = side_raw(io.vmn, tv, ok, C::NBV);
      }
    }
  };
  auto unpack_side = [&](uint2 r, float *v, int nb) {
    v[0] = f16_bits_to_f32(r.x & 0xFFFF);
    if (nb > 1) v[1] = f16_bits_to_f32(r.x >> 16);
    if (nb > 2) { v[2] = f16_bits_to_f32(r.y & 0xFFFF); v[3] = f16_bits_to_f32(r.y >> 16); }
  };

  if (first < io.t_end) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) load_k_nt(first, nt);
    load_v(first);
  }

  for (long long t0 = first; t0 < io.t_end; t0 += stride) {
    const long long tn = t0 + stride;
    const bool more = tn < io.t_end;
    // ---- QK: 4 N-tiles of 16 tokens
    float s[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      half8 kb[C::NKB];
#pragma unroll
      for (int j = 0; j < C::NKB; ++j) kb[j] = k_convert<C>(kr[nt][j]);
      float dk[4] = {1.f, 1.f, 1.f, 1.f}, mk[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (C::KFAM != FAM_F16) unpack_side(ksr[nt], dk, C::NBK);
      if constexpr (C::KFAM == FAM_1) unpack_side(kmr[nt], mk, C::NBK);
      if (more) load_k_nt(tn, nt);      // registers of N-tile nt are free again

      const long long t = t0 + 16 * nt + n;
      const bool valid = t < io.t_end;
      float sc[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (C::KFAM == FAM_F16) {
        floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < C::NKB; ++j) {
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[j], kb[j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[j], kb[j], c, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = c[r] * inv_r[r];
      } else {
#pragma unroll
        for (int j = 0; j < C::NKB; ++j) {
          floatx4 c = {0.f, 0.f, 0.f, 0.f};
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[j], kb[j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[j], kb[j], c, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sc[r] = fmaf(dk[j], c[r] * inv_r[r], sc[r]);
            if constexpr (C::KFAM == FAM_1) sc[r] = fmaf(mk[j], qs_r[r][j], sc[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[nt][r] = (valid && 4 * g + r < HG) ? sc[r] : NEG_INF;
    }

    // ---- online softmax (per wave; heads 4g + r live in row group g)
    float alpha[4], mnew[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mx = fmaxf(fmaxf(s[0][r], s[1][r]), fmaxf(s[2][r], s[3][r]));
      mx = row_max16(mx);
      mnew[r] = fmaxf(m_run[r], mx);
      alpha[r] = (mnew[r] == NEG_INF) ? 1.f : exp2f(m_run[r] - mnew[r]);
      m_run[r] = mnew[r];
    }

    // ---- stage this tile's V row, then p * d_j weights
    {
      uint8_t *row = vlds + lane * C::PITCH;
#pragma unroll
      for (int k = 0; k < NVW; k += 4) {
        if (k + 3 < NVW) {
          *reinterpret_cast<uint4 *>(row + 4 * k) = make_uint4(vw[k], vw[k + 1], vw[k + 2], vw[k + 3]);
        } else {
#pragma unroll
          for (int kk = k; kk < NVW; ++kk) *reinterpret_cast<uint32_t *>(row + 4 * kk) = vw[kk];
        }
      }
    }
    uint2 vsc_cur[4], vmn_cur[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      vsc_cur[nt] = vsr[nt];
      vmn_cur[nt] = vmr[nt];
    }
    if (more) load_v(tn);               // V registers are free again

#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const long long t = t0 + 16 * nt + n;
      const bool valid = t < io.t_end;
      float dvs[4] = {1.f, 1.f, 1.f, 1.f}, mvs[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (C::VFAM != FAM_F16) unpack_side(vsc_cur[nt], dvs, C::NBV);
      if constexpr (C::VFAM == FAM_1) unpack_side(vmn_cur[nt], mvs, C::NBV);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (s[nt][r] == NEG_INF) ? 0.f : exp2f(s[nt][r] - mnew[r]);
        l_lane[r] = (nt == 0 ? l_lane[r] * alpha[r] : l_lane[r]) + p[r];
      }
      if (g < C::NGRP) {
#pragma unroll
        for (int j = 0; j < C::NBV; ++j) {
          float *dst = pdlds + ((16 * nt + n) * C::NBV + j) * C::HGP + 4 * g;
          float4 wv;
          wv.x = valid ? p[0] * dvs[j] : 0.f;
          wv.y = valid ? p[1] * dvs[j] : 0.f;
          wv.z = valid ? p[2] * dvs[j] : 0.f;
          wv.w = valid ? p[3] * dvs[j] : 0.f;
          *reinterpret_cast<float4 *>(dst) = wv;
          if constexpr (C::VFAM == FAM_1) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              pm[j][r] = (nt == 0 ? pm[j][r] * alpha[r] : pm[j][r]) + (valid ? p[r] * mvs[j] : 0.f);
          }
        }
      }
    }

    // accumulators of head h are rescaled by that head's alpha (from its row group)
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float a = read_lane(alpha[h & 3], 16 * (h >> 2));
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[h][k] *= a;
    }
    wave_sync_lds();

    // ---- PV: channels 8*gi .. 8*gi+7 over tokens slot, slot + NSLOT, ...
#pragma unroll 4
    for (int u = slot; u < 64; u += C::NSLOT) {
      const uint8_t *row = vlds + u * C::PITCH;
      float val[8];
      if constexpr (C::VFAM == FAM_F16) {
        const uint4 rr = *reinterpret_cast<const uint4 *>(row + gi * 16);
        const uint32_t ww[4] = {rr.x, rr.y, rr.z, rr.w};
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
        uint32_t a2[2];
        a2[0] = sh ? ((lo >> sh) | (hi << (32 - sh))) : lo;
        a2[1] = sh ? (hi >> sh) : hi;
#pragma unroll
        for (int k = 0; k < 8; ++k) val[k] = (float)field<VB, C::VFAM == FAM_0>(a2, k * VB);
      }
      const float *pd = pdlds + (u * C::NBV + jv_g) * C::HGP;
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const float wgt = pd[h];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] = fmaf(wgt, val[k], acc[h][k]);
      }
    }
    wave_sync_lds();
  }

  // ---- close this wave: sums over the row's 16 lanes, accumulators over slots
  float lsum[4], pmsum[C::NBV][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    lsum[r] = row_sum16(l_lane[r]);
#pragma unroll
    for (int j = 0; j < C::NBV; ++j) pmsum[j][r] = C::VFAM == FAM_1 ? row_sum16(pm[j][r]) : 0.f;
  }
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float v = acc[h][k];
#pragma unroll
      for (int o = C::NGV; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      acc[h][k] = v;
    }
  __syncthreads();   // every wave is done with its LDS tiles

  // merge area: [wave][h][4 + NV]: m, l, -, -, o[NV]
  float *mg = reinterpret_cast<float *>(lds);
  constexpr int MS = C::NV + 4;
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    const int r = h & 3, grp = h >> 2;
    float *dst = mg + (wave * HG + h) * MS;
    if (lane == 16 * grp) {
      dst[0] = m_run[r];
      dst[1] = lsum[r];
    }
    float pmh = 0.f;   // min term of this lane's value block, head h
    if constexpr (C::VFAM == FAM_1) {
#pragma unroll
      for (int j = 0; j < C::NBV; ++j) {
        const float v = read_lane(pmsum[j][r], 16 * grp);
        pmh = (j == jv_g) ? v : pmh;
      }
    }
    if (slot == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[4 + gi * 8 + k] = acc[h][k] + pmh;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < HG * C::NV; idx += WG) {
    const int h = idx / C::NV, c = idx % C::NV;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, mg[(w * HG + h) * MS]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      const float *src = mg + (w * HG + h) * MS;
      const float wt = src[0] == NEG_INF ? 0.f : exp2f(src[0] - M);
      o = fmaf(wt, src[4 + c], o);
      L = fmaf(wt, src[1], L);
    }
    float *dst = io.part + h * io.part_head_stride;
    dst[4 + c] = o;
    if (c == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// ------------------------------------------------------------- kernels ----

__device__ inline void split_io_common(const DecodeArgs &a, int &b, int &kvh, int &hg, int &s) {
  int id = blockIdx.x;
  s = id % a.S_body;
  id /= a.S_body;
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
  io.scale = a.scale_body;
  const long long tps = (long long)a.tps_body * 64;
  io.t_begin = (long long)s * tps;
  io.t_end = io.t_begin + tps < a.body_tokens ? io.t_begin + tps : a.body_tokens;
  io.part = a.part + (((long long)b * a.Hq + head0) * a.S_total + s) * PSTRIDE;
  io.part_head_stride = (long long)a.S_total * PSTRIDE;
  attend_range<C>(io, lds);
}

template <int HG>
__device__ void run_tail(const DecodeArgs &a, int b, int kvh, int hg, int s, uint8_t *lds) {
  using C = Cfg<HG, KVQ_F16, KVQ_F16, D, D>;
  const long long plane = (long long)b * a.Hkv + kvh;
  const int head0 = kvh * a.G + hg * HG;
  const int st = s - a.S_body;
  SplitIO io;
  io.kcodes = reinterpret_cast<const uint8_t *>(a.k.tail) + plane * a.k.tail_len * (2 * D);
  io.vcodes = reinterpret_cast<const uint8_t *>(a.v.tail) + plane * a.v.tail_len * (2 * D);
  io.ksc = io.kmn = io.vsc = io.vmn = nullptr;
  io.q = a.q_tail + ((long long)b * a.Hq + head0) * D;
  io.scale = a.scale_tail;
  const long long tps = (long long)a.tps_tail * 64;
  io.t_begin = (long long)st * tps;
  io.t_end = io.t_begin + tps < a.tail_tokens ? io.t_begin + tps : a.tail_tokens;
  io.part = a.part + (((long long)b * a.Hq + head0) * a.S_total + s) * PSTRIDE;
  io.part_head_stride = (long long)a.S_total * PSTRIDE;
  attend_range<C>(io, lds);
}

// Occupancy targets (waves per SIMD) of the kernels: the register budget
// is 512 / target per lane.
template <int KC, int VC> struct Occ { static constexpr int value = (KC == KVQ_F16 || VC == KVQ_F16) ? 2 : 2; };

// Plain / KVarN body splits with fixed codecs.
template <int HG, int KC, int VC>
__global__ __launch_bounds__(WG, (Occ<KC, VC>::value)) void decode_kernel(DecodeArgs a) {
  using CB = Cfg<HG, KC, VC, D, D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[CB::LDS_BYTES];
  int b, kvh, hg, s;
  split_io_common(a, b, kvh, hg, s);
  run_body<CB>(a, b, kvh, hg, s, lds);
}

// Binary16 precision-tail splits (raw basis); blockIdx enumerates
// (b, kv head, head group, tail split) and the partial lands at split
// index S_body + tail split.
template <int HG>
__global__ __launch_bounds__(WG, 2) void decode_tail_kernel(DecodeArgs a) {
  using CT = Cfg<HG, KVQ_F16, KVQ_F16, D, D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[CT::LDS_BYTES];
  int id = blockIdx.x;
  const int st = id % a.S_tail;
  id /= a.S_tail;
  const int hg = id % a.NHG;
  id /= a.NHG;
  const int kvh = id % a.Hkv;
  const int b = id / a.Hkv;
  run_tail<HG>(a, b, kvh, hg, a.S_body + st, lds);
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
  static constexpr int bytes = cmax<Cfg<HG, KVQ_Q4_1, KVQ_Q4_1, 128, 128>::LDS_BYTES,
                                    Cfg<HG, KVQ_Q3_1, KVQ_Q3_1, 128, 128>::LDS_BYTES>::value;
};

template <int HG>
__global__ __launch_bounds__(WG, 2) void decode_lowrank_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LrLds<HG>::bytes];
  int b, kvh, hg, s;
  split_io_common(a, b, kvh, hg, s);
  const int codec = a.k.hcodec[kvh], rank = a.k.hrank[kvh];
#define KVQ_LR_DISPATCH(CC, RR)                                                           \
  if (codec == CC && rank == RR) {                                                        \
    run_body<Cfg<HG, CC, CC, RR, RR>>(a, b, kvh, hg, s, lds);                             \
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
hipError_t launch_decode_hg(const DecodeArgs &a, hipStream_t st) {
  const long long units = (long long)a.B * a.Hkv * a.NHG;
  if (a.S_tail > 0) {
    hipLaunchKernelGGL(decode_tail_kernel<HG>, dim3((unsigned)(units * a.S_tail)), dim3(WG), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.S_body == 0) return hipSuccess;
  const dim3 grid((unsigned)(units * a.S_body));
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
