// Device implementation of the split-K decode kernel.  Included by the
// per-head-group instantiation units.
//
// Work decomposition: a workgroup of NWAVE waves owns one context split of
// one (batch entry, kv head, group of HG <= 8 query heads).  Its waves are
// independent flash-decoders: each walks its own 64-token tiles of the split
// with its own running max, sum and output accumulators, so the main loop
// has no workgroup barrier.  The wave states are merged through LDS once, at
// the end of the split, and the split's partial is stored for the unit's
// final merge (combine_head, run by the unit's last workgroup).
//
// Quantised bodies run attend_q (kvq_decode_q.hpp: QK on the integer matrix
// cores, PV on binary16 MFMA).  The binary16 precision tail and F16 codecs
// run attend_range below: QK on v_mfma_f32_16x16x32_f16 with the query split
// into hi + lo binary16 parts (rows (head, part)), online softmax in the
// log2 domain with DPP row reductions, PV on the matrix cores with the
// weights staged in LDS and read back transposed.
#pragma once

#include <hip/hip_ext.h>
#include "kvq_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
#include "kvq_append_row.hpp"
}

namespace kvq {

constexpr int NWAVE = DECODE_WG_WAVES;
// Splits with at least this many tiles per wave hand tiles out at run time
// (the second wave of each SIMD gets its first tile several microseconds
// after the first; with a few tiles per wave a static round-robin is as
// fast and keeps the result independent of timing).
constexpr int DYN_TILES_PER_WAVE = 4;
constexpr int WG = 64 * NWAVE;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_huge_valf();

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

template <int A, int B> struct cmax { static constexpr int value = A > B ? A : B; };

union H8 {
  half8 h;
  uint32_t u[4];
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 16 x 16 x 32 MFMA step on 16-bit operands: binary16, or bfloat16 (BF) with
// the same bits carried in the half8 registers.
template <bool BF>
__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// x as a (hi, lo) pair of 16-bit values (hi = RN(x), lo = RN(x - hi)) packed
// hi | lo << 16: binary16, or bfloat16 (BF).
template <bool BF>
__device__ __forceinline__ uint32_t split16(float x) {
  if constexpr (BF) {
    const uint16_t hi = f32_to_bf16_bits(x);
    const uint16_t lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
    return (uint32_t)hi | ((uint32_t)lo << 16);
  } else {
    const _Float16 hi = (_Float16)x;
    const _Float16 lo = (_Float16)(x - (float)hi);
    return (uint32_t)__builtin_bit_cast(uint16_t, hi) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
  }
}

// ------------------------------------------------------------ DPP helpers --

// All-reduce over the 16 lanes of a DPP row (lanes 16r .. 16r+15).  Row
// rotations read only lanes of the same row; bound_ctrl only replaces the
// zero `old` operand, so the values are those of a plain rotation.  The max
// is IEEE maximum (NaN-propagating): no operand canonicalisation, and the
// same value as maxNum for the scores and exponents it sees (no NaN).
#define KVQ_ROR(x, ctrl) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xF, 0xF, true))
__device__ __forceinline__ float row_max16(float x) {
  x = __builtin_elementwise_maximum(x, KVQ_ROR(x, 0x128));
  x = __builtin_elementwise_maximum(x, KVQ_ROR(x, 0x124));
  x = __builtin_elementwise_maximum(x, KVQ_ROR(x, 0x122));
  x = __builtin_elementwise_maximum(x, KVQ_ROR(x, 0x121));
  return x;
}

__device__ __forceinline__ float row_sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xF, 0xF, true));
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

// -------------------------------------------- cross-workgroup exchange --
// Split partials travel between workgroups that may sit on different XCDs
// (each with its own L2) within one launch.  They are written and read with
// device-scope relaxed atomics, which the compiler emits as L2-coherent
// accesses (sc1), so no L2 write-back or invalidate is needed; ordering is
// by waiting for the stores to complete before the completion counter.
__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned *>(p), __builtin_bit_cast(unsigned, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<const unsigned *>(p), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float2 load2_agent(const float *p) {
  const unsigned long long u = __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__builtin_bit_cast(float, (unsigned)u), __builtin_bit_cast(float, (unsigned)(u >> 32)));
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
  static constexpr int NKB = NK < 32 ? 1 : NK / 32;          // 32-channel QK k-blocks
  static constexpr int NBK = KFAM == FAM_F16 ? 0 : NK / block_len(NK);
  static constexpr int LV = VFAM == FAM_F16 ? NV : block_len(NV);
  static constexpr int NBV = VFAM == FAM_F16 ? 1 : NV / LV;  // value scale blocks
  static constexpr int NDT = NV / 16;                        // 16-channel output tiles
  static constexpr int TT = (KFAM == FAM_F16 || VFAM == FAM_F16) ? 32 : 64;  // wave tile
  static constexpr int NT = TT / 16;                         // QK N-tiles per tile
  static constexpr int NCH = TT / 32;                        // PV K-chunks per tile
  static constexpr int TPT = 64 / TT;                        // lanes per token (staging)
  static constexpr int NGQ = (HG + 1) / 2;                   // row groups holding heads
  // LDS per wave: value rows (byte codes or binary16), weights [j][t][16
  // rows] binary16, probabilities [h][t] fp32
  static constexpr int VPITCH = VFAM == FAM_F16 ? 2 * NV + 32 : NV + 16;
  static constexpr int W_V = TT * VPITCH;
  static constexpr int W_A = NBV * TT * 32;
  static constexpr int W_P = 8 * TT * 4;
  static constexpr int W_BYTES = (W_V + W_A + W_P + 15) / 16 * 16;
  // query operands shared by the workgroup's waves: hi/lo rows
  // [NKB][64 lanes][16 bytes], then 2^-sh [8] and block sums [8][4]
  static constexpr int QA_OFF = NWAVE * W_BYTES;
  static constexpr int QA_BYTES = NKB * 64 * 16 + (8 + 8 * 4) * 4;
  static constexpr int MERGE = NWAVE * HG * (NV + 4) * 4;
  static constexpr int LDS_BYTES = cmax<QA_OFF + QA_BYTES, MERGE>::value;
  static_assert(2 * HG <= 16, "at most 8 query heads per workgroup");
  static_assert(TT == 64 || VFAM == FAM_F16 || (RV / 2) % CV == 0,
                "half-row staging needs chunk-aligned halves");
};

typedef short short4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));

// 8 binary16 values of MFMA operand rows from a token-major LDS array via
// the gfx950 transposing load (4 x 16-bit per read, two reads).
__device__ __forceinline__ half8 tr16_pair(const uint8_t *p0, const uint8_t *p1) {
  typedef __attribute__((address_space(3))) short4v lds_s4;
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p0));
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p1));
  H8 o;
  o.u[0] = (uint32_t)(uint16_t)a.x | ((uint32_t)(uint16_t)a.y << 16);
  o.u[1] = (uint32_t)(uint16_t)a.z | ((uint32_t)(uint16_t)a.w << 16);
  o.u[2] = (uint32_t)(uint16_t)b.x | ((uint32_t)(uint16_t)b.y << 16);
  o.u[3] = (uint32_t)(uint16_t)b.z | ((uint32_t)(uint16_t)b.w << 16);
  return o.h;
}

// 8 byte codes (offset binary u) via the 8-bit transposing load.
__device__ __forceinline__ uint2 tr8(const uint8_t *p) {
  typedef __attribute__((address_space(3))) int2v lds_i2;
  const int2v v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2 *)(p));
  return make_uint2((uint32_t)v.x, (uint32_t)v.y);
}

// Offset-binary byte codes u -> exact binary16 (u - off).
__device__ __forceinline__ half8 bytes_to_half8(uint2 x, float off) {
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  const uint32_t c64 = 0x64646464u;
  H8 o;
  o.u[0] = __builtin_amdgcn_perm(c64, x.x, 0x04010400u);
  o.u[1] = __builtin_amdgcn_perm(c64, x.x, 0x04030402u);
  o.u[2] = __builtin_amdgcn_perm(c64, x.y, 0x04010400u);
  o.u[3] = __builtin_amdgcn_perm(c64, x.y, 0x04030402u);
  const _Float16 bias = (_Float16)(-(1024.f + off));
  const half2v bias2 = {bias, bias};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    half2v v = __builtin_bit_cast(half2v, o.u[p]);
    v = v + bias2;
    o.u[p] = __builtin_bit_cast(uint32_t, v);
  }
  return o.h;
}

// Byte codes u <= 15 -> exact binary16 u: an E4M3 byte below 16 encodes
// u * 2^-9 (subnormal for u < 8, exponent 1 above), so the gfx950 scaled
// fp8 conversion with scale 2^9 gives u itself, two bytes per instruction.
__device__ __forceinline__ half8 small_bytes_to_half8(uint2 x) {
  H8 o;
  o.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.x, 512.f, false));
  o.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.x, 512.f, true));
  o.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.y, 512.f, false));
  o.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.y, 512.f, true));
  return o.h;
}

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
      const u32x4 v = ld_stream<u32x4>(plane + tiled_offset(t, byte / CC, R, CC) + byte % CC);
      r.u[0] = v.x; r.u[1] = v.y; r.u[2] = v.z; r.u[3] = v.w;
    } else {
      r.u[0] = r.u[1] = r.u[2] = r.u[3] = 0u;
    }
  } else if constexpr (b == 8) {
    const int byte = e0;
    if (in) {
      const u32x2 v = ld_stream<u32x2>(plane + tiled_offset(t, byte / CC, R, CC) + byte % CC);
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

// Split counts of one unit: body splits, tail splits, body tiles per split.
// Uniform over units for fixed-codec layers; per kv head for low rank.
struct Splits {
  int sb, st, tps;
};

struct SplitIO {
  const uint8_t *kcodes; const uint16_t *ksc; const uint16_t *kmn;
  const uint8_t *vcodes; const uint16_t *vsc; const uint16_t *vmn;
  const float *q;              // HG query rows (stride 128), raw binary32
  const float *rot_w;          // KVarN body: the kv head's vector w (the query is rotated), else null
  float scale;                 // multiplier into the log2 domain
  long long t_begin, t_end;    // token range (plane coordinates), t_begin % 64 == 0
  float *part;                 // partial row of head 0 of the group
  long long part_head_stride;  // floats between consecutive heads' partials
  int dyn;                     // integer path: waves claim tiles past their first at run time
};

// KVarN query rotation in the producers' layout: the 16 lanes of a DPP row
// hold one head, lane g channels 8g .. 8g + 7.  q' = H (q / w) / 128 with
// the butterflies (u, v) -> (u + v, u - v) in increasing stride: strides
// 1, 2, 4 inside the lane, then 8 .. 64 with the partner lane g ^ 1 .. g ^ 8.
// All 16 lanes of a row take part (rows of absent heads hold zeros).
__device__ __forceinline__ void rotate_row8(float (&x)[8], const float *w, int g) {
  const float4 w0 = reinterpret_cast<const float4 *>(w)[2 * g], w1 = reinterpret_cast<const float4 *>(w)[2 * g + 1];
  const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = x[e] / wv[e];
#pragma unroll
  for (int st = 1; st < 8; st <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e & st) continue;
      const float u = x[e], v = x[e + st];
      x[e] = u + v;
      x[e + st] = u - v;
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    const bool upper = (g & m) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __shfl_xor(x[e], m, 64);
      x[e] = upper ? (p - x[e]) : (x[e] + p);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= 1.f / 128.f;
}

__device__ __forceinline__ uint2 side_raw(const uint16_t *base, long long t, bool valid, int nb) {
  if (!valid) return make_uint2(0u, 0u);
  const uint16_t *p = base + t * nb;
  if (nb == 4) return *reinterpret_cast<const uint2 *>(p);
  if (nb == 2) return make_uint2(*reinterpret_cast<const uint32_t *>(p), 0u);
  return make_uint2((uint32_t)*p, 0u);
}

__device__ __forceinline__ void unpack_side(uint2 r, float *v, int nb) {
  v[0] = f16_bits_to_f32(r.x & 0xFFFF);
  if (nb > 1) v[1] = f16_bits_to_f32(r.x >> 16);
  if (nb > 2) { v[2] = f16_bits_to_f32(r.y & 0xFFFF); v[3] = f16_bits_to_f32(r.y >> 16); }
}

__device__ __forceinline__ float wave_max(float x) {
  x = row_max16(x);
  return fmaxf(fmaxf(read_lane(x, 0), read_lane(x, 16)), fmaxf(read_lane(x, 32), read_lane(x, 48)));
}

__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  return (read_lane(x, 0) + read_lane(x, 16)) + (read_lane(x, 32) + read_lane(x, 48));
}

// BF: the binary16 rows are bfloat16 (precision tail in bfloat16); only for
// the all-16-bit configuration.
// ------------------------------------------------ workgroup merge of waves --
// After the tile loops every wave holds a softmax state (m, l, o) per head.
// Each wave publishes its m, scales its own l and o by 2^(m_w - M) (M = the
// maximum over the workgroup's waves) and the split's partial is then a
// plain sum over the waves: one exponential per wave and head instead of one
// per wave, head and channel.
__device__ __forceinline__ float *merge_slots() {
  __shared__ float s[NWAVE * 8];   // [wave][head] m
  return s;
}

__device__ __forceinline__ float merge_max(const float *mw, int h) {
  float M = NEG_INF;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, mw[w * 8 + h]);
  return M;
}

// Scale of wave state m for head h: 2^(m - M), zero for a wave without tokens.
__device__ __forceinline__ float merge_scale(const float *mw, int h, float m) {
  return m == NEG_INF ? 0.f : exp2f(m - merge_max(mw, h));
}

// mg: [wave][h][4 + NV] (l at 1, scaled o at 4..), already scaled.
template <int HG, int NV>
__device__ __forceinline__ void merge_store(const float *mg, const float *mw, float *part,
                                            long long head_stride) {
  constexpr int MS = NV + 4;
  for (int idx = threadIdx.x; idx < HG * NV; idx += WG) {
    const int h = idx / NV, c = idx % NV;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) o += mg[(w * HG + h) * MS + 4 + c];
    float *dst = part + h * head_stride;
    store_agent(dst + 4 + c, o);
    if (c == 0) {
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) L += mg[(w * HG + h) * MS + 1];
      store_agent(dst, merge_max(mw, h));
      store_agent(dst + 1, L);
    }
  }
}

template <class C, bool BF = false>
__device__ void attend_range(const SplitIO &io, uint8_t *lds) {
  constexpr int HG = C::HG, TT = C::TT, NT = C::NT, NDT = C::NDT, NBV = C::NBV;
  constexpr int NBA = C::VFAM == FAM_F16 ? 1 : NBV;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  uint8_t *wl = lds + wave * C::W_BYTES;
  uint8_t *vlds = wl;                                               // [TT][VPITCH]
  uint8_t *alds = wl + C::W_V;                                      // [NBV][TT][16] f16
  float *plds = reinterpret_cast<float *>(wl + C::W_V + C::W_A);    // [8][TT]

  const int n = lane & 15, g = lane >> 4;   // MFMA layout: column n, row group g
  const int tl = lane % TT, tp = lane / TT; // staging layout: token tl, row part tp

  float m_run[2] = {NEG_INF, NEG_INF}, l_lane[2] = {0.f, 0.f};
  float pm[NBV][2];
  float O[NDT][2];
#pragma unroll
  for (int j = 0; j < NBV; ++j) pm[j][0] = pm[j][1] = 0.f;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) O[dt][0] = O[dt][1] = 0.f;

  // this wave's tiles: t_begin + TT * (wave + NWAVE * i)
  const long long first = io.t_begin + (long long)TT * wave;
  const long long stride = (long long)TT * NWAVE;

  // One full tile of register prefetch: while tile i is computed, every
  // load of tile i+1 is in flight.
  KRaw<C> kr[NT][C::NKB];
  uint2 ksr[NT], kmr[NT], vmr[NT];
  uint2 vst = make_uint2(0u, 0u);
  constexpr int NVCH = C::RV / C::CV;            // chunks per value row
  constexpr int PCH = NVCH / C::TPT;             // chunks per staged part
  constexpr int PB = C::RV / C::TPT;             // bytes per staged part
  constexpr int VW = (PB + 3) / 4;
  uint32_t vw[VW];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) ksr[nt] = kmr[nt] = vmr[nt] = make_uint2(0u, 0u);

  auto load_k_nt = [&](long long t0, int nt) {
    const long long t = t0 + 16 * nt + n;
    const bool valid = t < io.t_end;
#pragma unroll
    for (int j = 0; j < C::NKB; ++j) k_load<C>(io.kcodes, t, j, g, valid, kr[nt][j]);
    if constexpr (C::KFAM != FAM_F16) ksr[nt] = side_raw(io.ksc, t, valid, C::NBK);
    if constexpr (C::KFAM == FAM_1) kmr[nt] = side_raw(io.kmn, t, valid, C::NBK);
  };
  auto load_v = [&](long long t0) {
    const long long t = t0 + tl;
    const bool valid = t < io.t_end;
#pragma unroll
    for (int k = 0; k < VW; ++k) vw[k] = 0u;
    if (valid) {
#pragma unroll
      for (int kk = 0; kk < PCH; ++kk) {
        const int k = tp * PCH + kk;
        const uint8_t *p = io.vcodes + tiled_offset(t, k, C::RV, C::CV);
        if constexpr (C::CV == 16) {
          const u32x4 v = ld_stream<u32x4>(p);
          vw[4 * kk] = v.x; vw[4 * kk + 1] = v.y; vw[4 * kk + 2] = v.z; vw[4 * kk + 3] = v.w;
        } else if constexpr (C::CV == 8) {
          const u32x2 v = ld_stream<u32x2>(p);
          vw[2 * kk] = v.x; vw[2 * kk + 1] = v.y;
        } else if constexpr (C::CV == 4) {
          vw[kk] = *reinterpret_cast<const uint32_t *>(p);
        } else if constexpr (C::CV == 2) {
          vw[kk / 2] |= (uint32_t)(*reinterpret_cast<const uint16_t *>(p)) << (16 * (kk & 1));
        } else {
          vw[kk / 4] |= (uint32_t)(*p) << (8 * (kk & 3));
        }
      }
    }
    if constexpr (C::VFAM != FAM_F16) vst = side_raw(io.vsc, t, valid, NBV);
    if constexpr (C::VFAM == FAM_1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const long long tv = t0 + 16 * nt + n;
        vmr[nt] = side_raw(io.vmn, tv, tv < io.t_end, NBV);
      }
    }
  };

  if (first < io.t_end) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) load_k_nt(first, nt);
    load_v(first);
  }

  // ---- query operand (after the first tile's loads are out): row i = lane % 16 is (head i/2, part i%2 = hi/lo),
  // k-group lane / 16.  Prepared once per workgroup by waves 0 and 1 (lane =
  // (head 4w + lane/16, 8-channel group lane%16): the head's amax is a
  // reduction over its 16-lane row) and shared through LDS.
  uint8_t *qa_s = lds + C::QA_OFF;
  float *qinv_s = reinterpret_cast<float *>(qa_s + C::NKB * 64 * 16);
  float *qsum_s = qinv_s + 8;
  if (wave < 2) {
    const int h = 4 * wave + (lane >> 4), G = lane & 15, j = G >> 2, gk = G & 3;
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = h < HG && 8 * G + e < C::NK ? io.q[h * D + 8 * G + e] : 0.f;
    if (io.rot_w) rotate_row8(v, io.rot_w, G);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] *= io.scale;
      amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = row_max16(amax);
    int ex = 0;
    if (amax > 0.f) (void)frexpf(amax, &ex);
    const int sh = 14 - ex;                       // |q * 2^sh| < 2^14
    const float up = ldexpf(1.f, sh);
    H8 hi, lo;
    float ssum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t p0 = split16<BF>(v[e] * up), p1 = split16<BF>(v[e + 1] * up);
      hi.u[e / 2] = (p0 & 0xFFFFu) | (p1 << 16);
      lo.u[e / 2] = (p0 >> 16) | (p1 & 0xFFFF0000u);
      ssum += v[e];
      ssum += v[e + 1];
    }
    ssum += __shfl_xor(ssum, 1, 64);
    ssum += __shfl_xor(ssum, 2, 64);
    if (j < C::NKB) {
      uint4 *dst = reinterpret_cast<uint4 *>(qa_s) + j * 64 + 2 * (h & 7) + 16 * gk;
      dst[0] = make_uint4(hi.u[0], hi.u[1], hi.u[2], hi.u[3]);
      dst[1] = make_uint4(lo.u[0], lo.u[1], lo.u[2], lo.u[3]);
      if (gk == 0 && h < HG) qsum_s[h * 4 + j] = ssum;
      if (G == 0 && h < HG) qinv_s[h] = ldexpf(1.f, -sh);
    }
  }
  __syncthreads();
  half8 qa[C::NKB];
#pragma unroll
  for (int j = 0; j < C::NKB; ++j) {
    H8 a;
    const uint4 x = reinterpret_cast<const uint4 *>(qa_s)[j * 64 + lane];
    a.u[0] = x.x; a.u[1] = x.y; a.u[2] = x.z; a.u[3] = x.w;
    qa[j] = a.h;
  }

  // result layout (QK and PV alike): row group g holds heads 2g (rows 4g,
  // 4g+1: hi, lo) and 2g+1 (rows 4g+2, 4g+3)
  float inv_k[2], qs_k[2][C::NKB];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int h = 2 * g + k;
    inv_k[k] = h < HG ? qinv_s[h] : 0.f;
#pragma unroll
    for (int j = 0; j < C::NKB; ++j) qs_k[k][j] = (C::KFAM == FAM_1 && h < HG) ? qsum_s[h * 4 + j] : 0.f;
  }

  for (int i = lane; i < C::W_A / 16; i += 64)
    reinterpret_cast<uint4 *>(alds)[i] = make_uint4(0u, 0u, 0u, 0u);

  for (long long t0 = first; t0 < io.t_end; t0 += stride) {
    const long long tn = t0 + stride;
    const bool more = tn < io.t_end;

    // ---- stage the value row part: offset-binary byte codes, or binary16
    {
      uint8_t *dst = vlds + tl * C::VPITCH;
      if constexpr (C::VFAM == FAM_F16) {
        dst += tp * PB;
#pragma unroll
        for (int k = 0; k < VW; k += 4)
          *reinterpret_cast<uint4 *>(dst + 4 * k) = make_uint4(vw[k], vw[k + 1], vw[k + 2], vw[k + 3]);
      } else if constexpr (C::VBITS == 8) {
        dst += tp * (C::NV / C::TPT);
        const uint32_t fl = C::VFAM == FAM_0 ? 0x80808080u : 0u;
#pragma unroll
        for (int k = 0; k < VW; k += 4)
          *reinterpret_cast<uint4 *>(dst + 4 * k) = make_uint4(vw[k] ^ fl, vw[k + 1] ^ fl, vw[k + 2] ^ fl, vw[k + 3] ^ fl);
      } else if constexpr (C::VBITS == 4) {
        dst += tp * (C::NV / C::TPT);
        const uint32_t fl = C::VFAM == FAM_0 ? 0x88888888u : 0u;
#pragma unroll
        for (int k = 0; k < VW; ++k) {
          const uint32_t x = vw[k] ^ fl;
          const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
          *reinterpret_cast<uint2 *>(dst + 8 * k) =
              make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
        }
      } else {
        constexpr int b = C::VBITS;
        constexpr uint32_t off = C::VFAM == FAM_0 ? (1u << (b - 1)) : 0u;
        constexpr uint32_t m = (1u << b) - 1u;
        constexpr int NC = C::NV / C::TPT;       // codes in this part
#pragma unroll
        for (int c4 = 0; c4 < NC / 4; ++c4) {
          uint32_t w = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t u = ((uint32_t)field<b, false>(vw, (4 * c4 + e) * b) + off) & m;
            w |= u << (8 * e);
          }
          *reinterpret_cast<uint32_t *>(dst + 4 * c4) = w;
        }
      }
    }
    const uint2 vst_cur = vst;
    uint2 vmr_cur[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vmr_cur[nt] = vmr[nt];
    if (more) load_v(tn);               // value registers are free: next tile's values load during this one

    // ---- QK on the matrix cores
    float s[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      half8 kb[C::NKB];
#pragma unroll
      for (int j = 0; j < C::NKB; ++j) kb[j] = k_convert<C>(kr[nt][j]);
      float dk[4] = {1.f, 1.f, 1.f, 1.f}, mk[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (C::KFAM != FAM_F16) unpack_side(ksr[nt], dk, C::NBK);
      if constexpr (C::KFAM == FAM_1) unpack_side(kmr[nt], mk, C::NBK);
      if (more) load_k_nt(tn, nt);      // registers of N-tile nt are free again
      const long long t = t0 + 16 * nt + n;
      const bool valid = t < io.t_end;
      float a1[2] = {0.f, 0.f}, a2[2] = {0.f, 0.f};
      if constexpr (C::KFAM == FAM_F16) {
        floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < C::NKB; ++j) c = mfma16<BF>(qa[j], kb[j], c);
        a1[0] = c[0] + c[1];
        a1[1] = c[2] + c[3];
      } else {
#pragma unroll
        for (int j = 0; j < C::NKB; ++j) {
          const floatx4 z = {0.f, 0.f, 0.f, 0.f};
          const floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[j], kb[j], z, 0, 0, 0);
          a1[0] = fmaf(dk[j], c[0] + c[1], a1[0]);
          a1[1] = fmaf(dk[j], c[2] + c[3], a1[1]);
          if constexpr (C::KFAM == FAM_1) {
            a2[0] = fmaf(mk[j], qs_k[0][j], a2[0]);
            a2[1] = fmaf(mk[j], qs_k[1][j], a2[1]);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 2; ++k)
        s[nt][k] = (valid && 2 * g + k < HG) ? fmaf(a1[k], inv_k[k], a2[k]) : NEG_INF;
    }

    // ---- online softmax (per wave)
    float alpha[2], mnew[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float mx = s[0][k];
#pragma unroll
      for (int nt = 1; nt < NT; ++nt) mx = fmaxf(mx, s[nt][k]);
      mx = row_max16(mx);
      mnew[k] = fmaxf(m_run[k], mx);
      alpha[k] = (mnew[k] == NEG_INF) ? 1.f : __builtin_amdgcn_exp2f(m_run[k] - mnew[k]);
      m_run[k] = mnew[k];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mv[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (C::VFAM == FAM_1) unpack_side(vmr_cur[nt], mv, NBV);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float p = __builtin_amdgcn_exp2f(s[nt][k] - mnew[k]);   // exp2(-inf) = 0
        l_lane[k] = (nt == 0 ? l_lane[k] * alpha[k] : l_lane[k]) + p;
        if (2 * g + k < HG) plds[(2 * g + k) * TT + 16 * nt + n] = p;
        if constexpr (C::VFAM == FAM_1) {
#pragma unroll
          for (int j = 0; j < NBV; ++j) pm[j][k] = (nt == 0 ? pm[j][k] * alpha[k] : pm[j][k]) + p * mv[j];
        }
      }
    }

    wave_sync_lds();                    // probabilities and rows visible

    // ---- weights x = p * d_j * 2^(14 - e_j), split hi / lo, rows (head, part)
    float back[NBA];
    {
      float dv[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (C::VFAM != FAM_F16) unpack_side(vst_cur, dv, NBV);
      constexpr int H0 = 0, H1 = HG;       // heads this lane stages
      float ps[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) ps[h] = (h < HG && (C::TPT == 1 || (h >> 2) == tp)) ? plds[h * TT + tl] : 0.f;
      (void)H0; (void)H1;
#pragma unroll
      for (int j = 0; j < NBA; ++j) {
        int ex = 1;
        if constexpr (C::VFAM != FAM_F16) {
          const float emax = wave_max(dv[j]);
          ex = 0;
          if (emax > 0.f) (void)frexpf(emax, &ex);
        }
        const float scl = ldexpf(dv[j], 14 - ex);
        back[j] = ldexpf(1.f, ex - 14);
        // rows (2h, 2h+1) = (hi, lo) of head h; rows >= 2*HG stay zero
        uint32_t rw[HG];
#pragma unroll
        for (int h = 0; h < HG; ++h) rw[h] = split16<BF>(ps[h] * scl);
        uint32_t *dst = reinterpret_cast<uint32_t *>(alds + ((j * TT) + tl) * 32);
        if constexpr (C::TPT == 1) {
          if constexpr (HG == 4) {
            *reinterpret_cast<uint4 *>(dst) = make_uint4(rw[0], rw[1], rw[2], rw[3]);
          } else {
#pragma unroll
            for (int h = 0; h < HG; ++h) dst[h] = rw[h];
          }
        } else {
#pragma unroll
          for (int h = 0; h < HG; ++h)
            if ((h >> 2) == tp) dst[h] = rw[h];
        }
      }
    }
    wave_sync_lds();

    // ---- PV on the matrix cores: A = weights [rows][32 tokens], B = values
    floatx4 ct[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) ct[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < C::NCH; ++kc) {
      const int tok = 32 * kc + 8 * g;
#pragma unroll
      for (int j = 0; j < NBA; ++j) {
        const uint8_t *pa = alds + ((j * TT) + tok + (n >> 2)) * 32 + 8 * (n & 3);
        const half8 a = tr16_pair(pa, pa + 4 * 32);
        constexpr int DPB = C::VFAM == FAM_F16 ? NDT : C::LV / 16;   // tiles per A operand
#pragma unroll
        for (int d = 0; d < DPB; ++d) {
          const int dt = j * DPB + d;
          half8 bv;
          if constexpr (C::VFAM == FAM_F16) {
            const uint8_t *pb = vlds + (tok + (n >> 2)) * C::VPITCH + (16 * dt + 4 * (n & 3)) * 2;
            bv = tr16_pair(pb, pb + 4 * C::VPITCH);
          } else {
            const uint8_t *pb = vlds + (tok + (n >> 1)) * C::VPITCH + 16 * dt + 8 * (n & 1);
            constexpr float voff = C::VFAM == FAM_0 ? (float)(1 << (C::VBITS - 1)) : 0.f;
            bv = bytes_to_half8(tr8(pb), voff);
          }
          ct[dt] = mfma16<BF>(a, bv, ct[dt]);
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      constexpr int DPB = C::VFAM == FAM_F16 ? NDT : C::LV / 16;
      const float bk = back[dt / DPB];
      O[dt][0] = fmaf(O[dt][0], alpha[0], (ct[dt][0] + ct[dt][1]) * bk);
      O[dt][1] = fmaf(O[dt][1], alpha[1], (ct[dt][2] + ct[dt][3]) * bk);
    }
    wave_sync_lds();                    // LDS tiles are free for the next tile
  }

  // ---- close this wave: l and pm over the row's 16 lanes
  float lsum[2], pmsum[NBV][2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    lsum[k] = row_sum16(l_lane[k]);
#pragma unroll
    for (int j = 0; j < NBV; ++j) pmsum[j][k] = C::VFAM == FAM_1 ? row_sum16(pm[j][k]) : 0.f;
  }
  float *mw = merge_slots();
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (2 * g + k < HG && n == 0) mw[wave * 8 + 2 * g + k] = m_run[k];
  __syncthreads();   // every wave is done with its LDS tiles; wave maxima published

  // merge area: [wave][h][4 + NV]: -, l, -, -, o[NV], scaled to the
  // workgroup maximum
  float *mg = reinterpret_cast<float *>(lds);
  constexpr int MS = C::NV + 4;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int h = 2 * g + k;
    if (h < HG) {
      const float f = merge_scale(mw, h, m_run[k]);
      float *dst = mg + (wave * HG + h) * MS;
      if (n == 0) dst[1] = lsum[k] * f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        float o = O[dt][k];
        if constexpr (C::VFAM == FAM_1) o += pmsum[(16 * dt) / C::LV][k];
        dst[4 + 16 * dt + n] = o * f;
      }
    }
  }
  __syncthreads();
  merge_store<HG, C::NV>(mg, mw, io.part, io.part_head_stride);
}

#include "kvq_decode_q.hpp"

// LDS of a body configuration: the integer-QK path for quantised K and V,
// the binary16 path otherwise.
template <class C, bool INT = (C::KFAM != FAM_F16 && C::VFAM != FAM_F16)>
struct BodyLds {
  static constexpr bool INT_QK = false;
  static constexpr int bytes = C::LDS_BYTES;
};
template <class C>
struct BodyLds<C, true> {
  static constexpr bool INT_QK = true;
  static constexpr int bytes = QCfg<C>::LDS_BYTES;
};

// ------------------------------------------------------------- kernels ----


// Low-rank head tables of the decode's argument block (DecodeArgs is the
// kernels' first argument), read from the argument segment at run-time
// indices: indexing the by-value argument itself makes the compiler copy
// the whole block to scratch.  K and V share the tables.
template <class T>
__device__ __forceinline__ T decode_arg_at(size_t byte_off, int i) {
  typedef const __attribute__((address_space(4))) T *cptr;
  typedef const __attribute__((address_space(4))) uint8_t *bptr;
  return ((cptr)((bptr)__builtin_amdgcn_kernarg_segment_ptr() + byte_off))[i];
}
__device__ __forceinline__ int lr_rank(int h) {
  return decode_arg_at<int16_t>(offsetof(DecodeArgs, k) + offsetof(PlaneArgs, hrank), h);
}
__device__ __forceinline__ int lr_codec(int h) {
  return decode_arg_at<int8_t>(offsetof(DecodeArgs, k) + offsetof(PlaneArgs, hcodec), h);
}
__device__ __forceinline__ int lr_sbody(int h) { return decode_arg_at<int16_t>(offsetof(DecodeArgs, lr_sbody), h); }
__device__ __forceinline__ int lr_tps(int h) { return decode_arg_at<int16_t>(offsetof(DecodeArgs, lr_tps), h); }
__device__ __forceinline__ int lr_first(int h) { return decode_arg_at<int16_t>(offsetof(DecodeArgs, lr_first), h); }
// Geometry of low-rank plane (b, h): offsets are prefix sums over heads.
__device__ __forceinline__ HeadGeom lr_geom(const DecodeArgs &a, int b, int h) {
  HeadGeom g;
  g.codec = lr_codec(h);
  g.n = lr_rank(h);
  g.R = row_bytes(g.codec, g.n);
  g.c = chunk_bytes(g.R);
  g.L = block_len(g.n);
  g.nblk = g.n / g.L;
  const int rb = decode_arg_at<int32_t>(offsetof(DecodeArgs, k) + offsetof(PlaneArgs, hrow_before), h);
  const int nb = decode_arg_at<int32_t>(offsetof(DecodeArgs, k) + offsetof(PlaneArgs, hblk_before), h);
  g.codes_off = (long long)a.k.capacity * ((long long)b * a.k.row_all + rb);
  g.scales_off = (long long)a.k.capacity * ((long long)b * a.k.blk_all + nb);
  return g;
}

// Tokens of sequence b in a ragged batch: body and tail counts of its own
// T_b (the plan's ranges are for the longest sequence).
__device__ __forceinline__ void seq_counts(const DecodeArgs &a, int b, int &body, int &tail) {
  int Tb = a.seq[b] + a.seq_add;
  Tb = Tb < 0 ? 0 : Tb > a.T ? a.T : Tb;
  tail = a.N < Tb ? a.N : Tb;
  body = Tb - tail;
}

// Low-rank query coordinates of the group's HG heads: q'[h][n] = scale *
// sum_c q[h][c] P[c][n] for n < rank, into LDS rows of 128 floats at q_out.
// Wave w takes output columns 16w .. 16w + 15 on the matrix cores (binary32
// 16x16x4: row = head, k = input channel 4i + lane/16 in row order), then
// the workgroup waits for all of them.  Runs before the body's first loads;
// the rows stay untouched until the producers of the query operands read
// them (nothing writes LDS before that barrier).
template <int HG>
__device__ __forceinline__ void lr_query_project(const DecodeArgs &a, const float *q, int kvh, int rank,
                                                 float *q_out) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (16 * w < rank) {
    const int i_a = lane & 15, k_a = lane >> 4;
    const uint16_t *P = a.k.proj + (long long)kvh * D * D;
    const int n0 = 16 * w;
    // rows past the group read head 0 (every load unconditional, so the
    // products can start as operands arrive) and are zeroed before use
    const bool live = i_a < HG;
    const float *qr = q + (live ? i_a : 0) * D + k_a;
    float qa[D / 4];
    uint16_t pb[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      qa[i] = qr[4 * i];
      pb[i] = P[(4 * i + k_a) * D + n0 + i_a];
    }
    floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 4; ++i)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(live ? qa[i] : 0.f, f16_bits_to_f32(pb[i]), c, 0, 0, 0);
    // lane holds rows 4 (lane / 16) + rr of column lane % 16
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int h = 4 * k_a + rr;
      if (h < HG) q_out[h * D + n0 + i_a] = c[rr] * a.scale_body;
    }
  }
  __syncthreads();
}

// LR: per-head widths and codecs (low-rank planes, offsets from the head
// tables); otherwise every plane has the configuration's fixed geometry.
template <class C, bool LR>
__device__ __forceinline__ void run_body(const DecodeArgs &a, const Splits &sp, int b, int kvh, int hg, int s,
                                         uint8_t *lds) {
  long long kco, kso, vco, vso;
  if constexpr (LR) {
    const HeadGeom gk = lr_geom(a, b, kvh), gv = gk;
    kco = gk.codes_off; kso = gk.scales_off;
    vco = gv.codes_off; vso = gv.scales_off;
  } else {
    const long long rows = (long long)(b * a.Hkv + kvh) * a.k.capacity;
    kco = rows * C::RK; kso = rows * C::NBK;
    vco = rows * C::RV; vso = rows * (C::VFAM == FAM_F16 ? 0 : C::NBV);
  }
  const int head0 = kvh * a.G + hg * C::HG;
  SplitIO io;
  io.kcodes = a.k.codes + kco;
  io.ksc = a.k.scales ? a.k.scales + kso : nullptr;
  io.kmn = a.k.mins ? a.k.mins + kso : nullptr;
  io.vcodes = a.v.codes + vco;
  io.vsc = a.v.scales ? a.v.scales + vso : nullptr;
  io.vmn = a.v.mins ? a.v.mins + vso : nullptr;
  io.q = a.q_body + ((long long)b * a.Hq + head0) * D;
  io.scale = a.scale_body;
  io.rot_w = !LR && a.k.basis == KVQ_BASIS_HADAMARD ? a.k.w + (long long)kvh * D : nullptr;
  if constexpr (LR) lr_query_project<C::HG>(a, io.q, kvh, C::NK, reinterpret_cast<float *>(lds));
  const long long tps = (long long)sp.tps * 64;
  io.t_begin = (long long)s * tps;
  io.t_end = io.t_begin + tps < a.body_tokens ? io.t_begin + tps : a.body_tokens;
  if (a.seq) {
    int body, tail;
    seq_counts(a, b, body, tail);
    if (io.t_end > body) io.t_end = body;
  }
  io.part = a.part + (((long long)b * a.Hq + head0) * a.S_total + s) * PSTRIDE;
  io.part_head_stride = (long long)a.S_total * PSTRIDE;
  io.dyn = sp.tps >= DYN_TILES_PER_WAVE * NWAVE;
  if constexpr (BodyLds<C>::INT_QK) attend_q<C, LR>(io, lds);
  else attend_range<C>(io, lds);
}

template <int HG, bool BF>
__device__ __forceinline__ void run_tail(const DecodeArgs &a, const Splits &sp, int b, int kvh, int hg, int s,
                                         uint8_t *lds) {
  using C = Cfg<HG, KVQ_F16, KVQ_F16, D, D>;
  const long long plane = (long long)b * a.Hkv + kvh;
  const int head0 = kvh * a.G + hg * HG;
  const int st = s - sp.sb;
  SplitIO io;
  io.kcodes = reinterpret_cast<const uint8_t *>(a.k.tail) + plane * a.k.tail_len * (2 * D);
  io.vcodes = reinterpret_cast<const uint8_t *>(a.v.tail) + plane * a.v.tail_len * (2 * D);
  io.ksc = io.kmn = io.vsc = io.vmn = nullptr;
  io.q = a.q_tail + ((long long)b * a.Hq + head0) * D;
  io.rot_w = nullptr;
  io.scale = a.scale_tail;
  const long long tps = (long long)a.tps_tail * 64;
  io.t_begin = (long long)st * tps;
  io.t_end = io.t_begin + tps < a.tail_tokens ? io.t_begin + tps : a.tail_tokens;
  if (a.seq) {
    int body, tail;
    seq_counts(a, b, body, tail);
    if (io.t_end > tail) io.t_end = tail;
  }
  io.part = a.part + (((long long)b * a.Hq + head0) * a.S_total + s) * PSTRIDE;
  io.part_head_stride = (long long)a.S_total * PSTRIDE;
  attend_range<C, BF>(io, lds);
}

// ------------------------------------------------------ split combine ----

// Merge of one query head's split partials (the split-K decode of the
// forum post: M = max m_s, L = sum l_s 2^(m_s - M), o = sum o_s 2^(m_s - M)
// / L), one wave, in a single pass over the partials: every (m, l) and
// output load is issued before any arithmetic waits on it.  Body partials
// are in the stored basis and go back to the raw basis first (Hadamard
// transform and 1/w for KVarN, P_h for low rank) before they meet the tail
// partials.  `olow` holds 128 floats of LDS.
// ONE: body and tail partials share the raw basis (plain layers), so all
// splits merge into one accumulator.
template <bool ONE>
__device__ __forceinline__ void combine_head(const DecodeArgs &a, const Splits &sp, float *__restrict__ out,
                                             int b, int h, float *olow) {
  const int lane = threadIdx.x & 63;
  const long long bh = (long long)b * a.Hq + h;
  const float *pr = a.part + bh * a.S_total * PSTRIDE;
  const int S = sp.sb + sp.st, Sb = sp.sb;

  // Batches of up to 32 splits: every (m, l) and output load of a batch is
  // issued before any of it is used (one round trip to the coherent level
  // per batch); batches merge online.  Body (s < Sb) and tail splits are
  // merged separately, their outputs being in different bases.
  constexpr int NB = 32;
  float mb = NEG_INF, mt = NEG_INF;
  float lb = 0.f, lt = 0.f, ob0 = 0.f, ob1 = 0.f, ot0 = 0.f, ot1 = 0.f;
  for (int s0 = 0; s0 < S; s0 += NB) {
    const int cnt = S - s0 < NB ? S - s0 : NB;
    const int sl = s0 + (lane < cnt ? lane : cnt - 1);
    const float *pb = pr + (long long)s0 * PSTRIDE;          // this batch's first split
    const float2 ml = load2_agent(pb + (unsigned)((sl - s0) * PSTRIDE));
    const float *po = pb + 4 + 2 * lane;
    float2 v[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int i = k < cnt ? k : cnt - 1;                   // uniform
      v[k] = load2_agent(po + (unsigned)(i * PSTRIDE));
    }
    const bool own = lane < cnt, body = sl < Sb;
    if constexpr (ONE) {
      const float nm = fmaxf(mb, wave_max(own ? ml.x : NEG_INF));
      const float cb = mb == NEG_INF ? 0.f : exp2f(mb - nm);
      lb *= cb; ob0 *= cb; ob1 *= cb;
      mb = nm;
      const float wgt = !own || ml.x == NEG_INF ? 0.f : exp2f(ml.x - mb);
      lb += wave_sum(wgt * ml.y);
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float wk = read_lane(wgt, k);
        ob0 = fmaf(wk, v[k].x, ob0);
        ob1 = fmaf(wk, v[k].y, ob1);
      }
      continue;
    }
    const float xb = wave_max(own && body ? ml.x : NEG_INF), xt = wave_max(own && !body ? ml.x : NEG_INF);
    // rescale what earlier batches summed to the new segment maxima
    const float nmb = fmaxf(mb, xb), nmt = fmaxf(mt, xt);
    const float cb = mb == NEG_INF ? 0.f : exp2f(mb - nmb);
    const float ct = mt == NEG_INF ? 0.f : exp2f(mt - nmt);
    lb *= cb; ob0 *= cb; ob1 *= cb;
    lt *= ct; ot0 *= ct; ot1 *= ct;
    mb = nmb;
    mt = nmt;
    const float M = body ? mb : mt;
    const float wgt = !own || ml.x == NEG_INF ? 0.f : exp2f(ml.x - M);
    lb += wave_sum(body ? wgt * ml.y : 0.f);
    lt += wave_sum(body ? 0.f : wgt * ml.y);
    // split k's weight from lane k as a scalar operand (zero past cnt and in
    // the other segment): straight-line FMAs, no per-split branch or LDS
    // round trip
    const float wbl = body ? wgt : 0.f, wtl = body ? 0.f : wgt;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float wkb = read_lane(wbl, k), wkt = read_lane(wtl, k);
      ob0 = fmaf(wkb, v[k].x, ob0);
      ob1 = fmaf(wkb, v[k].y, ob1);
      ot0 = fmaf(wkt, v[k].x, ot0);
      ot1 = fmaf(wkt, v[k].y, ot1);
    }
  }

  // body sum back to the raw basis
  const int g = h / a.G;
  if (!ONE && Sb > 0) {
    if (a.v.basis == KVQ_BASIS_HADAMARD) {
      float x0 = ob0 + ob1, x1 = ob0 - ob1;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(x0, m, 64), p1 = __shfl_xor(x1, m, 64);
        const bool upper = (lane & m) != 0;
        x0 = upper ? (p0 - x0) : (x0 + p0);
        x1 = upper ? (p1 - x1) : (x1 + p1);
      }
      const float *wv = a.v.w + (long long)g * D;
      ob0 = x0 * (1.f / 128.f) / wv[2 * lane];
      ob1 = x1 * (1.f / 128.f) / wv[2 * lane + 1];
    } else if (a.v.basis == KVQ_BASIS_LOWRANK) {
      const int nv = lr_rank(g);
      olow[2 * lane] = 2 * lane < nv ? ob0 : 0.f;
      olow[2 * lane + 1] = 2 * lane + 1 < nv ? ob1 : 0.f;
      wave_sync_lds();
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
  const float M = fmaxf(mb, mt);
  const float wb = mb == NEG_INF ? 0.f : exp2f(mb - M);
  const float wt = mt == NEG_INF ? 0.f : exp2f(mt - M);
  const float L = wb * lb + wt * lt;
  const float inv = L > 0.f ? 1.f / L : 0.f;       // no tokens (empty sequence): zero output
  float2 o;
  o.x = (wb * ob0 + wt * ot0) * inv;
  o.y = (wb * ob1 + wt * ot1) * inv;
  reinterpret_cast<float2 *>(out + bh * D)[lane] = o;
}

// Word of unit u's completion counter: units u mod 16 sit in different
// 4 KB pages of the counter region (u / 16 is the word within the page).
// Device-scope atomics on one cache line are performed one after another,
// so counters packed side by side made every unit's splits queue behind
// the others' (up to 2 us on short contexts).
__device__ __forceinline__ unsigned *unit_counter(const DecodeArgs &a, int unit) {
  return a.cnt + (unit & (DECODE_CNT_PAGES - 1)) * (DECODE_MAX_UNITS / DECODE_CNT_PAGES) +
         unit / DECODE_CNT_PAGES;
}

// After a split's partials are stored: count the split as finished (one
// device-scope counter per unit in the workspace); the workgroup that
// finishes its unit last merges the unit's heads (wave w takes head w of
// the group) and re-arms the counter, so counters are zero between calls.
__device__ __forceinline__ void finish_split(const DecodeArgs &a, const Splits &sp, int b, int kvh, int hg,
                                             uint8_t *lds) {
  __shared__ unsigned s_last;
  __builtin_amdgcn_s_waitcnt(0);           // this thread's partial stores completed
  __syncthreads();
  unsigned *cnt = unit_counter(a, (b * a.Hkv + kvh) * a.NHG + hg);
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(sp.sb + sp.st - 1);
  __syncthreads();
  if (!s_last) return;
  const int w = threadIdx.x >> 6;
  if (w < a.HG) {
    float *olow = reinterpret_cast<float *>(lds) + w * D;
    if (a.v.basis == KVQ_BASIS_PLAIN) combine_head<true>(a, sp, a.out, b, kvh * a.G + hg * a.HG + w, olow);
    else combine_head<false>(a, sp, a.out, b, kvh * a.G + hg * a.HG + w, olow);
  }
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Plain / KVarN body with fixed codecs, plus the binary16 tail splits in
// the same launch (so the short tail work overlaps the body).  Grid:
// x = split (tail splits first, then body splits), y = kv head * NHG +
// head group, z = batch entry; one 32-bit division per workgroup.
__device__ __forceinline__ bool split_decode(const DecodeArgs &a, int &b, int &kvh, int &hg, int &s) {
  const unsigned x = blockIdx.x, y = blockIdx.y;
  const bool tail = x < (unsigned)a.S_tail;
  s = tail ? a.S_body + (int)x : (int)x - a.S_tail;
  const unsigned nhg = (unsigned)a.NHG;
  kvh = (int)(y / nhg);
  hg = (int)(y - (unsigned)kvh * nhg);
  b = (int)blockIdx.z;
  return tail;
}

// The arguments a workgroup reads before its first tile load, fetched in
// one batch of scalar loads at entry: the argument lines are cold at every
// launch, and loads issued behind branches would each pay that latency.
__device__ __forceinline__ void fetch_args(const DecodeArgs &a) {
  asm volatile("" ::"s"(a.S_tail), "s"(a.S_body), "s"(a.S_total), "s"(a.NHG), "s"(a.G),
               "s"(a.Hkv), "s"(a.Hq), "s"(a.body_tokens), "s"(a.tail_tokens), "s"(a.tps_body),
               "s"(a.tps_tail), "s"(a.scale_body), "s"(a.scale_tail), "s"(a.q_body),
               "s"(a.q_tail), "s"(a.part));
  asm volatile("" ::"s"(a.k.codes), "s"(a.k.scales), "s"(a.k.mins), "s"(a.k.tail),
               "s"(a.k.capacity), "s"(a.k.tail_len), "s"(a.v.codes), "s"(a.v.scales),
               "s"(a.v.mins), "s"(a.v.tail), "s"(a.k.tail_bf16), "s"(a.seq));
}

// Fused step (a.k_new non-null): the new token of sequence b sits at
// position t (its count before the step); the one workgroup whose tiles hold
// it (the tail split of ring slot t mod N, or without a tail the body split
// of row t) writes its K row (wave 0) and V row (wave 1) exactly as the
// append kernel does, then waits for the stores before any wave loads.  Only
// launched with one head group per kv head, so no other workgroup reads
// those tiles.
template <int CODEC>
__device__ __forceinline__ void fused_row(const PlaneArgs &p, const float *x_new, int b, int kvh, int t,
                                          uint8_t *lds) {
  const int lane = threadIdx.x & 63;
  const long long plane = (long long)b * p.hkv + kvh;
  const float2 x = reinterpret_cast<const float2 *>(x_new + plane * D)[lane];
  if (p.tail_len > 0) arow::store_tail(p, plane, t, x);
  float ac, cc;
  arow::stored_coords(p, kvh, x, ac, cc);
  arow::store_row<CODEC>(p, plane * p.capacity, t, ac, cc,
                         reinterpret_cast<uint32_t *>(lds) + (threadIdx.x >> 6) * 32);
}

template <int KC, int VC>
__device__ __forceinline__ void fused_append(const DecodeArgs &a, int b, int kvh, int s, bool tail,
                                             uint8_t *lds) {
  int t = a.T - 1;
  if (a.seq) {
    const int sb = a.seq[b];
    t = sb < 0 ? 0 : sb > a.T - 1 ? a.T - 1 : sb;
  }
  const bool mine = a.N > 0 ? tail && (s - a.S_body) == (t % a.N) / (a.tps_tail * 64)
                            : !tail && s == t / (a.tps_body * 64);
  if (!mine) return;
  const int w = threadIdx.x >> 6;
  if (w == 0) fused_row<KC>(a.k, a.k_new, b, kvh, t, lds);
  else if (w == 1) fused_row<VC>(a.v, a.v_new, b, kvh, t, lds);
  __builtin_amdgcn_s_waitcnt(0);           // the rows are in L2 before any wave loads
  __syncthreads();
}

// Low-rank layers: the new token's row of plane p (tail copy, u = P^T x,
// the head's own width and codec), exactly as the append kernel's one-token
// path stores it; this wave's 1280 bytes of LDS hold x, u and the packed row.
__device__ __forceinline__ void fused_row_lr(const PlaneArgs &p, const float *x_new, const HeadGeom &g, int b,
                                             int kvh, int t, uint8_t *lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long plane = (long long)b * p.hkv + kvh;
  const float2 x = reinterpret_cast<const float2 *>(x_new + plane * D)[lane];
  if (p.tail_len > 0) arow::store_tail(p, plane, t, x);
  float *xin = reinterpret_cast<float *>(lds + w * 1280), *coords = xin + D;
  arow::lr_project_row(p.proj + (long long)kvh * D * D, x, xin, coords);
  arow::lr_store_row(p, g, t, coords[2 * lane], coords[2 * lane + 1], reinterpret_cast<uint32_t *>(coords + D));
}

// The workgroup whose tiles hold the new token's position (the tail split
// of its ring slot, else the body split of its row) writes its K and V rows
// before any wave loads a tile.  With several head groups per kv head, the
// owner of every group writes the same bytes.
__device__ __forceinline__ void fused_append_lr(const DecodeArgs &a, const Splits &sp, int b, int kvh, int s,
                                                bool tail, uint8_t *lds) {
  int t = a.T - 1;
  if (a.seq) {
    const int sb = a.seq[b];
    t = sb < 0 ? 0 : sb > a.T - 1 ? a.T - 1 : sb;
  }
  const bool mine = a.N > 0 ? tail && (s - sp.sb) == (t % a.N) / (a.tps_tail * 64)
                            : !tail && s == t / (sp.tps * 64);
  if (!mine) return;
  const int w = threadIdx.x >> 6;
  const HeadGeom g = lr_geom(a, b, kvh);
  if (w == 0) fused_row_lr(a.k, a.k_new, g, b, kvh, t, lds);
  else if (w == 1) fused_row_lr(a.v, a.v_new, g, b, kvh, t, lds);
  __builtin_amdgcn_s_waitcnt(0);           // the rows are in L2 before any wave loads
  __syncthreads();
}

template <int HG, int KC, int VC>
__global__ __launch_bounds__(WG, DECODE_WG_PER_CU) void decode_kernel(DecodeArgs a) {
  using CB = Cfg<HG, KC, VC, D, D>;
  using CT = Cfg<HG, KVQ_F16, KVQ_F16, D, D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[cmax<BodyLds<CB>::bytes, CT::LDS_BYTES>::value];
  int b, kvh, hg, s;
  fetch_args(a);
  const Splits sp = {a.S_body, a.S_tail, a.tps_body};
  const bool tail = split_decode(a, b, kvh, hg, s);
  if (a.k_new) fused_append<KC, VC>(a, b, kvh, s, tail, lds);
  if (tail) {
    if (a.k.tail_bf16) run_tail<HG, true>(a, sp, b, kvh, hg, s, lds);
    else run_tail<HG, false>(a, sp, b, kvh, hg, s, lds);
  }
  else run_body<CB, false>(a, sp, b, kvh, hg, s, lds);
  finish_split(a, sp, b, kvh, hg, lds);
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
  static constexpr int bytes = cmax<cmax<BodyLds<Cfg<HG, KVQ_Q4_1, KVQ_Q4_1, 128, 128>>::bytes,
                                         BodyLds<Cfg<HG, KVQ_Q3_1, KVQ_Q3_1, 128, 128>>::bytes>::value,
                                    Cfg<HG, KVQ_F16, KVQ_F16, D, D>::LDS_BYTES>::value;
};

template <int HG>
__global__ __launch_bounds__(WG, DECODE_WG_PER_CU) void decode_lowrank_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LrLds<HG>::bytes];
  fetch_args(a);
  // Per-head split counts (a head's tiles cost more or less with its rank
  // and bits).  Grid x runs over every (kv head, split) of one batch entry
  // and head group: the body splits head by head (head h's first at
  // lr_first[h]), then S_tail tail splits per head; y = head group, z =
  // batch entry.
  const int x = (int)blockIdx.x, hg = (int)blockIdx.y, b = (int)blockIdx.z;
  const bool tail = x >= a.lr_body_all;
  int kvh = 0;
  if (!tail) {
    for (int h = 1; h < a.Hkv; ++h)
      if (x >= lr_first(h)) kvh = h;
  } else {
    kvh = (x - a.lr_body_all) / a.S_tail;
  }
  const Splits sp = {lr_sbody(kvh), a.S_tail, lr_tps(kvh)};
  const int s = tail ? sp.sb + (x - a.lr_body_all - kvh * a.S_tail) : x - lr_first(kvh);
  if (a.k_new) fused_append_lr(a, sp, b, kvh, s, tail, lds);
  if (tail) {
    if (a.k.tail_bf16) run_tail<HG, true>(a, sp, b, kvh, hg, s, lds);
    else run_tail<HG, false>(a, sp, b, kvh, hg, s, lds);
  } else {
    const int codec = lr_codec(kvh), rank = lr_rank(kvh);
#define KVQ_LR_DISPATCH(CC, RR)                                                           \
    if (codec == CC && rank == RR) run_body<Cfg<HG, CC, CC, RR, RR>, true>(a, sp, b, kvh, hg, s, lds); else
    KVQ_LR_CASES(KVQ_LR_DISPATCH) {}
#undef KVQ_LR_DISPATCH
  }
  finish_split(a, sp, b, kvh, hg, lds);
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

// ev0/ev1 (may be null): events stamped with the split-K kernel's own start
// and end (hipExtLaunchKernel), for timing without extra stream markers.
template <int HG>
hipError_t launch_decode_hg(const DecodeArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid((unsigned)(a.S_body + a.S_tail), (unsigned)(a.Hkv * a.NHG), (unsigned)a.B);
  if (a.k.basis == KVQ_BASIS_LOWRANK) {
    const dim3 lgrid((unsigned)(a.lr_body_all + a.Hkv * a.S_tail), (unsigned)a.NHG, (unsigned)a.B);
    hipExtLaunchKernelGGL(decode_lowrank_kernel<HG>, lgrid, dim3(WG), 0, st, ev0, ev1, 0, a);
    return hipGetLastError();
  }
  const int kc = a.k.codec, vc = a.v.codec;
#define KVQ_LAUNCH_PAIR(K, V)                                                               \
  if (kc == K && vc == V) {                                                                 \
    hipExtLaunchKernelGGL((decode_kernel<HG, K, V>), grid, dim3(WG), 0, st, ev0, ev1, 0, a); \
    return hipGetLastError();                                                               \
  }
  KVQ_DECODE_PAIRS(KVQ_LAUNCH_PAIR)
#undef KVQ_LAUNCH_PAIR
  return hipErrorNotSupported;
}

}  // namespace kvq
