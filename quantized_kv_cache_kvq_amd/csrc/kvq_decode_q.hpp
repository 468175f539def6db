// Quantised-body attention of one wave over its 64-token tiles, with the
// QK product on the integer matrix cores.  Included by kvq_decode_impl.hpp
// inside namespace kvq.
//
// QK (v_mfma_i32_16x16x32_i8).  The B operand is 16 tokens x 32 channels of
// codes as bytes: 8-bit codes straight from memory, narrower codes expanded
// in registers to offset-binary bytes.  The A operand holds the query as
// exact integers: per head, q * 2^sh is rounded to an integer |qi| < 2^20
// and written in three signed base-128 digits (one A row each), so every
// product and sum is exact and the three partial results recombine as
// c0 * 2^14 + c1 * 2^7 + c2.  Rows 4h + s = (head h, digit s); each 16-lane
// row of the result then belongs to one head.  Block scales, code offsets
// and _1 minima are applied to the integer block sums:
//   s = 2^-sh * sum_j [ d_j (C_j + beta Q_j) + m_j Q_j ],  Q_j = sum of qi
// over block j.  The query is rounded to ~21 significant bits relative to its
// largest component (the binary32 input has 24).
//
// Softmax: online, per 16-lane row (= per head), in the log2 domain.
//
// PV (v_mfma_f32_16x16x32_f16): A = weights p * d_j (value block scale)
// as binary16 hi + lo rows, staged in LDS by the lanes that computed p and
// read back transposed; B = value codes staged as offset-binary bytes and
// read with the transposing byte load.  Weights are scaled by 2^(28 - E_j),
// E_j the largest binary16 exponent of block j's scales in the tile, so the
// binary16 parts stay normal; the factor is undone on the fp32 result.
#pragma once

// Channel (0..7) held by byte e after expanding one 8-channel group of
// B-bit codes to bytes.
template <int B>
__host__ __device__ constexpr int grp8_perm(int e) {
  return B == 4 ? (e < 4 ? 2 * e : 2 * (e - 4) + 1)
       : B == 2 ? (e < 4 ? (e == 0 ? 0 : e == 1 ? 4 : e == 2 ? 2 : 6)
                         : (e == 4 ? 1 : e == 5 ? 5 : e == 6 ? 3 : 7))
       : e;
}

// Channel held by staged value byte `pos` of a row.  2-bit rows are staged
// a 32-bit word (16 codes, code i at bits 2i) at a time: byte 4k + i of the
// word's 16 bytes holds code 4i + k, so the four bytes of (w >> 2k) &
// 0x03030303 go out as one word.  Other widths: 8-channel groups,
// grp8_perm.
template <int B>
__host__ __device__ constexpr int vstage_ch(int pos) {
  return B == 2 ? 16 * (pos >> 4) + 4 * (pos & 3) + ((pos >> 2) & 3)
                : 8 * (pos >> 3) + grp8_perm<B>(pos & 7);
}

// vstage_ch is a permutation of a 128-channel row for every width.
template <int B>
constexpr bool vstage_is_permutation() {
  bool seen[128] = {};
  for (int pos = 0; pos < 128; ++pos) {
    const int ch = vstage_ch<B>(pos);
    if (ch < 0 || ch >= 128 || seen[ch]) return false;
    seen[ch] = true;
  }
  return true;
}
static_assert(vstage_is_permutation<1>() && vstage_is_permutation<2>() && vstage_is_permutation<3>() &&
                  vstage_is_permutation<4>() && vstage_is_permutation<5>() && vstage_is_permutation<6>() &&
                  vstage_is_permutation<8>(),
              "staged value bytes map one to one onto channels");

// Four B-bit codes (LSB first in the low 4*B bits of v; higher bits are
// ignored) spread to the four bytes of a word, code i in byte i: codes 2, 3
// move up to bit 16, then codes 1, 3 up by 8 - B.
template <int B>
__device__ __forceinline__ uint32_t spread4(uint32_t v) {
  constexpr uint32_t m2 = (1u << (2 * B)) - 1u;
  const uint32_t t = (v & m2) | ((v & (m2 << (2 * B))) << (16 - 2 * B));
  constexpr uint32_t m1 = ((1u << B) - 1u) * 0x10001u;
  return (t & m1) | ((t & (m1 << B)) << (8 - B));
}

// 8 codes of one group (LSB first in the low 8*B bits of w) as offset-binary
// bytes u (u = c + 2^(B-1) for _0 codes, u = c for _1 codes); byte e holds
// channel grp8_perm<B>(e).  8-bit codes are returned as stored.
template <int B, int FAM>
__device__ __forceinline__ uint2 group_bytes(uint64_t w) {
  if constexpr (B == 8) {
    return make_uint2((uint32_t)w, (uint32_t)(w >> 32));
  } else if constexpr (B == 4) {
    const uint32_t x = (uint32_t)w ^ (FAM == FAM_0 ? 0x88888888u : 0u);
    return make_uint2(x & 0x0F0F0F0Fu, (x >> 4) & 0x0F0F0F0Fu);
  } else if constexpr (B == 2) {
    const uint32_t x = ((uint32_t)w & 0xFFFFu) ^ (FAM == FAM_0 ? 0xAAAAu : 0u);
    const uint32_t e4 = x & 0x3333u, o4 = (x >> 2) & 0x3333u;   // codes 0,2,4,6 / 1,3,5,7
    return make_uint2((e4 | (e4 << 12)) & 0x0F0F0F0Fu, (o4 | (o4 << 12)) & 0x0F0F0F0Fu);
  } else if constexpr (B == 1) {
    const uint32_t x = (uint32_t)w & 0xFFu;
    return make_uint2(__umul24(x & 0xFu, 0x00204081u) & 0x01010101u,
                      __umul24(x >> 4, 0x00204081u) & 0x01010101u);
  } else {
    // 3, 5, 6 bits: codes 0-3 and 4-7 spread separately (bits of w above
    // 8*B are ignored)
    uint64_t sgn = 0;
    if constexpr (FAM == FAM_0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sgn |= (uint64_t)1 << (B * i + B - 1);
    }
    const uint64_t x = w ^ sgn;
    return make_uint2(spread4<B>((uint32_t)x), spread4<B>((uint32_t)(x >> (4 * B))));
  }
}

// Constants of the integer-QK path for a configuration.
template <class C>
struct QCfg {
  static constexpr int HG = C::HG, NK = C::NK, NV = C::NV;
  static constexpr int KB = C::KBITS, VB = C::VBITS;
  static constexpr int TT = 64, NT = 4, NCH = 2;
  static constexpr int HGRP = (HG + 3) / 4;            // 4-head row groups
  static constexpr int NKB = NK < 32 ? 1 : NK / 32;    // 32-channel QK k-blocks
  static constexpr int LK = block_len(NK);
  static constexpr int NBK = NK / LK;                  // K scale blocks (== NKB)
  static constexpr int LV = block_len(NV);
  static constexpr int NBV = NV / LV;                  // V scale blocks
  static constexpr int NDT = NV < 16 ? 1 : NV / 16;    // 16-channel PV tiles
  static constexpr int DPB = LV / 16;                  // PV tiles per V block
  static constexpr int RK = C::RK, CK = C::CK, RV = C::RV, CV = C::CV;
  // stored code = byte + KBIAS (the K operand bytes)
  static constexpr int KBIAS = C::KFAM == FAM_0 ? (KB == 8 ? 0 : -(1 << (KB - 1))) : (KB == 8 ? 128 : 0);
  static constexpr float VOFF = C::VFAM == FAM_0 ? (float)(1 << (VB - 1)) : 0.f;
  // Value codes of at most 4 bits (u <= 15) reach the PV matrix cores as
  // binary16 u through the fp8 (E4M3) conversion, exact for bytes below 16
  // once scaled by 2^9; a _0 code's offset then moves to a per-block term
  // -VOFF * sum_t p_t d_t, accumulated like the _1 minima.
  static constexpr bool VCVT = VB <= 4;
  static constexpr bool VMIN = C::VFAM == FAM_1 || (VCVT && C::VFAM == FAM_0);
  static constexpr float VMINF = C::VFAM == FAM_1 ? 1.f : -VOFF;
  static constexpr int VPITCH = NV + 16;               // staged value row (bytes)
  static constexpr int W_V = TT * VPITCH;
  static constexpr int W_A = NBV * TT * 32;            // [j][t][16 rows] binary16
  static constexpr int W_BYTES = (W_V + W_A + 15) / 16 * 16;
  // query operands shared by the workgroup's waves: digit rows
  // [HGRP][NKB][64 lanes][8 bytes], then 2^-sh [8] and block sums [8][4]
  static constexpr int QD_OFF = NWAVE * W_BYTES;
  static constexpr int QD_BYTES = HGRP * NKB * 64 * 8 + (8 + 8 * 4) * 4;
  static constexpr int MERGE = NWAVE * HG * (NV + 4) * 4;
  static constexpr int LDS_BYTES = cmax<QD_OFF + QD_BYTES, MERGE>::value;
  static_assert(NKB == NBK, "QK k-blocks are scale blocks");
  static_assert(KB == 1 || KB == 2 || KB == 4 || KB == 8 || KB == 3 || KB == 5 || KB == 6, "bits");
};

// Packed 16-bit unsigned max across the 16 lanes of a DPP row.
__device__ __forceinline__ uint32_t row_max_u16x2(uint32_t x) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
#define KVQ_STEP(ctrl)                                                                          \
  x = __builtin_bit_cast(uint32_t,                                                              \
                         __builtin_elementwise_max(__builtin_bit_cast(us2, x),                  \
                                                   __builtin_bit_cast(us2, (uint32_t)__builtin_amdgcn_update_dpp( \
                                                       0, (int)x, ctrl, 0xF, 0xF, true))));
  KVQ_STEP(0x128) KVQ_STEP(0x124) KVQ_STEP(0x122) KVQ_STEP(0x121)
#undef KVQ_STEP
  return x;
}

// Raw codes of the 8-channel group (k-block j, lane group g) of a token at
// in-tile position tok: the low 8*B bits of the result.
template <class Q>
__device__ __forceinline__ uint64_t kq_load(const uint8_t *__restrict__ tile, int tok, int j, int g) {
  constexpr int B = Q::KB, CK = Q::CK;
  // Every lane loads: a group past the row (rank 16 has two groups per
  // token) reads the row's first group and is zeroed by a select.  A load
  // skipped by a branch would make the compiler wait for every load in
  // flight, the prefetched tile included, before the branches join.
  const bool live = 32 * j + 8 * g < Q::NK;
  const int c0 = live ? 32 * j + 8 * g : 0;
  const int b0 = c0 * B / 8;
  uint64_t w;
  if constexpr (B == 8 || B == 4 || B == 2 || B == 1) {
    const uint8_t *p = tile + (unsigned)((b0 / CK) * (TILE * CK) + tok * CK + b0 % CK);
    if constexpr (B == 8) {
      const u32x2 v = ld_stream<u32x2>(p);
      w = (uint64_t)v.x | ((uint64_t)v.y << 32);
    } else if constexpr (B == 4) {
      w = ld_stream<uint32_t>(p);
    } else if constexpr (B == 2) {
      w = ld_stream<uint16_t>(p);
    } else {
      w = ld_stream<uint8_t>(p);
    }
  } else if constexpr (CK >= 4) {
    // the two aligned words around the group's B bytes (a word never
    // straddles a chunk; the second is clamped into the row when the group
    // ends inside the first), then a byte funnel shift
    const int q0 = b0 & ~3, sh = b0 & 3;
    const int q1 = q0 + 4 < Q::RK ? q0 + 4 : Q::RK - 4;
    const uint32_t d0 = ld_stream<uint32_t>(tile + (unsigned)((q0 / CK) * (TILE * CK) + tok * CK + q0 % CK));
    const uint32_t d1 = ld_stream<uint32_t>(tile + (unsigned)((q1 / CK) * (TILE * CK) + tok * CK + q1 % CK));
    const uint32_t lo = __builtin_amdgcn_alignbyte(d1, d0, (uint32_t)sh);
    w = (uint64_t)lo | ((uint64_t)(d1 >> (8 * sh)) << 32);
  } else {
    w = 0;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int b = b0 + i;
      w |= (uint64_t)ld_stream<uint8_t>(tile + (unsigned)((b / CK) * (TILE * CK) + tok * CK + b % CK))
           << (8 * i);
    }
  }
  return live ? w : 0;
}

// QL: the group's query rows sit at the start of LDS, already in the log2
// domain (low-rank bodies project them there); else io.q (raw, rotated here
// when io.rot_w is set).
template <class C, bool QL>
__device__ void attend_q(const SplitIO &io, uint8_t *lds) {
  using Q = QCfg<C>;
  constexpr int HG = Q::HG, TT = Q::TT, NT = Q::NT, NKB = Q::NKB, NBV = Q::NBV, NDT = Q::NDT;
  constexpr int HGRP = Q::HGRP, KB = Q::KB, VB = Q::VB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
  const int n = lane & 15, g = lane >> 4;
  uint8_t *wl = lds + wave * Q::W_BYTES;
  uint8_t *vlds = wl;                                              // [TT][VPITCH]
  uint8_t *alds = wl + Q::W_V;                                     // [NBV][TT][16] f16

  // run-time tiles: every wave takes its first tile by index, then claims
  // the next unclaimed one from a workgroup counter each time it starts a
  // tile, so waves whose data arrive first take more tiles (the counter is
  // set while the waves still enter together)
  __shared__ int tile_ctr;
  if (io.dyn) {
    if (tid == 0) tile_ctr = 0;
    __syncthreads();
  }

  // The query operands are prepared once per workgroup by HGRP producer
  // waves (wave rg handles row group rg: lane = (head 4rg + lane/16, 8-channel
  // group lane%16)) and shared through LDS; the other waves only issue their
  // tile loads and wait at one barrier.  The producers' query loads go out
  // before their tile loads.
  const bool producer = wave < HGRP;
  const int ph = 4 * wave + (lane >> 4), pG = lane & 15;   // producer: head, channel group
  float qv[8];
  if (producer && ph < HG && 8 * pG < Q::NK) {
    float4 x0, x1;
    if constexpr (QL) {
      x0 = reinterpret_cast<const float4 *>(lds)[(ph * D + 8 * pG) / 4];
      x1 = reinterpret_cast<const float4 *>(lds)[(ph * D + 8 * pG + 4) / 4];
    } else {
      x0 = *reinterpret_cast<const float4 *>(io.q + (unsigned)(ph * D + 8 * pG));
      x1 = *reinterpret_cast<const float4 *>(io.q + (unsigned)(ph * D + 8 * pG + 4));
    }
    qv[0] = x0.x; qv[1] = x0.y; qv[2] = x0.z; qv[3] = x0.w;
    qv[4] = x1.x; qv[5] = x1.y; qv[6] = x1.z; qv[7] = x1.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = 0.f;
  }

  // ---- tiles of this wave: t_begin / TT + wave, then every NWAVE-th (or,
  // for long splits, the ones it claims; tile indices: the loop carries the
  // tile index, which keeps fewer values live than a token counter); 32-bit
  // in-plane offsets; tokens past t_end load token t_end - 1 (masked later)
  const int t_end = (int)io.t_end;
  const int lim_tiles = (t_end + TT - 1) / TT;
  const int tile0 = (int)(io.t_begin / TT);
  int cur = tile0 + wave;

  uint64_t kr[NT][NKB];
  uint2 ksr[NT], kmr[NT], vsr[NT], vmr[NT];
  constexpr int VW = (Q::RV + 3) / 4;
  uint32_t vw[VW];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) ksr[nt] = kmr[nt] = vsr[nt] = vmr[nt] = make_uint2(0u, 0u);

  auto side = [&](const uint16_t *base, int t, int nb) -> uint2 {
    const uint16_t *p = base + (unsigned)(t * nb);
    if (nb == 4) {
      const u32x2 v = ld_stream<u32x2>(p);
      return make_uint2(v.x, v.y);
    }
    if (nb == 2) return make_uint2(ld_stream<uint32_t>(p), 0u);
    return make_uint2((uint32_t)ld_stream<uint16_t>(p), 0u);
  };
  // lim: last valid in-tile position (0 for the dummy prefetch after the
  // last tile, which then reads one line per chunk, an L2 hit)
  auto load_k_nt = [&](int t0, int lim, int nt) {
    const int tok = min(16 * nt + n, lim);
    const uint8_t *tile = io.kcodes + (unsigned)t0 * Q::RK;
#pragma unroll
    for (int j = 0; j < NKB; ++j) kr[nt][j] = kq_load<Q>(tile, tok, j, g);
    ksr[nt] = side(io.ksc, t0 + tok, Q::NBK);
    if constexpr (C::KFAM == FAM_1) kmr[nt] = side(io.kmn, t0 + tok, Q::NBK);
    vsr[nt] = side(io.vsc, t0 + tok, NBV);
    if constexpr (C::VFAM == FAM_1) vmr[nt] = side(io.vmn, t0 + tok, NBV);
  };
  auto load_v = [&](int t0, int lim) {
    const int tok = min(lane, lim);
    const uint8_t *tile = io.vcodes + (unsigned)t0 * Q::RV;
    constexpr int CV = Q::CV, NCV = Q::RV / CV;
#pragma unroll
    for (int k = 0; k < NCV; ++k) {
      const uint8_t *p = tile + (unsigned)(k * (TILE * CV) + tok * CV);
      if constexpr (CV == 16) {
        const u32x4 x = ld_stream<u32x4>(p);
        vw[4 * k] = x.x; vw[4 * k + 1] = x.y; vw[4 * k + 2] = x.z; vw[4 * k + 3] = x.w;
      } else if constexpr (CV == 8) {
        const u32x2 x = ld_stream<u32x2>(p);
        vw[2 * k] = x.x; vw[2 * k + 1] = x.y;
      } else if constexpr (CV == 4) {
        vw[k] = ld_stream<uint32_t>(p);
      } else if constexpr (CV == 2) {
        const uint32_t x = ld_stream<uint16_t>(p);
        if (k & 1) vw[k / 2] |= x << 16; else vw[k / 2] = x;
      } else {
        const uint32_t x = ld_stream<uint8_t>(p);
        if (k & 3) vw[k / 4] |= x << (8 * (k & 3)); else vw[k / 4] = x;
      }
    }
  };

  // The first tile's loads go out before the query work below.  Loads are
  // unconditional (a wave without tiles, and the prefetch after the last
  // tile, read only token 0 of a valid tile), so the
  // compiler can count outstanding loads exactly and never has to drain
  // the prefetched tile early.
  {
    const int lt0 = cur < lim_tiles ? cur * TT : (int)io.t_begin;
    const int lim0 = cur < lim_tiles ? t_end - 1 - lt0 : 0;
    load_v(lt0, lim0);                 // the loop's prefetch order, so waits count exactly
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) load_k_nt(lt0, lim0, nt);
  }
  __builtin_amdgcn_sched_barrier(0);    // keep the tile loads ahead of the query work

  // ---- query digits.  A row n of group rg = (head 4rg + n/4, digit n%4):
  // per head, q * 2^sh (|q * 2^sh| < 2^20) rounded to an integer and written
  // as three signed base-128 digits; byte e of k-group g in block j holds
  // channel 32j + 8g + grp8_perm(e).  A producer lane computes all digit
  // rows of its (head, 8-channel group); the head's amax is a reduction over
  // its 16-lane row.
  uint64_t *qd = reinterpret_cast<uint64_t *>(lds + Q::QD_OFF);
  float *qinv_s = reinterpret_cast<float *>(lds + Q::QD_OFF + HGRP * NKB * 64 * 8);
  float *qsum_s = qinv_s + 8;
  if (producer) {
    const int hh = lane >> 4, j = pG >> 2, gk = pG & 3;
    float v[8];
    float amax = 0.f;
    if (!QL && io.rot_w) rotate_row8(qv, io.rot_w, pG);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = QL ? qv[grp8_perm<KB>(e)] : qv[grp8_perm<KB>(e)] * io.scale;
      amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = row_max16(amax);
    int ex = 0;
    if (amax > 0.f) (void)frexpf(amax, &ex);
    const int sh = 20 - ex;                         // |q * 2^sh| < 2^20
    uint32_t w[3][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}};
    int qs = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int qi = (int)rintf(ldexpf(v[e], sh));
      const int d2 = ((qi + 64) & 127) - 64;
      const int r = (qi - d2) >> 7;
      const int d1 = ((r + 64) & 127) - 64;
      const int d0 = (r - d1) >> 7;
      w[0][e >> 2] |= (uint32_t)(d0 & 0xFF) << (8 * (e & 3));
      w[1][e >> 2] |= (uint32_t)(d1 & 0xFF) << (8 * (e & 3));
      w[2][e >> 2] |= (uint32_t)(d2 & 0xFF) << (8 * (e & 3));
      qs += qi;
    }
    // block sum over the 4 channel groups of block j (lanes 4j .. 4j+3 of the row)
    qs += __shfl_xor(qs, 1, 64);
    qs += __shfl_xor(qs, 2, 64);
    if (j < NKB) {
      uint64_t *dst = qd + ((wave * NKB + j) * 64 + 4 * hh + 16 * gk);
#pragma unroll
      for (int dg = 0; dg < 3; ++dg) dst[dg] = (uint64_t)w[dg][0] | ((uint64_t)w[dg][1] << 32);
      dst[3] = 0ull;
      if (gk == 0 && ph < HG) qsum_s[ph * 4 + j] = (float)qs;
      if (pG == 0 && ph < HG) qinv_s[ph] = ldexpf(1.f, -sh);
    }
  }
  __syncthreads();
  // lane (n, g) of the QK result holds head g + 4rg
  long qA[HGRP][NKB];
  float inv[HGRP], Qb[HGRP][NKB], Qm[HGRP][NKB];
#pragma unroll
  for (int rg = 0; rg < HGRP; ++rg) {
    const bool live = g + 4 * rg < HG;
    inv[rg] = live ? qinv_s[g + 4 * rg] : 0.f;
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
      qA[rg][j] = (long)qd[(rg * NKB + j) * 64 + lane];
      const float qsv = live ? qsum_s[(g + 4 * rg) * 4 + j] : 0.f;
      Qb[rg][j] = (float)Q::KBIAS * qsv;
      Qm[rg][j] = qsv;
    }
  }
  for (int i = lane; i < Q::W_A / 16; i += 64)
    reinterpret_cast<uint4 *>(alds)[i] = make_uint4(0u, 0u, 0u, 0u);

  float m_run[HGRP], l_lane[HGRP], pm[HGRP][NBV], O[HGRP][NDT];
#pragma unroll
  for (int rg = 0; rg < HGRP; ++rg) {
    m_run[rg] = NEG_INF;
    l_lane[rg] = 0.f;
#pragma unroll
    for (int j = 0; j < NBV; ++j) pm[rg][j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[rg][dt] = 0.f;
  }

  while (cur < lim_tiles) {
    int nxt = cur + NWAVE;
    if (io.dyn) {
      int claim = 0;
      if (lane == 0)
        claim = __hip_atomic_fetch_add(&tile_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      nxt = tile0 + NWAVE + __builtin_amdgcn_readfirstlane(claim);
    }
    const bool more = nxt < lim_tiles;
    const int t0 = cur * TT;
    const int tn = more ? nxt * TT : t0;               // prefetch target
    const int limn = more ? t_end - 1 - tn : 0;
    const int lim = t_end - 1 - t0;

    // ---- value row of token `lane` into LDS as offset-binary bytes; byte
    // pos holds channel vstage_ch<VB>(pos)
    if constexpr (VB == 2) {
      uint8_t *dst = vlds + lane * Q::VPITCH;
#pragma unroll
      for (int m = 0; m < Q::NV / 16; ++m) {
        const uint32_t x = vw[m] ^ (C::VFAM == FAM_0 ? 0xAAAAAAAAu : 0u);
        *reinterpret_cast<uint4 *>(dst + 16 * m) =
            make_uint4(x & 0x03030303u, (x >> 2) & 0x03030303u, (x >> 4) & 0x03030303u, (x >> 6) & 0x03030303u);
      }
    } else {
      uint8_t *dst = vlds + lane * Q::VPITCH;
#pragma unroll
      for (int G = 0; G < Q::NV / 8; ++G) {
        uint64_t w;
        if constexpr (VB == 8) {
          w = (uint64_t)vw[2 * G] | ((uint64_t)vw[2 * G + 1] << 32);
        } else if constexpr (VB == 4) {
          w = vw[G];
        } else if constexpr (VB == 2) {
          w = (vw[G / 2] >> (16 * (G & 1))) & 0xFFFFu;
        } else if constexpr (VB == 1) {
          w = (vw[G / 4] >> (8 * (G & 3))) & 0xFFu;
        } else {
          // VB bytes starting at byte VB * G of the row: funnel shifts over
          // the (at most three) words they touch, on named words (a 64-bit
          // read across the word array kept it in scratch for 5 and 6 bits)
          const int bit = 8 * VB * G;
          const int wi = bit >> 5, sh = bit & 31;
          const uint32_t w0 = vw[wi];
          const uint32_t w1 = wi + 1 < VW ? vw[wi + 1] : 0u;
          const uint32_t w2 = wi + 2 < VW ? vw[wi + 2] : 0u;
          const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, (uint32_t)sh);
          const uint32_t hi = __builtin_amdgcn_alignbit(w2, w1, (uint32_t)sh);
          w = (uint64_t)lo | ((uint64_t)hi << 32);
        }
        uint2 b = group_bytes<VB, C::VFAM>(w);
        if constexpr (VB == 8 && C::VFAM == FAM_0) { b.x ^= 0x80808080u; b.y ^= 0x80808080u; }
        *reinterpret_cast<uint2 *>(dst + 8 * G) = b;
      }
    }
    uint2 vs_cur[NT], vm_cur[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) { vs_cur[nt] = vsr[nt]; vm_cur[nt] = vmr[nt]; }
    load_v(tn, limn);

    // ---- QK on the integer matrix cores
    float sc[HGRP][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float dk[4] = {1.f, 1.f, 1.f, 1.f}, mk[4] = {0.f, 0.f, 0.f, 0.f};
      unpack_side(ksr[nt], dk, Q::NBK);
      if constexpr (C::KFAM == FAM_1) unpack_side(kmr[nt], mk, Q::NBK);
      long kb[NKB];
#pragma unroll
      for (int j = 0; j < NKB; ++j) {
        const uint2 b = group_bytes<KB, C::KFAM>(kr[nt][j]);
        uint2 bb = b;
        if constexpr (KB == 8 && C::KFAM == FAM_1) { bb.x ^= 0x80808080u; bb.y ^= 0x80808080u; }
        kb[j] = (long)((uint64_t)bb.x | ((uint64_t)bb.y << 32));
      }
      // the N-tile's matrix ops read its codes before the next tile's loads
      // reuse their registers (loads issued first would land in other
      // registers, copied back at the end of every tile)
      typedef int intx4 __attribute__((ext_vector_type(4)));
      intx4 cq[HGRP][NKB];
#pragma unroll
      for (int rg = 0; rg < HGRP; ++rg)
#pragma unroll
        for (int j = 0; j < NKB; ++j)
          cq[rg][j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(qA[rg][j], kb[j], intx4{0, 0, 0, 0}, 0, 0, 0);
      load_k_nt(tn, limn, nt);          // N-tile nt's registers are free again
      const bool valid = 16 * nt + n <= lim;
#pragma unroll
      for (int rg = 0; rg < HGRP; ++rg) {
        // (summing from zero keeps the masked select below a branch the
        // compiler skips for absent heads; starting from the first block's
        // product instead made the six-head decode 4% slower)
        float a1 = 0.f, a2 = 0.f;
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
          const intx4 c = cq[rg][j];
          float f = fmaf((float)c[0], 16384.f, (float)(c[1] * 128 + c[2]));
          if constexpr (Q::KBIAS != 0) f += Qb[rg][j];
          a1 = fmaf(dk[j], f, a1);
          if constexpr (C::KFAM == FAM_1) a2 = fmaf(mk[j], Qm[rg][j], a2);
        }
        sc[rg][nt] = (valid && g + 4 * rg < HG) ? (a1 + a2) * inv[rg] : NEG_INF;
      }
    }

    // ---- online softmax, one head per 16-lane row
    float alpha[HGRP], p[HGRP][NT];
#pragma unroll
    for (int rg = 0; rg < HGRP; ++rg) {
      float mx = sc[rg][0];
#pragma unroll
      for (int nt = 1; nt < NT; ++nt) mx = fmaxf(mx, sc[rg][nt]);
      mx = row_max16(mx);
      const float mnew = __builtin_elementwise_maximum(m_run[rg], mx);   // no NaN: IEEE maximum, no canonicalisation
      alpha[rg] = m_run[rg] == NEG_INF ? (mnew == NEG_INF ? 1.f : 0.f) : __builtin_amdgcn_exp2f(m_run[rg] - mnew);
      m_run[rg] = mnew;
      float ps = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        p[rg][nt] = mnew == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(sc[rg][nt] - mnew);
        ps += p[rg][nt];
      }
      l_lane[rg] = fmaf(l_lane[rg], alpha[rg], ps);
      if constexpr (C::VFAM != FAM_1 && Q::VMIN) {
#pragma unroll
        for (int j = 0; j < NBV; ++j) pm[rg][j] *= alpha[rg];
      }
      if constexpr (C::VFAM == FAM_1) {
#pragma unroll
        for (int j = 0; j < NBV; ++j) {
          float acc = pm[rg][j] * alpha[rg];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            float mv[4] = {0.f, 0.f, 0.f, 0.f};
            unpack_side(vm_cur[nt], mv, NBV);
            acc = fmaf(p[rg][nt], mv[j], acc);
          }
          pm[rg][j] = acc;
        }
      }
    }

    // ---- weights x = p * dv_j * 2^(28 - E_j) as (hi, lo) binary16 rows
    // 4g + 2rg, 4g + 2rg + 1 of token 16nt + n
    float back[NBV];
    {
      uint32_t e01 = 0u, e23 = 0u;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        typedef unsigned short us2 __attribute__((ext_vector_type(2)));
        e01 = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, e01),
                  __builtin_bit_cast(us2, vs_cur[nt].x & 0x7C007C00u)));
        if (NBV > 2)
          e23 = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, e23),
                    __builtin_bit_cast(us2, vs_cur[nt].y & 0x7C007C00u)));
      }
      e01 = row_max_u16x2(e01);
      if (NBV > 2) e23 = row_max_u16x2(e23);
      float fwd[4];
#pragma unroll
      for (int j = 0; j < NBV; ++j) {
        const uint32_t word = j < 2 ? e01 : e23;
        int E = (int)((word >> (16 * (j & 1) + 10)) & 31u);
        E = E < 1 ? 1 : E;
        fwd[j] = __builtin_bit_cast(float, (uint32_t)(28 - E + 127) << 23);
        back[j] = __builtin_bit_cast(float, (uint32_t)(E - 28 + 127) << 23);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float dv[4] = {1.f, 1.f, 1.f, 1.f};
        unpack_side(vs_cur[nt], dv, NBV);
#pragma unroll
        for (int j = 0; j < NBV; ++j) {
          const float scl = dv[j] * fwd[j];
          uint32_t *dst = reinterpret_cast<uint32_t *>(alds + ((j * TT) + 16 * nt + n) * 32 + 8 * g);
#pragma unroll
          for (int rg = 0; rg < HGRP; ++rg) {
            if constexpr (C::VFAM != FAM_1 && Q::VMIN) pm[rg][j] = fmaf(p[rg][nt], dv[j], pm[rg][j]);
            const float x = p[rg][nt] * scl;
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
            h2 hl;
            hl.x = (_Float16)x;                                   // hi
            hl.y = (_Float16)(x - (float)hl.x);                   // lo, into the upper half
            dst[rg] = __builtin_bit_cast(uint32_t, hl);
          }
        }
      }
    }
    wave_sync_lds();

    // ---- PV on the matrix cores: A = weights [16 rows][32 tokens], B = values
    floatx4 ct[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) ct[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < Q::NCH; ++kc) {
      const int tok = 32 * kc + 8 * g;
#pragma unroll
      for (int j = 0; j < NBV; ++j) {
        const uint8_t *pa = alds + ((j * TT) + tok + (n >> 2)) * 32 + 8 * (n & 3);
        const half8 a = tr16_pair(pa, pa + 4 * 32);
#pragma unroll
        for (int d = 0; d < Q::DPB; ++d) {
          const int dt = j * Q::DPB + d;
          const uint8_t *pb = vlds + (tok + (n >> 1)) * Q::VPITCH + 16 * dt + 8 * (n & 1);
          half8 bv;
          if constexpr (Q::VCVT) bv = small_bytes_to_half8(tr8(pb));
          else bv = bytes_to_half8(tr8(pb), Q::VOFF);
          ct[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bv, ct[dt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float bk = back[dt / Q::DPB];
#pragma unroll
      for (int rg = 0; rg < HGRP; ++rg)
        O[rg][dt] = fmaf(O[rg][dt], alpha[rg], (ct[dt][2 * rg] + ct[dt][2 * rg + 1]) * bk);
    }
    wave_sync_lds();                    // LDS tiles are free for the next tile
    cur = nxt;
  }

  // ---- close this wave: l and pm over the row's 16 lanes
  float lsum[HGRP], pmsum[HGRP][NBV];
#pragma unroll
  for (int rg = 0; rg < HGRP; ++rg) {
    lsum[rg] = row_sum16(l_lane[rg]);
#pragma unroll
    for (int j = 0; j < NBV; ++j) pmsum[rg][j] = Q::VMIN ? Q::VMINF * row_sum16(pm[rg][j]) : 0.f;
  }
  float *mw = merge_slots();
#pragma unroll
  for (int rg = 0; rg < HGRP; ++rg)
    if (g + 4 * rg < HG && n == 0) mw[wave * 8 + g + 4 * rg] = m_run[rg];
  __syncthreads();   // every wave is done with its LDS tiles; wave maxima published

  // merge area: [wave][h][4 + NV]: -, l, -, -, o[NV] (raw channel order),
  // scaled to the workgroup maximum
  float *mg = reinterpret_cast<float *>(lds);
  constexpr int MS = Q::NV + 4;
#pragma unroll
  for (int rg = 0; rg < HGRP; ++rg) {
    const int h = g + 4 * rg;
    if (h < HG) {
      const float f = merge_scale(mw, h, m_run[rg]);
      float *dst = mg + (wave * HG + h) * MS;
      if (n == 0) dst[1] = lsum[rg] * f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int pos = 16 * dt + n;                       // staged byte position
        if (pos < Q::NV) {
          const int ch = vstage_ch<VB>(pos);
          float o = O[rg][dt];
          if constexpr (Q::VMIN) o += pmsum[rg][pos / Q::LV];
          dst[4 + ch] = o * f;
        }
      }
    }
  }
  __syncthreads();
  merge_store<HG, Q::NV>(mg, mw, io.part, io.part_head_stride);
  // low rank: the channels past the rank are zero, so the combine (which
  // reads all 128 of every split) never meets stale workspace contents
  if constexpr (Q::NV < D) {
    for (int idx = tid; idx < HG * (D - Q::NV); idx += WG) {
      const int h = idx / (D - Q::NV), c = Q::NV + idx % (D - Q::NV);
      store_agent(io.part + h * io.part_head_stride + 4 + c, 0.f);
    }
  }
}
