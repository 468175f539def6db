// Device code shared by the append kernel and the fused append + decode
// launch: DPP row reductions, the in-wave Walsh-Hadamard transform, and the
// store of one token's row of a plain or KVarN plane (tail copy, stored
// coordinates, block scales, codes, bit packing).  Included inside
// namespace kvq.
#pragma once

namespace arow {

// All-reduce over the 16 lanes of a DPP row (lanes 16r .. 16r+15).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f<0x128>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  x = fmaxf(x, dpp_f<0x122>(x));
  return fmaxf(x, dpp_f<0x121>(x));
}
__device__ __forceinline__ float row_min16(float x) {
  x = fminf(x, dpp_f<0x128>(x));
  x = fminf(x, dpp_f<0x124>(x));
  x = fminf(x, dpp_f<0x122>(x));
  return fminf(x, dpp_f<0x121>(x));
}

// In-wave fast Walsh-Hadamard transform of 128 values, lane l holding
// elements 2l (a) and 2l+1 (b).  Butterflies (u+v, u-v) at every stride give
// the Sylvester (natural-order) H applied to the vector.
__device__ inline void fwht128_wave(float &a, float &b) {
  const int lane = threadIdx.x & 63;
  float s = a + b, d = a - b;          // stride 1: inside the lane
  a = s;
  b = d;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {   // stride 2m: partner lane l ^ m
    float pa = __shfl_xor(a, m, 64);
    float pb = __shfl_xor(b, m, 64);
    bool upper = (lane & m) != 0;
    a = upper ? (pa - a) : (a + pa);
    b = upper ? (pb - b) : (b + pb);
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Unsigned all-reduce steps over lanes of a DPP row; with full row and bank
// masks the move folds into the consuming ALU instruction.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t row_umax16(uint32_t x) {
  x = max(x, dpp_u<0x128>(x));
  x = max(x, dpp_u<0x124>(x));
  x = max(x, dpp_u<0x122>(x));
  return max(x, dpp_u<0x121>(x));
}
// OR over each aligned group of K lanes (K = 2, 4, 8, 16), every lane of the
// group receiving it: quad swaps (1 0 3 2, then 2 3 0 1), then the half-row
// and row mirrors, which pair each quad / half with the other.
template <int K>
__device__ __forceinline__ uint32_t group_or(uint32_t w) {
  w |= dpp_u<0xB1>(w);
  if constexpr (K >= 4) w |= dpp_u<0x4E>(w);
  if constexpr (K >= 8) w |= dpp_u<0x141>(w);
  if constexpr (K >= 16) w |= dpp_u<0x140>(w);
  return w;
}

// Per-block scale (and min) and codes of one token whose stored coordinates
// are held two per lane (a = coordinate 2l, c = 2l + 1), for a plain or
// KVarN plane of a fixed codec: blocks of 32 are the 16 lanes of a DPP row,
// so every reduction is a row reduction.  Returns this lane's 2*BITS code
// bits (codes of coordinates 2l, 2l + 1 at bits [0, BITS), [BITS, 2 BITS));
// dh / mh: the binary16 bits of the lane's block scale (and min).  Inputs
// are finite: the block maximum of |x| is taken on the bit patterns.
template <int BITS, int FAM>
__device__ __forceinline__ uint32_t row_fields(float a, float c, uint16_t &dh, uint16_t &mh) {
  float d, m = 0.f;
  if constexpr (FAM == FAM_0) {
    const uint32_t ua = __float_as_uint(a) & 0x7fffffffu, uc = __float_as_uint(c) & 0x7fffffffu;
    const float amax = __uint_as_float(row_umax16(max(ua, uc)));
    constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
    dh = f32_to_f16_bits(amax / qmax);
    mh = 0;
    d = f16_bits_to_f32(dh);
  } else {
    const float lo = row_min16(fminf(a, c)), hi = row_max16(fmaxf(a, c));
    mh = f32_to_f16_bits(lo);
    m = f16_bits_to_f32(mh);
    constexpr float levels = (float)((1 << BITS) - 1);
    dh = f32_to_f16_bits((hi - m) / levels);
    d = f16_bits_to_f32(dh);
  }
  constexpr uint32_t mask = (1u << BITS) - 1u;
  uint32_t q0 = 0, q1 = 0;
  if (d != 0.f) {
    if constexpr (FAM == FAM_0) {
      constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
      q0 = (uint32_t)(int)fminf(fmaxf(rintf(a / d), -qmax), qmax);
      q1 = (uint32_t)(int)fminf(fmaxf(rintf(c / d), -qmax), qmax);
    } else {
      constexpr float levels = (float)((1 << BITS) - 1);
      q0 = (uint32_t)(int)fminf(fmaxf(rintf((a - m) / d), 0.f), levels);
      q1 = (uint32_t)(int)fminf(fmaxf(rintf((c - m) / d), 0.f), levels);
    }
  }
  return (q0 & mask) | ((q1 & mask) << BITS);
}

// The packed row (16 * BITS bytes, this lane's bits at bit 2*BITS*lane) into
// LDS at `row` (dword aligned): 8/4/2/1-bit fields are OR-ed across lanes
// by DPP and written a dword per group of lanes; 3/5/6-bit fields are OR-ed
// into the zeroed row by LDS atomics.  Ends with the row complete in LDS.
template <int BITS>
__device__ __forceinline__ void pack_row_lds(uint32_t v, uint32_t *row) {
  const int lane = threadIdx.x & 63;
  if constexpr (BITS == 8 || BITS == 4 || BITS == 2 || BITS == 1) {
    constexpr int K = 16 / BITS;                   // lanes per dword
    const uint32_t w = group_or<K>(v << (2 * BITS * (lane % K)));
    if (lane % K == 0) row[lane / K] = w;
  } else {
    constexpr int NW = 4 * BITS;                   // dwords of the row
    if (lane < NW) row[lane] = 0u;
    wave_sync();
    const int o = 2 * BITS * lane, k = o >> 5, sh = o & 31;
    __hip_atomic_fetch_or(row + k, v << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (sh + 2 * BITS > 32)
      __hip_atomic_fetch_or(row + k + 1, v >> (32 - sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// Codes, scale (and min) of one row straight to the cache: tile = start of
// the token's 64-token tile in its plane, tt = the token's slot in it, srow
// / mrow = its scale (min) entries; stage: 32 words of this wave's LDS.
// Every lane executes every store (lanes sharing an address store the same
// value), so no store sits on a branch.
template <int BITS, int FAM>
__device__ __forceinline__ void quantize_row_at(uint8_t *tile, int tt, uint16_t *srow, uint16_t *mrow,
                                                float a, float c, uint32_t *stage) {
  constexpr int RB = 16 * BITS;
  constexpr int CK = chunk_bytes(RB);
  const int lane = threadIdx.x & 63;
  uint16_t dh, mh;
  const uint32_t v = row_fields<BITS, FAM>(a, c, dh, mh);
  srow[lane >> 4] = dh;
  if constexpr (FAM == FAM_1) mrow[lane >> 4] = mh;
  if constexpr (BITS == 8 || BITS == 4 || BITS == 2 || BITS == 1) {
    constexpr int K = 16 / BITS;                   // lanes per dword
    const uint32_t w = group_or<K>(v << (2 * BITS * (lane % K)));
    const int byte = 4 * (lane / K);
    *reinterpret_cast<uint32_t *>(tile + ((byte / CK) * TILE + tt) * CK + byte % CK) = w;
  } else {
    constexpr int NW = RB / 4;
    pack_row_lds<BITS>(v, stage);
    wave_sync();
    const int wl = lane % NW;                      // lanes past NW repeat a word
    const int byte = 4 * wl;
    *reinterpret_cast<uint32_t *>(tile + ((byte / CK) * TILE + tt) * CK + byte % CK) = stage[wl];
    wave_sync();                                   // stage is free for the next item
  }
}

// Row of token slot tt of a tile (codec CODEC, plain or KVarN plane; a, c =
// this lane's stored coordinates 2l, 2l + 1).  stage: 32 words of this
// wave's LDS.
template <int CODEC>
__device__ __forceinline__ void store_row_at(uint8_t *tile, int tt, uint16_t *srow, uint16_t *mrow, float a,
                                             float c, uint32_t *stage) {
  const int lane = threadIdx.x & 63;
  if constexpr (CODEC == KVQ_F16) {
    // binary16 row: dword `lane` holds coordinates 2*lane, 2*lane+1
    const uint32_t pair = (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(c) << 16);
    const int byte = 4 * lane;
    *reinterpret_cast<uint32_t *>(tile + ((byte / 16) * TILE + tt) * 16 + byte % 16) = pair;
  } else {
    quantize_row_at<codec_bits(CODEC), codec_family(CODEC)>(tile, tt, srow, mrow, a, c, stage);
  }
}

// Row of token t of codec CODEC in the plane whose rows start at row `rows`
// of the layer's planes.
template <int CODEC, class PA>
__device__ __forceinline__ void store_row(const PA &p, long long rows, int t, float a, float c,
                                          uint32_t *stage) {
  constexpr int RB = row_bytes(CODEC, D);
  constexpr int NB = codec_family(CODEC) == FAM_F16 ? 0 : D / 32;
  uint8_t *tile = p.codes + rows * RB + (long long)(t / TILE) * TILE * RB;
  const long long so = (rows + t) * NB;
  store_row_at<CODEC>(tile, t % TILE, p.scales + so, codec_family(CODEC) == FAM_1 ? p.mins + so : nullptr, a,
                      c, stage);
}

// 16-bit tail copy (binary16 or bfloat16) of raw channels x of token t into
// ring slot t mod tail_len of plane `plane` (= b * hkv + h).
template <class PA>
__device__ __forceinline__ void store_tail(const PA &p, long long plane, int t, float2 x) {
  const int lane = threadIdx.x & 63;
  const int slot = t % p.tail_len;
  const uint32_t pair =
      p.tail_bf16 ? (uint32_t)f32_to_bf16_bits(x.x) | ((uint32_t)f32_to_bf16_bits(x.y) << 16)
                  : (uint32_t)f32_to_f16_bits(x.x) | ((uint32_t)f32_to_f16_bits(x.y) << 16);
  uint8_t *base = reinterpret_cast<uint8_t *>(p.tail) + plane * p.tail_len * (2 * D);
  const int byte = 4 * lane;
  *reinterpret_cast<uint32_t *>(base + tiled_offset(slot, byte / 16, 2 * D, 16) + byte % 16) = pair;
}

// Stored coordinates of raw channels x of kv head h: x itself (plain), or
// H (x * w) by the in-wave transform (KVarN).
template <class PA>
__device__ __forceinline__ void stored_coords(const PA &p, int h, float2 x, float &a, float &c) {
  const int lane = threadIdx.x & 63;
  a = x.x;
  c = x.y;
  if (p.basis == KVQ_BASIS_HADAMARD) {
    const float *w = p.w + (long long)h * D;
    a *= w[2 * lane];
    c *= w[2 * lane + 1];
    fwht128_wave(a, c);
  }
}

// Low-rank stored coordinates of one token: u = P^T x (P: 128 x 128
// binary16, row c = input channel), lane l holding raw channels x = (2l,
// 2l + 1) and getting nothing back: u lands in coords[0 .. 128).  xin,
// coords: 128 floats of this wave's LDS each.  The wave reads all of P in
// one round trip: load i of lane l is row 4i + l/16, columns 8(l%16) .. +8;
// each lane sums its 8 columns over its 32 rows in row order, then the four
// lanes holding the same columns (l, l^16, l^32, l^48) add their sums.
__device__ inline void lr_project_row(const uint16_t *P, float2 x, float *xin, float *coords) {
  const int lane = threadIdx.x & 63;
  xin[2 * lane] = x.x;
  xin[2 * lane + 1] = x.y;
  wave_sync();
  const u32x4 *P4 = reinterpret_cast<const u32x4 *>(P);
  u32x4 pv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) pv[i] = P4[64 * i + lane];
  const int rsub = lane >> 4, c0 = 8 * (lane & 15);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    const float xr = xin[4 * i + rsub];
    const uint32_t wv[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(f16_bits_to_f32((uint16_t)(wv[e] & 0xFFFFu)), xr, acc[2 * e]);
      acc[2 * e + 1] = fmaf(f16_bits_to_f32((uint16_t)(wv[e] >> 16)), xr, acc[2 * e + 1]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] += __shfl_xor(acc[e], 16, 64);
    acc[e] += __shfl_xor(acc[e], 32, 64);
  }
  if (rsub == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) coords[c0 + e] = acc[e];
  }
  wave_sync();
}

// Low-rank row of token t in plane geometry g: lane l holds stored
// coordinates 2l, 2l+1 (v0, v1; lanes past the rank are ignored).  Block
// scale (and min) per block of L = min(32, rank) coordinates, codes, packing
// through pk (this wave's 128 bytes of LDS), store in the tiled layout.
__device__ __forceinline__ void lr_store_row(const PlaneArgs &p, const HeadGeom &g, int t, float v0,
                                             float v1, uint32_t *pk) {
  const int lane = threadIdx.x & 63;
  uint8_t *row_codes = p.codes + g.codes_off;
  const int fam = codec_family(g.codec);
  const int bits = codec_bits(g.codec);
  // lane l holds stored coordinates 2l, 2l+1; block j (L = min(32, rank)
  // coordinates) is lanes [j L/2, (j+1) L/2), reduced by shuffles within
  // those aligned lane groups
  const bool act = 2 * lane < g.n;
  if (!act) v0 = v1 = 0.f;
  const int half = g.L / 2;
  const int j = lane / half, lead = j * half;
  float d = 0.f, m = 0.f;
  if (fam == FAM_0) {
    float amax = fmaxf(fabsf(v0), fabsf(v1));
    for (int o = half / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float qmax = (float)((1 << (bits - 1)) - 1);
    const uint16_t dh = f32_to_f16_bits(amax / qmax);
    if (act && lane == lead) p.scales[g.scales_off + (long long)t * g.nblk + j] = dh;
    d = f16_bits_to_f32(dh);
  } else {
    float lo = act ? fminf(v0, v1) : __builtin_huge_valf(), hi = act ? fmaxf(v0, v1) : -__builtin_huge_valf();
    for (int o = half / 2; o > 0; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o, 64));
      hi = fmaxf(hi, __shfl_xor(hi, o, 64));
    }
    const uint16_t mh = f32_to_f16_bits(lo);
    m = f16_bits_to_f32(mh);
    const float levels = (float)((1 << bits) - 1);
    const uint16_t dh = f32_to_f16_bits((hi - m) / levels);
    if (act && lane == lead) {
      const long long so = g.scales_off + (long long)t * g.nblk + j;
      p.scales[so] = dh;
      p.mins[so] = mh;
    }
    d = f16_bits_to_f32(dh);
  }

  // codes of the lane's two coordinates, OR-ed into the packed row in LDS
  // (code e at bits [e b, e b + b) of the row)
  if (lane < D / 4) pk[lane] = 0u;
  wave_sync();
  if (act) {
    const uint32_t mask = (1u << bits) - 1u;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float x = k ? v1 : v0;
      int q = 0;
      if (fam == FAM_0) {
        const float qmax = (float)((1 << (bits - 1)) - 1);
        if (d != 0.f) q = (int)fminf(fmaxf(rintf(x / d), -qmax), qmax);
      } else {
        const float levels = (float)((1 << bits) - 1);
        const float y = x - m;
        if (d != 0.f) q = (int)fminf(fmaxf(rintf(y / d), 0.f), levels);
      }
      const uint32_t v = (uint32_t)q & mask;
      const int bit = (2 * lane + k) * bits, wd = bit >> 5, sh = bit & 31;
      __hip_atomic_fetch_or(pk + wd, v << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
      if (sh + bits > 32)
        __hip_atomic_fetch_or(pk + wd + 1, v >> (32 - sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    }
  }
  wave_sync();

  // store: unit u (us bytes) is bytes [us u, us (u+1)) of the packed row
  const int us = g.c < 4 ? g.c : 4;
  const int nunits = g.R / us;
  if (lane < nunits) {
    const int byte = us * lane;
    uint8_t *dst = row_codes + tiled_offset(t, byte / g.c, g.R, g.c) + byte % g.c;
    if (us == 4)
      *reinterpret_cast<uint32_t *>(dst) = pk[lane];
    else if (us == 2)
      *reinterpret_cast<uint16_t *>(dst) = reinterpret_cast<const uint16_t *>(pk)[lane];
    else
      *dst = reinterpret_cast<const uint8_t *>(pk)[lane];
  }
}

}  // namespace arow
