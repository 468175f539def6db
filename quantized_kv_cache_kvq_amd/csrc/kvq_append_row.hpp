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

// Per-block scale (and min), codes and bit-packed row of one token whose
// stored coordinates are held two per lane (a = coordinate 2l, c = 2l + 1),
// for a plain or KVarN plane of a fixed codec: blocks of 32 are the 16
// lanes of a DPP row, so every reduction is a row reduction and nothing goes
// through LDS except the 3/5/6-bit pack.  `rows` = rows before this
// (b, kv head) plane.
template <int BITS, int FAM>
__device__ __forceinline__ void quantize_row(const PlaneArgs &p, long long rows, int t, float a, float c,
                                             uint32_t *stage) {
  constexpr int RB = row_bytes(FAM == FAM_0 ? KVQ_Q8_0 : KVQ_Q8_1, D) * BITS / 8;   // 16 * BITS
  constexpr int CK = chunk_bytes(RB);
  const int lane = threadIdx.x & 63;
  const long long so = (rows + t) * 4 + (lane >> 4);
  float d, m = 0.f;
  if constexpr (FAM == FAM_0) {
    const float amax = row_max16(fmaxf(fabsf(a), fabsf(c)));
    constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
    const uint16_t dh = f32_to_f16_bits(amax / qmax);
    if ((lane & 15) == 0) p.scales[so] = dh;
    d = f16_bits_to_f32(dh);
  } else {
    const float lo = row_min16(fminf(a, c)), hi = row_max16(fmaxf(a, c));
    const uint16_t mh = f32_to_f16_bits(lo);
    m = f16_bits_to_f32(mh);
    constexpr float levels = (float)((1 << BITS) - 1);
    const uint16_t dh = f32_to_f16_bits((hi - m) / levels);
    if ((lane & 15) == 0) {
      p.scales[so] = dh;
      p.mins[so] = mh;
    }
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
  // this lane's 2*BITS bits start at bit 2*BITS*lane of the row
  const uint32_t v = (q0 & mask) | ((q1 & mask) << BITS);
  uint8_t *tile = p.codes + rows * RB + (long long)(t / TILE) * TILE * RB;
  const int tt = t % TILE;
  if constexpr (BITS == 8 || BITS == 4 || BITS == 2 || BITS == 1) {
    constexpr int K = 16 / BITS;                   // lanes per dword
    uint32_t w = v << (2 * BITS * (lane % K));
#pragma unroll
    for (int o = 1; o < K; o <<= 1) w |= __shfl_xor(w, o, 64);
    if (lane % K == 0) {
      const int byte = 4 * (lane / K);
      *reinterpret_cast<uint32_t *>(tile + ((byte / CK) * TILE + tt) * CK + byte % CK) = w;
    }
  } else {
    // 3, 5, 6 bits: OR each lane's field into the row's dwords in LDS
    if (lane < RB / 4) stage[lane] = 0u;
    wave_sync();
    const int o = 2 * BITS * lane, k = o >> 5, sh = o & 31;
    __hip_atomic_fetch_or(stage + k, v << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (sh + 2 * BITS > 32)
      __hip_atomic_fetch_or(stage + k + 1, v >> (32 - sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    wave_sync();
    if (lane < RB / 4) {
      const int byte = 4 * lane;
      *reinterpret_cast<uint32_t *>(tile + ((byte / CK) * TILE + tt) * CK + byte % CK) = stage[lane];
    }
    wave_sync();                                   // stage is free for the next item
  }
}

// Row of token t of codec CODEC (plain or KVarN plane; a, c = this lane's
// stored coordinates 2l, 2l + 1).  stage: 32 words of this wave's LDS.
template <int CODEC>
__device__ __forceinline__ void store_row(const PlaneArgs &p, long long rows, int t, float a, float c,
                                          uint32_t *stage) {
  const int lane = threadIdx.x & 63;
  if constexpr (CODEC == KVQ_F16) {
    // binary16 row: dword `lane` holds coordinates 2*lane, 2*lane+1
    const uint32_t pair = (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(c) << 16);
    const int byte = 4 * lane;
    *reinterpret_cast<uint32_t *>(p.codes + rows * (2 * D) + tiled_offset(t, byte / 16, 2 * D, 16) +
                                  byte % 16) = pair;
  } else {
    quantize_row<codec_bits(CODEC), codec_family(CODEC)>(p, rows, t, a, c, stage);
  }
}

// 16-bit tail copy (binary16 or bfloat16) of raw channels x of token t into
// ring slot t mod tail_len of plane `plane` (= b * hkv + h).
__device__ __forceinline__ void store_tail(const PlaneArgs &p, long long plane, int t, float2 x) {
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
__device__ __forceinline__ void stored_coords(const PlaneArgs &p, int h, float2 x, float &a, float &c) {
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

}  // namespace arow
