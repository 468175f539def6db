// Append kernels: rotate / project, block-quantise, bit-pack and store new
// tokens, plus their 16-bit precision-tail copy.  Steps, after the BeeLlama
// v0.4.0 notes (KVarN and precision-tail sections) and the KV-COBRA
// explainer (projection with the Hadamard rotation fused in):
//   1. tail copy: the raw vector rounded to the tail format (binary16 or
//      bfloat16) into ring slot t mod tail_len;
//   2. stored coordinates: x (plain), H (x * w) by a fast Walsh-Hadamard
//      transform (hadamard), or P_h^T x (low rank);
//   3. per 32-block (or min(32, rank) block) scale (and min);
//   4. codes with correctly rounded binary32 division and rint (ties even):
//      this reproduces the exact-quotient definition bit for bit;
//   5. bit-pack the row and store it in the 64-token tiled layout.
// Three kernels: layers with only plain / KVarN planes take one lane per
// (token, 32-channel block) (append_flat_kernel); layers with a low-rank
// plane take one wave per (token, kv head, K|V) item (append_kernel), and
// prefill-sized low-rank appends project on the matrix cores
// (append_lowrank_kernel).
#include "kvq_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {

#include "kvq_append_row.hpp"
using namespace arow;

// Items are plane-major, token-minor: item = ((K|V * B + b) * Hkv + h) * n_new
// + i, so a workgroup's waves take consecutive new tokens of one plane and
// its stores fill whole lines of the 64-token tiled layout (the chunks of
// consecutive tokens are adjacent) inside one XCD's L2.
struct Item {
  int which, b, h, i;
};
__device__ __forceinline__ Item item_of(unsigned item, int hkv, int n_new, int batch) {
  Item r;
  r.i = (int)(item % (unsigned)n_new);
  unsigned pl = item / (unsigned)n_new;
  r.h = (int)(pl % (unsigned)hkv);
  pl /= (unsigned)hkv;
  r.b = (int)(pl % (unsigned)batch);
  r.which = (int)(pl / (unsigned)batch);
  return r;
}

// Source row of an item.
__device__ __forceinline__ const float *item_src(const float *__restrict__ k_new,
                                                 const float *__restrict__ v_new, int n_new,
                                                 int hkv, const Item &it) {
  return (it.which ? v_new : k_new) + (((long long)it.b * n_new + it.i) * hkv + it.h) * D;
}

// One item, one wave; x = this lane's two raw channels (loaded by the
// caller ahead of time); p is the item's plane (a kernel argument bound at
// the call site, so its fields stay scalar loads of the argument buffer).
// The LDS arrays are this wave's own.
template <bool LR>
__device__ __forceinline__ void append_item(const PlaneArgs &p, int n_new, int t0, const Item &it,
                                            float2 x, float *xin, float *coords, uint8_t *codes) {
  const int hkv = p.hkv;
  const int h = it.h, i = it.i, b = it.b;
  const int t = t0 + i;
  const int lane = threadIdx.x & 63;
  if ((unsigned)t >= (unsigned)p.capacity) return;   // ragged position out of contract: no write

  // 1. precision tail: 16-bit raw copy (binary16 or bfloat16), slot t mod N,
  //    256-byte rows.  Only the newest N tokens of this call write: older
  //    ones in the same call would race for the slots they share with newer
  //    ones.
  if (p.tail_len > 0 && i + p.tail_len >= n_new) store_tail(p, (long long)b * hkv + h, t, x);

  // 2. plain and KVarN planes: coordinates stay in registers (the rotation
  //    is an in-wave transform), codec fixed at compile time per case
  if (!LR || p.basis != KVQ_BASIS_LOWRANK) {
    float a, c;
    stored_coords(p, h, x, a, c);
    const long long rows = ((long long)b * hkv + h) * p.capacity;
    uint32_t *stage = reinterpret_cast<uint32_t *>(coords);
    switch (p.codec) {
#define KVQ_ROW_CASE(CC) case CC: store_row<CC>(p, rows, t, a, c, stage); break;
      KVQ_ROW_CASE(KVQ_F16)
      KVQ_ROW_CASE(KVQ_Q8_0) KVQ_ROW_CASE(KVQ_Q6_0) KVQ_ROW_CASE(KVQ_Q5_0) KVQ_ROW_CASE(KVQ_Q4_0)
      KVQ_ROW_CASE(KVQ_Q3_0) KVQ_ROW_CASE(KVQ_Q2_0)
      KVQ_ROW_CASE(KVQ_Q8_1) KVQ_ROW_CASE(KVQ_Q6_1) KVQ_ROW_CASE(KVQ_Q5_1) KVQ_ROW_CASE(KVQ_Q4_1)
      KVQ_ROW_CASE(KVQ_Q3_1) KVQ_ROW_CASE(KVQ_Q2_1) KVQ_ROW_CASE(KVQ_Q1_1)
#undef KVQ_ROW_CASE
      default: break;
    }
    return;
  }
  if constexpr (LR) {

  // 3. low rank: u = P_h^T x, then per-head width and codec
  lr_project_row(p.proj + (long long)h * D * D, x, xin, coords);
  lr_store_row(p, head_geom(p, b, h), t, coords[2 * lane], coords[2 * lane + 1],
               reinterpret_cast<uint32_t *>(codes));
  }  // LR
}

// Every wave takes a contiguous run of items (consecutive new tokens of one
// plane, moving on to the next plane at its end): the item's coordinates
// advance by increments, with no division per item, and the next item's
// row is loaded while the current one is processed.  8-wave workgroups;
// far fewer workgroups than items for a prefill-sized append.
constexpr int AP_WAVES = 8;

// LR: the layer has low-rank planes (their projection path is compiled only
// into this instance, which needs far more registers).
template <bool LR>
__global__ __launch_bounds__(64 * AP_WAVES) void append_kernel(PlaneArgs kp, PlaneArgs vp,
                                                               const float *__restrict__ k_new,
                                                               const float *__restrict__ v_new,
                                                               int n_new, int t0, int batch,
                                                               const int32_t *__restrict__ seq,
                                                               unsigned items) {
  __shared__ float xin[AP_WAVES][D];
  __shared__ float coords[AP_WAVES][D];
  __shared__ __attribute__((aligned(16))) uint8_t codes[AP_WAVES][D];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hkv = kp.hkv;
  const unsigned waves = gridDim.x * (unsigned)AP_WAVES;
  const unsigned run = (items + waves - 1) / waves;
  const unsigned begin = (blockIdx.x * (unsigned)AP_WAVES + w) * run;
  if (begin >= items) return;
  const unsigned end = begin + run < items ? begin + run : items;
  auto next = [&](Item it) {
    if (++it.i == n_new) {
      it.i = 0;
      if (++it.h == hkv) {
        it.h = 0;
        if (++it.b == batch) {
          it.b = 0;
          ++it.which;
        }
      }
    }
    return it;
  };
  auto load = [&](const Item &it) {
    return reinterpret_cast<const float2 *>(item_src(k_new, v_new, n_new, hkv, it))[lane];
  };
  Item it = item_of(begin, hkv, n_new, batch);
  float2 x = load(it);
  for (unsigned item = begin; item < end; ++item) {
    const Item nx = item + 1 < end ? next(it) : it;
    const float2 xn = load(nx);            // the last item re-reads its own row
    // ragged batch: sequence b appends at its own position
    const int tb = seq ? __builtin_amdgcn_readfirstlane(seq[it.b]) : t0;
    if (it.which)
      append_item<LR>(vp, n_new, tb, it, x, xin[w], coords[w], codes[w]);
    else
      append_item<LR>(kp, n_new, tb, it, x, xin[w], coords[w], codes[w]);
    it = nx;
    x = xn;
  }
}


// The scalar fields of one plain or KVarN plane that append_flat_kernel
// reads, picked from the K or V argument with scalar selects (a run-time
// choice between the two argument blocks would copy them to scratch).
struct RowPlane {
  uint8_t *codes;
  uint16_t *scales;
  uint16_t *mins;
  uint16_t *tail;
  const float *w;
  int codec, basis, hkv, capacity, tail_len, tail_bf16;
};

__device__ __forceinline__ RowPlane row_plane(const PlaneArgs &kp, const PlaneArgs &vp, bool v) {
  RowPlane r;
  r.codes = v ? vp.codes : kp.codes;
  r.scales = v ? vp.scales : kp.scales;
  r.mins = v ? vp.mins : kp.mins;
  r.tail = v ? vp.tail : kp.tail;
  r.w = v ? vp.w : kp.w;
  r.codec = v ? vp.codec : kp.codec;
  r.basis = v ? vp.basis : kp.basis;
  r.hkv = v ? vp.hkv : kp.hkv;
  r.capacity = v ? vp.capacity : kp.capacity;
  r.tail_len = v ? vp.tail_len : kp.tail_len;
  r.tail_bf16 = v ? vp.tail_bf16 : kp.tail_bf16;
  return r;
}

// Layers whose K and V planes are both plain or KVarN, one lane per
// (new token, 32-channel block): a wave takes 16 consecutive new tokens of
// one plane x 4 blocks (lane 4r + j = token r, block j), a 256-thread
// workgroup 64 tokens.  Each lane reads its block's 32 binary32 values
// (128 contiguous bytes), and quantises it on its own (maximum, scale,
// codes, packing in registers), so no row-wide reduction crosses lanes; the
// 16 tokens' chunks of one block are contiguous in the 64-token tiled
// layout, so the code, scale and tail stores of a wave fill whole lines.
// The KVarN transform (sign vector, then the Walsh-Hadamard butterflies in
// increasing stride) runs strides 1..16 inside the lane and strides 32, 64
// between the four lanes of a token (quad DPP), with the same butterflies
// and order as the one-row-per-wave transform, so both give the same bits.
constexpr int AF_TOKENS = 64;                    // tokens per workgroup
constexpr int AF_THREADS = 4 * AF_TOKENS;

// Partner lane's value in the same quad: xor 1 (QP = 0xB1) or xor 2 (0x4E).
template <int QP>
__device__ __forceinline__ float quad_xor(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), QP, 0xF, 0xF, true));
}

// Block j (32 values x) of token t of the plane whose rows start at row
// `rows`: scale (and min), codes, packed field, stored in the tiled layout.
template <int CODEC>
__device__ __forceinline__ void encode_block_lane(const RowPlane &p, long long rows, int t, int j,
                                                  const float (&x)[32]) {
  constexpr int RB = row_bytes(CODEC, D);
  uint8_t *tile = p.codes + rows * RB + (long long)(t >> 6) * (TILE * RB);
  const int tt = t & (TILE - 1);
  auto chunk_ptr = [&](int byte) { return tile + ((byte >> 4) * TILE + tt) * 16 + (byte & 15); };
  if constexpr (CODEC == KVQ_F16) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = (uint32_t)f32_to_f16_bits(x[8 * s + 2 * e]) | ((uint32_t)f32_to_f16_bits(x[8 * s + 2 * e + 1]) << 16);
      *reinterpret_cast<u32x4 *>(chunk_ptr(64 * j + 16 * s)) = v;
    }
  } else {
    constexpr int BITS = codec_bits(CODEC), FAM = codec_family(CODEC);
    constexpr uint32_t mask = (1u << BITS) - 1u;
    const long long so = (rows + t) * (D / 32) + j;
    float d, m = 0.f;
    uint32_t q[32];
    if constexpr (FAM == FAM_0) {
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
      constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
      const uint16_t dh = f32_to_f16_bits(amax / qmax);
      p.scales[so] = dh;
      d = f16_bits_to_f32(dh);
#pragma unroll
      for (int e = 0; e < 32; ++e)
        q[e] = d != 0.f ? (uint32_t)(int)fminf(fmaxf(rintf(x[e] / d), -qmax), qmax) & mask : 0u;
    } else {
      float lo = x[0], hi = x[0];
#pragma unroll
      for (int e = 1; e < 32; ++e) {
        lo = fminf(lo, x[e]);
        hi = fmaxf(hi, x[e]);
      }
      const uint16_t mh = f32_to_f16_bits(lo);
      m = f16_bits_to_f32(mh);
      constexpr float levels = (float)((1 << BITS) - 1);
      const uint16_t dh = f32_to_f16_bits((hi - m) / levels);
      p.scales[so] = dh;
      p.mins[so] = mh;
      d = f16_bits_to_f32(dh);
#pragma unroll
      for (int e = 0; e < 32; ++e)
        q[e] = d != 0.f ? (uint32_t)(int)fminf(fmaxf(rintf((x[e] - m) / d), 0.f), levels) : 0u;
    }
    // the block's field: code e at bits [e BITS, (e + 1) BITS), BITS dwords
    uint32_t w[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = 0u;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int bit = e * BITS;
      w[bit >> 5] |= q[e] << (bit & 31);
      if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= q[e] >> (32 - (bit & 31));
    }
    if constexpr (BITS % 4 == 0) {
#pragma unroll
      for (int s = 0; s < BITS / 4; ++s)
        *reinterpret_cast<u32x4 *>(chunk_ptr(4 * BITS * j + 16 * s)) = u32x4{w[4 * s], w[4 * s + 1], w[4 * s + 2], w[4 * s + 3]};
    } else {
#pragma unroll
      for (int k = 0; k < BITS; ++k) *reinterpret_cast<uint32_t *>(chunk_ptr(4 * BITS * j + 4 * k)) = w[k];
    }
  }
}

__global__ __launch_bounds__(AF_THREADS) void append_flat_kernel(PlaneArgs kp, PlaneArgs vp,
                                                                 const float *__restrict__ k_new,
                                                                 const float *__restrict__ v_new, int n_new,
                                                                 int t0, int batch,
                                                                 const int32_t *__restrict__ seq) {
  __shared__ float wsh[D];
  const bool isv = (int)blockIdx.z >= batch;
  const int b = isv ? (int)blockIdx.z - batch : (int)blockIdx.z;
  const int h = blockIdx.y;
  const RowPlane p = row_plane(kp, vp, isv);
  const bool rot = p.basis == KVQ_BASIS_HADAMARD;
  if (rot) {
    if (threadIdx.x < D / 4)
      reinterpret_cast<float4 *>(wsh)[threadIdx.x] = reinterpret_cast<const float4 *>(p.w + (long long)h * D)[threadIdx.x];
    __syncthreads();
  }
  const int i = (int)blockIdx.x * AF_TOKENS + (int)(threadIdx.x >> 2);
  const int j = threadIdx.x & 3;
  if (i >= n_new) return;                          // all four lanes of a token leave together
  const int t = (seq ? seq[b] : t0) + i;
  if ((unsigned)t >= (unsigned)p.capacity) return;   // ragged position out of contract: no write
  const float *src = (isv ? v_new : k_new) + (((long long)b * n_new + i) * p.hkv + h) * D + 32 * j;
  float x[32];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float4 v = reinterpret_cast<const float4 *>(src)[s];
    x[4 * s] = v.x;
    x[4 * s + 1] = v.y;
    x[4 * s + 2] = v.z;
    x[4 * s + 3] = v.w;
  }
  const long long plane = (long long)b * p.hkv + h;
  // precision tail: the raw values of the newest tail_len tokens of this call
  if (p.tail_len > 0 && i + p.tail_len >= n_new) {
    const int slot = t % p.tail_len;
    uint8_t *tile = reinterpret_cast<uint8_t *>(p.tail) + plane * p.tail_len * (2 * D) +
                    (long long)(slot >> 6) * (TILE * 2 * D);
    const int st = slot & (TILE - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = x[8 * s + 2 * e], hi = x[8 * s + 2 * e + 1];
        v[e] = p.tail_bf16 ? (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16)
                           : (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
      }
      *reinterpret_cast<u32x4 *>(tile + ((4 * j + s) * TILE + st) * 16) = v;
    }
  }
  if (rot) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float4 wv = reinterpret_cast<const float4 *>(wsh + 32 * j)[s];
      x[4 * s] *= wv.x;
      x[4 * s + 1] *= wv.y;
      x[4 * s + 2] *= wv.z;
      x[4 * s + 3] *= wv.w;
    }
    // strides 1 .. 16 inside the lane: (u, v) -> (u + v, u - v)
#pragma unroll
    for (int st = 1; st < 32; st <<= 1) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        if (e & st) continue;
        const float u = x[e], v = x[e + st];
        x[e] = u + v;
        x[e + st] = u - v;
      }
    }
    // strides 32 and 64: partner lane j ^ 1, j ^ 2 of the same token
    const bool up1 = (j & 1) != 0, up2 = (j & 2) != 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float px = quad_xor<0xB1>(x[e]);
      x[e] = up1 ? px - x[e] : x[e] + px;
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float px = quad_xor<0x4E>(x[e]);
      x[e] = up2 ? px - x[e] : x[e] + px;
    }
  }
  const long long rows = plane * p.capacity;
  switch (p.codec) {
#define KVQ_FLAT_CASE(CC) \
  case CC: encode_block_lane<CC>(p, rows, t, j, x); break;
    KVQ_FLAT_CASE(KVQ_F16)
    KVQ_FLAT_CASE(KVQ_Q8_0) KVQ_FLAT_CASE(KVQ_Q6_0) KVQ_FLAT_CASE(KVQ_Q5_0) KVQ_FLAT_CASE(KVQ_Q4_0)
    KVQ_FLAT_CASE(KVQ_Q3_0) KVQ_FLAT_CASE(KVQ_Q2_0)
    KVQ_FLAT_CASE(KVQ_Q8_1) KVQ_FLAT_CASE(KVQ_Q6_1) KVQ_FLAT_CASE(KVQ_Q5_1) KVQ_FLAT_CASE(KVQ_Q4_1)
    KVQ_FLAT_CASE(KVQ_Q3_1) KVQ_FLAT_CASE(KVQ_Q2_1) KVQ_FLAT_CASE(KVQ_Q1_1)
#undef KVQ_FLAT_CASE
    default: break;
  }
}

// Low-rank planes, prefill-sized appends: u = P_h^T x for 16 tokens at a
// time on the matrix cores (v_mfma_f32_16x16x32_f16).  A workgroup of 4
// waves takes LRM_CHUNKS runs of 64 consecutive new tokens of one (K|V,
// batch entry, kv head); P_h (binary16, exact) is staged in LDS once and
// read back transposed as the B operand; each wave's A operand is its 16
// token rows split into binary16 hi + lo parts (x = hi + lo to ~22 bits;
// both products are exact and accumulate in binary32).  The 16 x rank
// result goes through LDS; then lane (token r, block j) quantises block j of
// token r on its own (the formulas of the one-token path, so the same codes
// for the same u) and stores the block's field, scale and min.
constexpr int LRM_WAVES = 4;
constexpr int LRM_ROWS = 16;                    // tokens per wave
constexpr int LRM_CHUNKS = 16;                  // 64-token runs per workgroup
constexpr int LRM_PPITCH = 2 * D + 32;          // staged P row (bytes)
constexpr int LRM_UPITCH = D + 4;               // staged result row (floats)

typedef _Float16 lrm_half8 __attribute__((ext_vector_type(8)));
typedef float lrm_floatx4 __attribute__((ext_vector_type(4)));
typedef short lrm_short4 __attribute__((ext_vector_type(4)));

// 8 binary16 B-operand values (rows k .. k+7 of column n of a row-major LDS
// array) by two transposing loads.
__device__ __forceinline__ lrm_half8 lrm_tr16(const uint8_t *p0, const uint8_t *p1) {
  typedef __attribute__((address_space(3))) lrm_short4 lds_s4;
  const lrm_short4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p0));
  const lrm_short4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p1));
  lrm_short4 v[2] = {a, b};
  return __builtin_bit_cast(lrm_half8, v);
}

// Block j (L = g.L coordinates ub[0 .. L) of token t) of a low-rank row of
// BITS-bit codes: scale (and min), codes as in the one-token path, and the
// block's field (code e at bit e * BITS, L * BITS / 8 bytes at row byte
// j * L * BITS / 8), stored in the tiled layout.
template <int BITS>
__device__ __forceinline__ void lr_block_store(const PlaneArgs &p, const HeadGeom &g, int t, int j,
                                               const float *ub) {
  const int L = g.L;
  const bool f0 = codec_family(g.codec) == FAM_0;
  const long long so = g.scales_off + (long long)t * g.nblk + j;
  float x[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) x[e] = e < L ? ub[e] : 0.f;
  float d, m = 0.f;
  if (f0) {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
    constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
    const uint16_t dh = f32_to_f16_bits(amax / qmax);
    p.scales[so] = dh;
    d = f16_bits_to_f32(dh);
  } else {
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int e = 1; e < 32; ++e)
      if (e < L) {
        lo = fminf(lo, x[e]);
        hi = fmaxf(hi, x[e]);
      }
    const uint16_t mh = f32_to_f16_bits(lo);
    m = f16_bits_to_f32(mh);
    constexpr float levels = (float)((1 << BITS) - 1);
    const uint16_t dh = f32_to_f16_bits((hi - m) / levels);
    p.scales[so] = dh;
    p.mins[so] = mh;
    d = f16_bits_to_f32(dh);
  }
  constexpr uint32_t mask = (1u << BITS) - 1u;
  uint32_t w[BITS];
#pragma unroll
  for (int k = 0; k < BITS; ++k) w[k] = 0u;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    uint32_t q = 0u;
    if (d != 0.f && e < L) {
      if (f0) {
        constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
        q = (uint32_t)(int)fminf(fmaxf(rintf(x[e] / d), -qmax), qmax) & mask;
      } else {
        constexpr float levels = (float)((1 << BITS) - 1);
        q = (uint32_t)(int)fminf(fmaxf(rintf((x[e] - m) / d), 0.f), levels);
      }
    }
    const int bit = e * BITS;
    w[bit >> 5] |= q << (bit & 31);
    if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= q >> (32 - (bit & 31));
  }
  // the field in units no wider than the layout's chunk: dwords when
  // chunks hold 4+ bytes (then the field is whole dwords), else 16-bit
  // halves (rows of 2, 6 or 10 bytes: rank 16 at 1, 3 or 5 bits)
  uint8_t *row = p.codes + g.codes_off;
  const int fbytes = L * BITS / 8, fb = j * fbytes;
  if (g.c >= 4) {
#pragma unroll
    for (int k = 0; k < BITS; ++k)
      if (4 * k < fbytes) {
        const int byte = fb + 4 * k;
        *reinterpret_cast<uint32_t *>(row + tiled_offset(t, byte / g.c, g.R, g.c) + byte % g.c) = w[k];
      }
  } else {
#pragma unroll
    for (int k = 0; k < 2 * BITS; ++k)
      if (2 * k < fbytes) {
        const int byte = fb + 2 * k;
        *reinterpret_cast<uint16_t *>(row + tiled_offset(t, byte / g.c, g.R, g.c) + byte % g.c) =
            (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
      }
  }
}

// LRM_CHUNKS runs of 64 tokens of one (plane, batch entry b, kv head h) whose
// codes have BITS bits (one quantiser per instantiation keeps the loop's
// registers low); p is bound at the call site (a run-time choice between
// the two plane arguments would copy them to scratch).
template <int BITS>
__device__ __forceinline__ void lowrank_runs(const PlaneArgs &p, const float *__restrict__ src, int b,
                                             int h, int n_new, int tb, uint8_t *pl, float *ul) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hkv = p.hkv;

  // stage P_h: row c (input channel) at c * LRM_PPITCH, 256 bytes each
  {
    const u32x4 *P4 = reinterpret_cast<const u32x4 *>(p.proj + (long long)h * D * D);
    for (int i = threadIdx.x; i < D * D / 8; i += 64 * LRM_WAVES) {
      const int c = i / (D / 8), k = i % (D / 8);
      *reinterpret_cast<u32x4 *>(pl + c * LRM_PPITCH + 16 * k) = P4[i];
    }
  }
  __syncthreads();
  const HeadGeom g = head_geom(p, b, h);
  const long long plane = (long long)b * hkv + h;
  float *u = ul + w * (LRM_ROWS * LRM_UPITCH);
  const int r = lane & 15, kg = lane >> 4;
  // A operand: row r is token i0 + r of this wave's run (rows past n_new
  // repeat the last token and are not stored), k-group kg; lane (r, kg)
  // holds channels 32 kc + 8 kg .. + 8 of its token.  The next run's rows
  // load while this run is projected and stored (the loads are
  // unconditional, clamped into the input, so the wait for them is exact).
  const int run0 = (int)blockIdx.x * LRM_CHUNKS * (LRM_WAVES * LRM_ROWS) + w * LRM_ROWS;
  if (run0 >= n_new) return;
  float xv[D / 4];
#define KVQ_LRM_LOAD_ROWS(I0)                                                                      \
  {                                                                                                \
    const int ir_ = (I0) + r < n_new ? (I0) + r : n_new - 1;                                       \
    const float *xr_ = src + (((long long)b * n_new + ir_) * hkv + h) * D;                         \
    _Pragma("unroll") for (int kc = 0; kc < D / 32; ++kc) {                                        \
      const float4 x0 = *reinterpret_cast<const float4 *>(xr_ + 32 * kc + 8 * kg);                 \
      const float4 x1 = *reinterpret_cast<const float4 *>(xr_ + 32 * kc + 8 * kg + 4);             \
      xv[8 * kc] = x0.x; xv[8 * kc + 1] = x0.y; xv[8 * kc + 2] = x0.z; xv[8 * kc + 3] = x0.w;      \
      xv[8 * kc + 4] = x1.x; xv[8 * kc + 5] = x1.y; xv[8 * kc + 6] = x1.z; xv[8 * kc + 7] = x1.w;  \
    }                                                                                              \
  }
  KVQ_LRM_LOAD_ROWS(run0)
  for (int ch = 0;; ++ch) {
    const int i0 = run0 + ch * (LRM_WAVES * LRM_ROWS);
    // precision tail of the newest tail_len tokens: the lane's 4 chunks of
    // 8 channels, 16 bytes each
    const int ti = i0 + r, tt = tb + ti;
    const bool row_ok = ti < n_new && (unsigned)tt < (unsigned)p.capacity;
    if (row_ok && p.tail_len > 0 && ti + p.tail_len >= n_new) {
      const int slot = tt % p.tail_len;
      uint8_t *base = reinterpret_cast<uint8_t *>(p.tail) + plane * p.tail_len * (2 * D);
#pragma unroll
      for (int kc = 0; kc < D / 32; ++kc) {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = xv[8 * kc + 2 * e], hi = xv[8 * kc + 2 * e + 1];
          v[e] = p.tail_bf16 ? (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16)
                             : (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
        }
        *reinterpret_cast<u32x4 *>(base + tiled_offset(slot, 4 * kc + kg, 2 * D, 16)) = v;
      }
    }
    lrm_half8 ahi[D / 32], alo[D / 32];
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 hi = (_Float16)xv[8 * kc + e];
        ahi[kc][e] = hi;
        alo[kc][e] = (_Float16)(xv[8 * kc + e] - (float)hi);
      }
    }
    const bool more = ch + 1 < LRM_CHUNKS && i0 + LRM_WAVES * LRM_ROWS < n_new;
    KVQ_LRM_LOAD_ROWS(more ? i0 + LRM_WAVES * LRM_ROWS : i0)
    for (int ct = 0; ct < (g.n + 15) / 16; ++ct) {
      lrm_floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < D / 32; ++kc) {
        // column n = lane % 16 of tile ct, rows 32kc + 8kg .. +7
        const uint8_t *pb = pl + (32 * kc + 8 * kg + (r >> 2)) * LRM_PPITCH + (16 * ct + 4 * (r & 3)) * 2;
        const lrm_half8 bv = lrm_tr16(pb, pb + 4 * LRM_PPITCH);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kc], bv, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[kc], bv, c, 0, 0, 0);
      }
      // lane (n, g) holds rows 4g .. 4g+3 of column n
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) u[(4 * kg + rr) * LRM_UPITCH + 16 * ct + r] = c[rr];
    }
    wave_sync();
    // lane (token r, block j = kg) quantises and stores its block
    if (row_ok && kg < g.nblk) lr_block_store<BITS>(p, g, tt, kg, u + r * LRM_UPITCH + kg * g.L);
    wave_sync();                                   // u is free for the next run
    if (!more) break;
  }
#undef KVQ_LRM_LOAD_ROWS
}

__global__ __launch_bounds__(64 * LRM_WAVES) void append_lowrank_kernel(PlaneArgs kp, PlaneArgs vp,
                                                                         const float *__restrict__ k_new,
                                                                         const float *__restrict__ v_new,
                                                                         int n_new, int t0, int batch,
                                                                         const int32_t *__restrict__ seq) {
  __shared__ __attribute__((aligned(16))) uint8_t pl[D * LRM_PPITCH];
  __shared__ __attribute__((aligned(16))) float ul[LRM_WAVES * LRM_ROWS * LRM_UPITCH];
  // grid: x = run of LRM_CHUNKS x 64 tokens, y = kv head, z = K|V * batch + b
  const int which = (int)blockIdx.z / batch, b = (int)blockIdx.z % batch, h = (int)blockIdx.y;
  const int tb = seq ? __builtin_amdgcn_readfirstlane(seq[b]) : t0;
  // the head's code width (K and V share it), one loop per width
  switch (codec_bits(kp.hcodec[h])) {
#define KVQ_LRM_CASE(BB)                                       \
  case BB:                                                     \
    if (which) lowrank_runs<BB>(vp, v_new, b, h, n_new, tb, pl, ul); \
    else lowrank_runs<BB>(kp, k_new, b, h, n_new, tb, pl, ul);      \
    break;
    KVQ_LRM_CASE(1) KVQ_LRM_CASE(2) KVQ_LRM_CASE(3) KVQ_LRM_CASE(4) KVQ_LRM_CASE(5) KVQ_LRM_CASE(6)
    KVQ_LRM_CASE(8)
#undef KVQ_LRM_CASE
    default: break;
  }
}

hipError_t launch_append(const PlaneArgs &kp, const PlaneArgs &vp, const float *k_new,
                         const float *v_new, int batch, int n_new, int t0, const int32_t *seq,
                         hipStream_t stream) {
  const long long items = (long long)batch * n_new * kp.hkv * 2;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  long long blocks = (items + AP_WAVES - 1) / AP_WAVES;
  if (blocks > 1024) blocks = 1024;
  if (kp.basis == KVQ_BASIS_LOWRANK && vp.basis == KVQ_BASIS_LOWRANK && n_new >= LRM_ROWS) {
    const int per = LRM_CHUNKS * LRM_WAVES * LRM_ROWS;
    const dim3 grid((unsigned)((n_new + per - 1) / per), (unsigned)kp.hkv, (unsigned)(2 * batch));
    hipLaunchKernelGGL(append_lowrank_kernel, grid, dim3(64 * LRM_WAVES), 0, stream, kp, vp, k_new,
                       v_new, n_new, t0, batch, seq);
  } else if (kp.basis == KVQ_BASIS_LOWRANK || vp.basis == KVQ_BASIS_LOWRANK)
    hipLaunchKernelGGL(append_kernel<true>, dim3((unsigned)blocks), dim3(64 * AP_WAVES), 0, stream, kp,
                       vp, k_new, v_new, n_new, t0, batch, seq, (unsigned)items);
  else {
    const dim3 grid((unsigned)((n_new + AF_TOKENS - 1) / AF_TOKENS), (unsigned)kp.hkv, (unsigned)(2 * batch));
    hipLaunchKernelGGL(append_flat_kernel, grid, dim3(AF_THREADS), 0, stream, kp, vp, k_new, v_new, n_new, t0,
                       batch, seq);
  }
  return hipGetLastError();
}

}  // namespace kvq
