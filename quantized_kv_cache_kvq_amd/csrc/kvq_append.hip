// Append kernel: rotate / project, block-quantise, bit-pack and store new
// tokens, plus their 16-bit precision-tail copy.
//
// One wave (64 lanes) per item = (batch entry, new token, kv head, K|V);
// 8-wave workgroups stride over the items.  Lane l owns raw channels 2l,
// 2l+1.  Steps, after the BeeLlama v0.4.0 notes (KVarN and precision-tail
// sections) and the KV-COBRA explainer (projection with the Hadamard
// rotation fused in):
//   1. tail copy: the raw vector rounded to the tail format (binary16 or
//      bfloat16) into ring slot t mod tail_len;
//   2. stored coordinates: x (plain), H (x * w) by an in-wave fast
//      Walsh-Hadamard transform (hadamard), or P_h^T x (low rank);
//   3. per 32-block (or min(32, rank) block) scale (and min);
//   4. codes with correctly rounded binary32 division and rint (ties even):
//      this reproduces the exact-quotient definition bit for bit;
//   5. bit-pack the row and store it in the 64-token tiled layout.
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

  // 3. low rank: u = P_h^T x through LDS, then per-head width and codec
  xin[2 * lane] = x.x;
  xin[2 * lane + 1] = x.y;
  wave_sync();
  {
    // The wave reads all of P_h (128 x 128 binary16, 32 KiB) in one round
    // trip: load i of lane l is row 4i + l/16, columns 8(l%16) .. +8.  Each
    // lane sums its 8 columns over its 32 rows; the four lanes holding the
    // same columns (l, l^16, l^32, l^48) then add their sums.
    const u32x4 *P4 = reinterpret_cast<const u32x4 *>(p.proj + (long long)h * D * D);
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
  }
  wave_sync();

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


// Low-rank planes, prefill-sized appends: u = P_h^T x for 16 tokens at a
// time on the matrix cores (v_mfma_f32_16x16x32_f16), so P_h is read once
// per 64 tokens instead of once per token.  A workgroup of 4 waves takes 64
// consecutive new tokens of one (K|V, batch entry, kv head); P_h (binary16,
// exact) is staged in LDS once and read back transposed as the B operand;
// each wave's A operand is its 16 token rows split into binary16 hi + lo
// parts (x = hi + lo to ~22 bits; both products are exact and accumulate in
// binary32).  The 16 x rank result goes through LDS to one row per pass of
// lr_store_row, the same quantiser as the one-token path.
constexpr int LRM_WAVES = 4;
constexpr int LRM_ROWS = 16;                    // tokens per wave
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

// One (plane, batch entry b, kv head h, 64-token chunk); p is bound at the
// call site (a run-time choice between the two plane arguments would copy
// them to scratch).
__device__ __forceinline__ void lowrank_chunk(const PlaneArgs &p, const float *__restrict__ src, int b,
                                              int h, int n_new, int tb, uint8_t *pl, float *ul,
                                              uint32_t *pk) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hkv = p.hkv;
  const int i0 = (int)blockIdx.x * (LRM_WAVES * LRM_ROWS) + w * LRM_ROWS;   // this wave's first token

  // stage P_h: row c (input channel) at c * LRM_PPITCH, 256 bytes each
  {
    const u32x4 *P4 = reinterpret_cast<const u32x4 *>(p.proj + (long long)h * D * D);
    for (int i = threadIdx.x; i < D * D / 8; i += 64 * LRM_WAVES) {
      const int c = i / (D / 8), k = i % (D / 8);
      *reinterpret_cast<u32x4 *>(pl + c * LRM_PPITCH + 16 * k) = P4[i];
    }
  }
  __syncthreads();
  if (i0 >= n_new) return;

  // A operand: row r = lane % 16 is token i0 + r (rows past n_new repeat
  // the last token and are not stored), k-group kg = lane / 16
  const int r = lane & 15, kg = lane >> 4;
  const int ir = i0 + r < n_new ? i0 + r : n_new - 1;
  const float *xr = src + (((long long)b * n_new + ir) * hkv + h) * D;
  lrm_half8 ahi[D / 32], alo[D / 32];
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc) {
    const float4 x0 = *reinterpret_cast<const float4 *>(xr + 32 * kc + 8 * kg);
    const float4 x1 = *reinterpret_cast<const float4 *>(xr + 32 * kc + 8 * kg + 4);
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const _Float16 hi = (_Float16)xs[e];
      ahi[kc][e] = hi;
      alo[kc][e] = (_Float16)(xs[e] - (float)hi);
    }
  }
  const HeadGeom g = head_geom(p, b, h);
  float *u = ul + w * (LRM_ROWS * LRM_UPITCH);
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

  const long long plane = (long long)b * hkv + h;
  for (int rr = 0; rr < LRM_ROWS; ++rr) {
    const int i = i0 + rr;
    if (i >= n_new) break;
    const int t = tb + i;
    if ((unsigned)t >= (unsigned)p.capacity) continue;   // ragged position out of contract
    if (p.tail_len > 0 && i + p.tail_len >= n_new) {
      const float2 x = reinterpret_cast<const float2 *>(src + (((long long)b * n_new + i) * hkv + h) * D)[lane];
      store_tail(p, plane, t, x);
    }
    const float2 uv = *reinterpret_cast<const float2 *>(u + rr * LRM_UPITCH + 2 * lane);
    lr_store_row(p, g, t, uv.x, uv.y, pk + w * (D / 4));
  }
}

__global__ __launch_bounds__(64 * LRM_WAVES) void append_lowrank_kernel(PlaneArgs kp, PlaneArgs vp,
                                                                         const float *__restrict__ k_new,
                                                                         const float *__restrict__ v_new,
                                                                         int n_new, int t0, int batch,
                                                                         const int32_t *__restrict__ seq) {
  __shared__ __attribute__((aligned(16))) uint8_t pl[D * LRM_PPITCH];
  __shared__ __attribute__((aligned(16))) float ul[LRM_WAVES * LRM_ROWS * LRM_UPITCH];
  __shared__ __attribute__((aligned(16))) uint32_t pk[LRM_WAVES * (D / 4)];
  // grid: x = 64-token chunk, y = kv head, z = K|V * batch + b
  const int which = (int)blockIdx.z / batch, b = (int)blockIdx.z % batch, h = (int)blockIdx.y;
  const int tb = seq ? __builtin_amdgcn_readfirstlane(seq[b]) : t0;
  if (which)
    lowrank_chunk(vp, v_new, b, h, n_new, tb, pl, ul, pk);
  else
    lowrank_chunk(kp, k_new, b, h, n_new, tb, pl, ul, pk);
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
    const int per = LRM_WAVES * LRM_ROWS;
    const dim3 grid((unsigned)((n_new + per - 1) / per), (unsigned)kp.hkv, (unsigned)(2 * batch));
    hipLaunchKernelGGL(append_lowrank_kernel, grid, dim3(64 * LRM_WAVES), 0, stream, kp, vp, k_new,
                       v_new, n_new, t0, batch, seq);
  } else if (kp.basis == KVQ_BASIS_LOWRANK || vp.basis == KVQ_BASIS_LOWRANK)
    hipLaunchKernelGGL(append_kernel<true>, dim3((unsigned)blocks), dim3(64 * AP_WAVES), 0, stream, kp,
                       vp, k_new, v_new, n_new, t0, batch, seq, (unsigned)items);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3((unsigned)blocks), dim3(64 * AP_WAVES), 0, stream, kp,
                       vp, k_new, v_new, n_new, t0, batch, seq, (unsigned)items);
  return hipGetLastError();
}

}  // namespace kvq
