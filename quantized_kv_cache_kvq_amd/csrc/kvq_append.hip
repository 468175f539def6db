// Append kernel: rotate / project, block-quantise, bit-pack and store new
// tokens, plus their 16-bit precision-tail copy.
//
// One wave (64 lanes) per item = (batch entry, new token, kv head, K|V);
// 4-wave workgroups stride over the items.  Lane l owns raw channels 2l,
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

// Source row of an item = (batch entry, new token, kv head, K|V).
__device__ __forceinline__ const float *item_src(const PlaneArgs &kp, const float *__restrict__ k_new,
                                                 const float *__restrict__ v_new, int n_new,
                                                 unsigned item) {
  unsigned id = item;
  const int which = id & 1;
  id >>= 1;
  const unsigned hkv = (unsigned)kp.hkv;
  const unsigned h = id % hkv;
  id /= hkv;
  const unsigned i = id % (unsigned)n_new;
  const unsigned b = id / (unsigned)n_new;
  return (which ? v_new : k_new) + (((long long)b * n_new + i) * hkv + h) * D;
}

// One item, one wave; x = this lane's two raw channels (loaded by the
// caller ahead of time).  The LDS arrays are this wave's own.
__device__ void append_item(const PlaneArgs &kp, const PlaneArgs &vp, int n_new, int t0,
                            unsigned item, float2 x, float *xin, float *coords, uint8_t *codes,
                            float *s_scale, float *s_min) {
  unsigned id = item;
  const int which = id & 1;
  id >>= 1;
  const PlaneArgs &p = which ? vp : kp;
  const int hkv = p.hkv;
  const int h = (int)(id % (unsigned)hkv);
  id /= (unsigned)hkv;
  const int i = (int)(id % (unsigned)n_new);
  const int b = (int)(id / (unsigned)n_new);
  const int t = t0 + i;
  const int lane = threadIdx.x & 63;


  // 1. precision tail: 16-bit raw copy (binary16 or bfloat16), slot t mod N,
  //    256-byte rows.  Only
  //    the newest N tokens of this call write: older ones in the same call
  //    would race for the slots they share with newer ones.
  if (p.tail_len > 0 && i + p.tail_len >= n_new) {
    const long long plane = (long long)b * hkv + h;
    const int slot = t % p.tail_len;
    const uint32_t pair =
        p.tail_bf16 ? (uint32_t)f32_to_bf16_bits(x.x) | ((uint32_t)f32_to_bf16_bits(x.y) << 16)
                    : (uint32_t)f32_to_f16_bits(x.x) | ((uint32_t)f32_to_f16_bits(x.y) << 16);
    uint8_t *base = reinterpret_cast<uint8_t *>(p.tail) + plane * p.tail_len * (2 * D);
    const int byte = 4 * lane;
    *reinterpret_cast<uint32_t *>(base + tiled_offset(slot, byte / 16, 2 * D, 16) + byte % 16) = pair;
  }

  const HeadGeom g = head_geom(p, b, h);

  // 2. stored coordinates
  if (p.basis == KVQ_BASIS_HADAMARD) {
    const float *w = p.w + (long long)h * D;
    float a = x.x * w[2 * lane];
    float c = x.y * w[2 * lane + 1];
    fwht128_wave(a, c);
    coords[2 * lane] = a;
    coords[2 * lane + 1] = c;
  } else if (p.basis == KVQ_BASIS_LOWRANK) {
    xin[2 * lane] = x.x;
    xin[2 * lane + 1] = x.y;
    wave_sync();
    const uint16_t *P = p.proj + (long long)h * D * D;
    for (int k = lane; k < g.n; k += 64) {
      float acc = 0.f;
      for (int r = 0; r < D; ++r) acc = fmaf(f16_bits_to_f32(P[r * D + k]), xin[r], acc);
      coords[k] = acc;
    }
  } else {
    coords[2 * lane] = x.x;
    coords[2 * lane + 1] = x.y;
  }
  wave_sync();

  uint8_t *row_codes = p.codes + g.codes_off;
  const int fam = codec_family(g.codec);
  if (fam == FAM_F16) {
    // binary16 row: dword `lane` holds coordinates 2*lane, 2*lane+1
    uint32_t pair = (uint32_t)f32_to_f16_bits(coords[2 * lane]) |
                    ((uint32_t)f32_to_f16_bits(coords[2 * lane + 1]) << 16);
    const int byte = 4 * lane;
    *reinterpret_cast<uint32_t *>(row_codes + tiled_offset(t, byte / g.c, g.R, g.c) + byte % g.c) = pair;
    return;
  }

  const int bits = codec_bits(g.codec);
  if (p.basis != KVQ_BASIS_LOWRANK && (bits == 8 || bits == 4 || bits == 2 || bits == 1)) {
    // 128 coordinates, lane l holds 2l and 2l+1: block j is the DPP row of
    // lanes 16j .. 16j+15, so block statistics are row reductions; the
    // row's bits are gathered 16/bits lanes to a dword and stored whole.
    const float a = coords[2 * lane], c = coords[2 * lane + 1];
    const long long so = g.scales_off + (long long)t * 4 + (lane >> 4);
    float d, m = 0.f;
    if (fam == FAM_0) {
      const float amax = row_max16(fmaxf(fabsf(a), fabsf(c)));
      const float qmax = (float)((1 << (bits - 1)) - 1);
      const uint16_t dh = f32_to_f16_bits(amax / qmax);
      if ((lane & 15) == 0) p.scales[so] = dh;
      d = f16_bits_to_f32(dh);
    } else {
      const float lo = row_min16(fminf(a, c)), hi = row_max16(fmaxf(a, c));
      const uint16_t mh = f32_to_f16_bits(lo);
      m = f16_bits_to_f32(mh);
      const float R = hi - m;
      const float levels = (float)((1 << bits) - 1);
      const uint16_t dh = f32_to_f16_bits(R / levels);
      if ((lane & 15) == 0) {
        p.scales[so] = dh;
        p.mins[so] = mh;
      }
      d = f16_bits_to_f32(dh);
    }
    const uint32_t mask = (1u << bits) - 1u;
    uint32_t q0 = 0, q1 = 0;
    if (d != 0.f) {
      if (fam == FAM_0) {
        const float qmax = (float)((1 << (bits - 1)) - 1);
        q0 = (uint32_t)(int)fminf(fmaxf(rintf(a / d), -qmax), qmax);
        q1 = (uint32_t)(int)fminf(fmaxf(rintf(c / d), -qmax), qmax);
      } else {
        const float levels = (float)((1 << bits) - 1);
        q0 = (uint32_t)(int)fminf(fmaxf(rintf((a - m) / d), 0.f), levels);
        q1 = (uint32_t)(int)fminf(fmaxf(rintf((c - m) / d), 0.f), levels);
      }
    }
    const int K = 16 / bits;                       // lanes per dword
    uint32_t w = ((q0 & mask) | ((q1 & mask) << bits)) << (2 * bits * (lane % K));
    for (int o = 1; o < K; o <<= 1) w |= __shfl_xor(w, o, 64);
    if (lane % K == 0) {
      const int byte = 4 * (lane / K);
      *reinterpret_cast<uint32_t *>(row_codes + tiled_offset(t, byte / g.c, g.R, g.c) + byte % g.c) = w;
    }
    return;
  }
  // 3. block scale (and min), one lane per block
  if (lane < g.nblk) {
    const float *blk = coords + lane * g.L;
    const long long so = g.scales_off + (long long)t * g.nblk + lane;
    if (fam == FAM_0) {
      float amax = 0.f;
      for (int e = 0; e < g.L; ++e) amax = fmaxf(amax, fabsf(blk[e]));
      const float qmax = (float)((1 << (bits - 1)) - 1);
      uint16_t dh = f32_to_f16_bits(amax / qmax);
      p.scales[so] = dh;
      s_scale[lane] = f16_bits_to_f32(dh);
    } else {
      float lo = blk[0], hi = blk[0];
      for (int e = 1; e < g.L; ++e) {
        lo = fminf(lo, blk[e]);
        hi = fmaxf(hi, blk[e]);
      }
      uint16_t mh = f32_to_f16_bits(lo);
      const float m = f16_bits_to_f32(mh);
      const float R = hi - m;
      const float levels = (float)((1 << bits) - 1);
      uint16_t dh = f32_to_f16_bits(R / levels);
      p.scales[so] = dh;
      p.mins[so] = mh;
      s_scale[lane] = f16_bits_to_f32(dh);
      s_min[lane] = m;
    }
  }
  wave_sync();

  // 4. codes (masked to `bits` bits)
  const uint32_t mask = (1u << bits) - 1u;
  for (int e = lane; e < g.n; e += 64) {
    const int j = e / g.L;
    const float d = s_scale[j];
    int q = 0;
    if (fam == FAM_0) {
      const float qmax = (float)((1 << (bits - 1)) - 1);
      if (d != 0.f) q = (int)fminf(fmaxf(rintf(coords[e] / d), -qmax), qmax);
    } else {
      const float levels = (float)((1 << bits) - 1);
      const float y = coords[e] - s_min[j];
      if (d != 0.f) q = (int)fminf(fmaxf(rintf(y / d), 0.f), levels);
    }
    codes[e] = (uint8_t)((uint32_t)q & mask);
  }
  wave_sync();

  // 5. pack: unit u (us bytes) holds row bits [8*us*u, 8*us*(u+1))
  const int us = g.c < 4 ? g.c : 4;
  const int nunits = g.R / us;
  if (lane < nunits) {
    const int bit0 = 8 * us * lane, bit1 = bit0 + 8 * us;
    uint64_t acc = 0;
    for (int e = bit0 / bits; e < g.n && e * bits < bit1; ++e) {
      const int sh = e * bits - bit0;
      const uint64_t v = codes[e];
      acc |= sh >= 0 ? (v << sh) : (v >> (-sh));
    }
    const int byte = us * lane;
    uint8_t *dst = row_codes + tiled_offset(t, byte / g.c, g.R, g.c) + byte % g.c;
    if (us == 4)
      *reinterpret_cast<uint32_t *>(dst) = (uint32_t)acc;
    else if (us == 2)
      *reinterpret_cast<uint16_t *>(dst) = (uint16_t)acc;
    else
      *dst = (uint8_t)acc;
  }
}

// Items strided over a grid of 4-wave workgroups: far fewer workgroups
// than items, so a prefill-sized append is not bound by workgroup dispatch.
__global__ __launch_bounds__(256) void append_kernel(PlaneArgs kp, PlaneArgs vp,
                                                     const float *__restrict__ k_new,
                                                     const float *__restrict__ v_new, int n_new,
                                                     int t0, unsigned items) {
  __shared__ float xin[4][D];
  __shared__ float coords[4][D];
  __shared__ uint8_t codes[4][D];
  __shared__ float s_scale[4][4];
  __shared__ float s_min[4][4];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned stride = gridDim.x * 4u;
  // two items of prefetch per wave (loads past the end re-read the last item)
  auto load = [&](unsigned it) {
    const unsigned c = it < items ? it : items - 1;
    return reinterpret_cast<const float2 *>(item_src(kp, k_new, v_new, n_new, c))[lane];
  };
  unsigned item = blockIdx.x * 4u + w;
  float2 x0 = load(item), x1 = load(item + stride);
  for (; item < items; item += stride) {
    const float2 x = x0;
    x0 = x1;
    x1 = load(item + 2 * stride);
    append_item(kp, vp, n_new, t0, item, x, xin[w], coords[w], codes[w], s_scale[w], s_min[w]);
  }
}

hipError_t launch_append(const PlaneArgs &kp, const PlaneArgs &vp, const float *k_new,
                         const float *v_new, int batch, int n_new, int t0, hipStream_t stream) {
  const long long items = (long long)batch * n_new * kp.hkv * 2;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  long long blocks = (items + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kp, vp, k_new,
                     v_new, n_new, t0, (unsigned)items);
  return hipGetLastError();
}

}  // namespace kvq
