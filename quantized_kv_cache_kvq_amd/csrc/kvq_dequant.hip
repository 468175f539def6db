// Dequantize a plane: the binary32 vectors decode attention attends over,
// in the raw (input) basis, for every stored token of every (batch, kv head).
//
// A reader of the cache sees, for token t of n tokens:
//  - the 16-bit tail ring slot t mod tail_len when t is one of the newest
//    min(tail_len, n) tokens (BeeLlama.cpp v0.4.0 release notes, precision
//    tail section);
//  - otherwise the block-coded row decoded (q*d for _0, fma(u, d, m) for _1,
//    the binary16 value for F16) and taken back to the raw basis:
//      KVarN (same release notes, KVarN section): x = (H y / 128) / w, H the
//        order-128 Sylvester Hadamard matrix (H H = 128 I);
//      low rank (KV-COBRA explainer, rank and bits per head): x = P_h u.
// Decode's scores and outputs equal those of plain attention over these
// vectors (q . P u = (P^T q) . u, q . (H y / 128) / w = (H (q / w) / 128) . y).
//
// One wave per (b, t, kv head) row; lane l holds stored coordinates 2l and
// 2l + 1.  Throughput is not a goal: this is the cache's read-back view
// (quality measurement, inspection).
#include "kvq_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {

namespace {

constexpr int DQ_WAVES = 4;

// Code (or binary16 bits) of stored coordinate c of token t in a plane with
// geometry g: gathered bytewise from the 64-token tiled layout.
__device__ inline uint32_t field_of(const uint8_t *base, const HeadGeom &g, long long t, int c,
                                    int bits) {
  const int bit0 = c * bits;
  uint32_t v = 0;
  const int b0 = bit0 >> 3, b1 = (bit0 + bits - 1) >> 3;
  for (int b = b0; b <= b1; ++b)
    v |= (uint32_t)base[tiled_offset(t, b / g.c, g.R, g.c) + b % g.c] << (8 * (b - b0));
  v >>= bit0 & 7;
  return bits == 32 ? v : v & ((1u << bits) - 1u);
}

__global__ __launch_bounds__(64 * DQ_WAVES) void dequant_kernel(PlaneArgs p, int T,
                                                                const int32_t *__restrict__ seq,
                                                                float *__restrict__ out) {
  __shared__ float coords[DQ_WAVES][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * DQ_WAVES + wave;
  const int h = blockIdx.y, b = blockIdx.z;
  if (t >= T) return;
  int Tb = T;                                      // this sequence's tokens
  if (seq) {
    const int s = seq[b];
    Tb = s < 0 ? 0 : s > T ? T : s;
  }
  const int n_tail = p.tail_len < Tb ? p.tail_len : Tb;
  float x0 = 0.f, x1 = 0.f;
  if (t >= Tb) {
    // past this sequence's tokens: zeros
  } else if (t >= Tb - n_tail) {
    // 16-bit ring row: 256-byte rows in the tiled layout (16-byte chunks)
    const long long plane = (long long)b * p.hkv + h;
    const uint8_t *ring = reinterpret_cast<const uint8_t *>(p.tail) + plane * p.tail_len * (2 * D);
    const int slot = t % p.tail_len, byte = 4 * lane;
    const uint32_t w =
        *reinterpret_cast<const uint32_t *>(ring + tiled_offset(slot, byte / 16, 2 * D, 16) + byte % 16);
    x0 = tail_to_f32((uint16_t)(w & 0xFFFF), p.tail_bf16);
    x1 = tail_to_f32((uint16_t)(w >> 16), p.tail_bf16);
  } else {
    const HeadGeom g = head_geom(p, b, h);
    const int fam = codec_family(g.codec), bits = codec_bits(g.codec);
    const uint8_t *base = p.codes + g.codes_off;
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 2 * lane + e;
      float val = 0.f;
      if (c < g.n) {
        const uint32_t f = field_of(base, g, t, c, bits);
        if (fam == FAM_F16) {
          val = f16_bits_to_f32((uint16_t)f);
        } else {
          const long long so = g.scales_off + t * g.nblk + c / g.L;
          const float d = f16_bits_to_f32(p.scales[so]);
          if (fam == FAM_0) {
            const int q = (int)(f << (32 - bits)) >> (32 - bits);
            val = (float)q * d;
          } else {
            val = fmaf((float)f, d, f16_bits_to_f32(p.mins[so]));
          }
        }
      }
      v[e] = val;
    }
    x0 = v[0];
    x1 = v[1];
    if (p.basis == KVQ_BASIS_HADAMARD) {
      // H y with coordinate index bit 0 inside the lane, bits 1..6 across lanes
      float a0 = x0 + x1, a1 = x0 - x1;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float p0 = __shfl_xor(a0, m, 64), p1 = __shfl_xor(a1, m, 64);
        const bool upper = (lane & m) != 0;
        a0 = upper ? (p0 - a0) : (a0 + p0);
        a1 = upper ? (p1 - a1) : (a1 + p1);
      }
      const float *w = p.w + (long long)h * D;
      x0 = a0 * (1.f / 128.f) / w[2 * lane];
      x1 = a1 * (1.f / 128.f) / w[2 * lane + 1];
    } else if (p.basis == KVQ_BASIS_LOWRANK) {
      coords[wave][2 * lane] = x0;
      coords[wave][2 * lane + 1] = x1;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint16_t *P = p.proj + (long long)h * D * D;
      float y0 = 0.f, y1 = 0.f;
      for (int k = 0; k < g.n; ++k) {
        y0 = fmaf(f16_bits_to_f32(P[(long long)(2 * lane) * D + k]), coords[wave][k], y0);
        y1 = fmaf(f16_bits_to_f32(P[(long long)(2 * lane + 1) * D + k]), coords[wave][k], y1);
      }
      x0 = y0;
      x1 = y1;
    }
  }
  float2 *dst = reinterpret_cast<float2 *>(out + (((long long)b * T + t) * p.hkv + h) * D);
  dst[lane] = make_float2(x0, x1);
}

}  // namespace

hipError_t launch_dequant(const PlaneArgs &p, int batch, int T, const int32_t *seq, float *out,
                          hipStream_t stream) {
  const dim3 grid((unsigned)((T + DQ_WAVES - 1) / DQ_WAVES), (unsigned)p.hkv, (unsigned)batch);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(64 * DQ_WAVES), 0, stream, p, T, seq, out);
  return hipGetLastError();
}

}  // namespace kvq
