// Shared definitions of the HIP library: codec traits, plane addressing and
// the kernel-side plane description.  Included by every translation unit.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int D = KVQ_HEAD_DIM;
constexpr int TILE = KVQ_TILE_TOKENS;
constexpr int MAXLR = KVQ_MAX_LOWRANK_HEADS;

enum Family { FAM_F16 = 0, FAM_0 = 1, FAM_1 = 2 };

__host__ __device__ constexpr int codec_bits(int c) {
  return c == KVQ_F16 ? 16
       : c == KVQ_Q8_0 || c == KVQ_Q8_1 ? 8
       : c == KVQ_Q6_0 || c == KVQ_Q6_1 ? 6
       : c == KVQ_Q5_0 || c == KVQ_Q5_1 ? 5
       : c == KVQ_Q4_0 || c == KVQ_Q4_1 ? 4
       : c == KVQ_Q3_0 || c == KVQ_Q3_1 ? 3
       : c == KVQ_Q2_0 || c == KVQ_Q2_1 ? 2 : 1;
}

__host__ __device__ constexpr int codec_family(int c) {
  return c == KVQ_F16 ? FAM_F16 : (c >= KVQ_Q8_0 && c <= KVQ_Q2_0) ? FAM_0 : FAM_1;
}

// Row size in bytes of n coordinates.
__host__ __device__ constexpr int row_bytes(int c, int n) {
  return codec_family(c) == FAM_F16 ? 2 * n : n * codec_bits(c) / 8;
}

// Chunk size of the 64-token tiled layout: largest of 16, 8, 4, 2, 1 dividing R.
__host__ __device__ constexpr int chunk_bytes(int R) {
  return R % 16 == 0 ? 16 : R % 8 == 0 ? 8 : R % 4 == 0 ? 4 : R % 2 == 0 ? 2 : 1;
}

__host__ __device__ constexpr int block_len(int n) { return n < 32 ? n : 32; }

// Byte offset of chunk k of token t inside a plane with R-byte rows.
__host__ __device__ inline long long tiled_offset(long long t, int k, int R, int c) {
  return (t / TILE) * (long long)TILE * R + ((long long)k * TILE + (t % TILE)) * c;
}

// Kernel-side description of one plane (K or V of one layer).  For the
// low-rank basis every head has its own width and codec; plane offsets are
// prefix sums over heads, recomputed on the fly from the small tables.
struct PlaneArgs {
  uint8_t *codes;
  uint16_t *scales;
  uint16_t *mins;
  uint16_t *tail;
  const float *w;
  const uint16_t *proj;
  int codec;          // uniform codec (plain / hadamard)
  int basis;
  int hkv;
  int capacity;
  int tail_len;
  int tail_bf16;      // tail rows are bfloat16 (else binary16)
  int8_t hcodec[MAXLR];   // low-rank: codec of head h
  int16_t hrank[MAXLR];   // low-rank: width of head h
  // low-rank: per token, row bytes and scale blocks of the heads before h,
  // and of all heads (a plane's offsets are prefix sums over heads)
  int32_t hrow_before[MAXLR];
  int32_t hblk_before[MAXLR];
  int32_t row_all;
  int32_t blk_all;
};

struct HeadGeom {
  int codec, n, R, c, nblk, L;
  long long codes_off;    // bytes from `codes`
  long long scales_off;   // binary16 elements from `scales` / `mins`
};

// Geometry of plane (b, h).
__host__ __device__ inline HeadGeom head_geom(const PlaneArgs &p, int b, int h) {
  HeadGeom g;
  if (p.basis != KVQ_BASIS_LOWRANK) {
    g.codec = p.codec;
    g.n = D;
    g.R = row_bytes(g.codec, D);
    g.c = chunk_bytes(g.R);
    g.L = 32;
    g.nblk = codec_family(g.codec) == FAM_F16 ? 0 : D / 32;
    long long plane = (long long)b * p.hkv + h;
    g.codes_off = plane * p.capacity * g.R;
    g.scales_off = plane * p.capacity * g.nblk;
    return g;
  }
  g.codec = p.hcodec[h];
  g.n = p.hrank[h];
  g.R = row_bytes(g.codec, g.n);
  g.c = chunk_bytes(g.R);
  g.L = block_len(g.n);
  g.nblk = g.n / g.L;
  g.codes_off = (long long)p.capacity * ((long long)b * p.row_all + p.hrow_before[h]);
  g.scales_off = (long long)p.capacity * ((long long)b * p.blk_all + p.hblk_before[h]);
  return g;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Load of data that one call streams once (cache codes and scales): marked
// non-temporal, so the stream does not push reused lines (code, arguments,
// split partials) out of the caches.
template <class T>
__device__ __forceinline__ T ld_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T *>(p));
}

// Binary16 <-> binary32 with round-to-nearest-even.
__device__ inline uint16_t f32_to_f16_bits(float x) {
  return __half_as_ushort(__float2half_rn(x));
}
__device__ inline float f16_bits_to_f32(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

// Binary32 <-> bfloat16: round to nearest, ties to even, on the 16 bits
// dropped (finite inputs; a carry into the exponent is the correct result).
__device__ inline uint16_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Raw-vector tail element of a plane from its 16 stored bits.
__device__ inline float tail_to_f32(uint16_t bits, bool bf16) {
  return bf16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
}

}  // namespace kvq
