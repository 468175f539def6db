// Layer transcode (VBR degrade step): decode every body row with the source
// codec and re-encode it with the destination codec, out of place.
//
// The VBR announcement thread (opening posts) describes a cache that starts
// at 16 bits and moves layers to lower-precision codecs as the context grows;
// this kernel is that move for one layer.  Decoding gives the binary32 value
// a reader sees (q*d for _0, fma(u, d, m) for _1, the binary16 value for
// F16); encoding is the append kernel's block quantiser, so a transcoded row
// equals the row the destination codec would have stored for those values.
//
// One thread per (token, 32-channel block): a block's source field and
// destination field are whole dwords in every codec (4*b bytes), so each
// thread reads and writes only its own dwords.  A wave covers 16 tokens x 4
// blocks; consecutive waves walk consecutive tokens of a plane.
#include "kvq_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {

template <int BITS, bool SIGNED>
__device__ __forceinline__ int get_field(const uint32_t *w, int bit) {
  const int wi = bit >> 5, sh = bit & 31;
  uint32_t lo = w[wi] >> sh;
  if (sh + BITS > 32) lo |= w[wi + 1] << (32 - sh);
  if (SIGNED) return ((int32_t)(lo << (32 - BITS))) >> (32 - BITS);
  return (int)(lo & ((1u << BITS) - 1u));
}

// Decode block j of token t into x[32].
template <int SC>
__device__ __forceinline__ void decode_block(const PlaneArgs &p, const HeadGeom &g, long long t,
                                             int j, float (&x)[32]) {
  constexpr int fam = codec_family(SC), bits = codec_bits(SC);
  constexpr int R = row_bytes(SC, D), C = chunk_bytes(R);
  constexpr int FB = fam == FAM_F16 ? 64 : 4 * bits;    // field bytes of a block
  uint32_t w[16];
  const uint8_t *base = p.codes + g.codes_off;
#pragma unroll
  for (int i = 0; i < FB / 4; ++i) {
    const int byte = j * FB + 4 * i;
    w[i] = *reinterpret_cast<const uint32_t *>(base + tiled_offset(t, byte / C, R, C) + byte % C);
  }
  if constexpr (fam == FAM_F16) {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = f16_bits_to_f32((uint16_t)((w[e >> 1] >> (16 * (e & 1))) & 0xFFFF));
  } else {
    const long long so = g.scales_off + t * (D / 32) + j;
    const float d = f16_bits_to_f32(p.scales[so]);
    if constexpr (fam == FAM_0) {
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = (float)get_field<bits, true>(w, e * bits) * d;
    } else {
      const float m = f16_bits_to_f32(p.mins[so]);
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = fmaf((float)get_field<bits, false>(w, e * bits), d, m);
    }
  }
}

// Encode x[32] as block j of token t.
template <int DC>
__device__ __forceinline__ void encode_block(const PlaneArgs &p, const HeadGeom &g, long long t,
                                             int j, const float (&x)[32]) {
  constexpr int fam = codec_family(DC), bits = codec_bits(DC);
  constexpr int R = row_bytes(DC, D), C = chunk_bytes(R);
  constexpr int FB = fam == FAM_F16 ? 64 : 4 * bits;
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = 0u;
  if constexpr (fam == FAM_F16) {
#pragma unroll
    for (int e = 0; e < 32; ++e) w[e >> 1] |= (uint32_t)f32_to_f16_bits(x[e]) << (16 * (e & 1));
  } else {
    const long long so = g.scales_off + t * (D / 32) + j;
    uint32_t codes[32];
    if constexpr (fam == FAM_0) {
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
      const float qmax = (float)((1 << (bits - 1)) - 1);
      const uint16_t dh = f32_to_f16_bits(amax / qmax);
      const float d = f16_bits_to_f32(dh);
      p.scales[so] = dh;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        int q = d != 0.f ? (int)fminf(fmaxf(rintf(x[e] / d), -qmax), qmax) : 0;
        codes[e] = (uint32_t)q & ((1u << bits) - 1u);
      }
    } else {
      float lo = x[0], hi = x[0];
#pragma unroll
      for (int e = 1; e < 32; ++e) {
        lo = fminf(lo, x[e]);
        hi = fmaxf(hi, x[e]);
      }
      const uint16_t mh = f32_to_f16_bits(lo);
      const float m = f16_bits_to_f32(mh);
      const float levels = (float)((1 << bits) - 1);
      const uint16_t dh = f32_to_f16_bits((hi - m) / levels);
      const float d = f16_bits_to_f32(dh);
      p.scales[so] = dh;
      p.mins[so] = mh;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float y = x[e] - m;
        int q = d != 0.f ? (int)fminf(fmaxf(rintf(y / d), 0.f), levels) : 0;
        codes[e] = (uint32_t)q;
      }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int bit = e * bits;
      w[bit >> 5] |= codes[e] << (bit & 31);
      if ((bit & 31) + bits > 32) w[(bit >> 5) + 1] |= codes[e] >> (32 - (bit & 31));
    }
  }
  uint8_t *base = p.codes + g.codes_off;
#pragma unroll
  for (int i = 0; i < FB / 4; ++i) {
    const int byte = j * FB + 4 * i;
    *reinterpret_cast<uint32_t *>(base + tiled_offset(t, byte / C, R, C) + byte % C) = w[i];
  }
}

template <int SC, int DC>
__global__ __launch_bounds__(256) void transcode_kernel(PlaneArgs src, PlaneArgs dst, int T,
                                                        long long total) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int j = (int)(gid & 3);
  long long r = gid >> 2;
  const long long t = r % T;
  r /= T;
  const int h = (int)(r % src.hkv);
  const int b = (int)(r / src.hkv);
  float x[32];
  decode_block<SC>(src, head_geom(src, b, h), t, j, x);
  encode_block<DC>(dst, head_geom(dst, b, h), t, j, x);
}

template <int SC>
static hipError_t dispatch_dst(const PlaneArgs &s, const PlaneArgs &d, int T, long long total,
                               hipStream_t st) {
  const dim3 grid((unsigned)((total + 255) / 256));
  switch (d.codec) {
#define KVQ_DST(DC)                                                                        \
  case DC:                                                                                  \
    hipLaunchKernelGGL((transcode_kernel<SC, DC>), grid, dim3(256), 0, st, s, d, T, total); \
    break;
    KVQ_DST(KVQ_F16) KVQ_DST(KVQ_Q8_0) KVQ_DST(KVQ_Q6_0) KVQ_DST(KVQ_Q5_0) KVQ_DST(KVQ_Q4_0)
    KVQ_DST(KVQ_Q3_0) KVQ_DST(KVQ_Q2_0) KVQ_DST(KVQ_Q8_1) KVQ_DST(KVQ_Q6_1) KVQ_DST(KVQ_Q5_1)
    KVQ_DST(KVQ_Q4_1) KVQ_DST(KVQ_Q3_1) KVQ_DST(KVQ_Q2_1) KVQ_DST(KVQ_Q1_1)
#undef KVQ_DST
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_transcode(const PlaneArgs &src, const PlaneArgs &dst, int batch, int T,
                            hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const long long total = (long long)batch * src.hkv * T * 4;
  switch (src.codec) {
#define KVQ_SRC(SC) \
  case SC: return dispatch_dst<SC>(src, dst, T, total, stream);
    KVQ_SRC(KVQ_F16) KVQ_SRC(KVQ_Q8_0) KVQ_SRC(KVQ_Q6_0) KVQ_SRC(KVQ_Q5_0) KVQ_SRC(KVQ_Q4_0)
    KVQ_SRC(KVQ_Q3_0) KVQ_SRC(KVQ_Q2_0) KVQ_SRC(KVQ_Q8_1) KVQ_SRC(KVQ_Q6_1) KVQ_SRC(KVQ_Q5_1)
    KVQ_SRC(KVQ_Q4_1) KVQ_SRC(KVQ_Q3_1) KVQ_SRC(KVQ_Q2_1) KVQ_SRC(KVQ_Q1_1)
#undef KVQ_SRC
    default: return hipErrorNotSupported;
  }
}

}  // namespace kvq
