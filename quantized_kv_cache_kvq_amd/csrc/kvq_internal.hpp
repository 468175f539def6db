// Internal host-side interface between the C ABI and the kernel launchers.
#pragma once

#include "kvq_common.hpp"

namespace kvq {

// Partial result of one context split for one query head:
// {m (log2 domain), l, pad, pad, o[128]}.
constexpr int PSTRIDE = 132;

struct DecodePlan {
  int B, Hkv, Hq, G, HG, NHG;     // HG heads per workgroup, NHG = G / HG
  int T, body_tokens, tail_tokens;
  int tt_body;                    // tokens per workgroup tile of the body
  int S_body, S_tail, S_total;    // context splits per (b, kv head, head group)
  int tiles_per_split_body, tiles_per_split_tail;
};

// Kernel arguments of the split-K decode.  The scalars and pointers every
// workgroup reads before its first load come first, so they share the first
// lines of the argument buffer; the plane descriptions (with the low-rank
// tables) follow.
struct DecodeArgs {
  int S_tail, S_body, S_total;    // context splits per (b, kv head, head group)
  int NHG, HG, G;                 // head groups per kv head, heads per group, GQA group
  int B, Hkv, Hq;
  int body_tokens, tail_tokens;
  int tps_body, tps_tail;         // 64-token tiles per split
  int tt_body;
  float scale_body;               // multiplier taking body scores to the log2 domain
  float scale_tail;
  const float *q_body;    // [B][Hq][128] raw query (KVarN / low-rank bodies transform it in LDS)
  const float *q_tail;    // [B][Hq][128] raw query
  float *part;            // [B][Hq][S_total][PSTRIDE]
  float *out;             // [B][Hq][128] final output
  unsigned *cnt;          // [B][Hkv][NHG] finished-split counters (zero between calls)
  const int32_t *seq;     // ragged batch: tokens of each sequence (null: all T)
  int seq_add;            // added to every seq entry (1 when a token was just appended)
  int T, N;               // tokens (maximum over sequences), tail length
  const float *k_new;     // fused step (non-null): the new token's K and V rows
  const float *v_new;     // [B][Hkv][128], written before the decode reads
  PlaneArgs k, v;
  int16_t lr_sbody[MAXLR];  // low rank: body splits of kv head h (S_body is the largest)
  int16_t lr_tps[MAXLR];    // low rank: body tiles per split of kv head h
  int16_t lr_first[MAXLR];  // low rank: grid x of kv head h's first body split
  int lr_body_all;          // low rank: body splits of all kv heads
};

hipError_t launch_append(const PlaneArgs &kp, const PlaneArgs &vp, const float *k_new,
                         const float *v_new, int batch, int n_new, int t0, const int32_t *seq,
                         hipStream_t stream);

// Raw-basis binary32 view of plane p, out[B][T][hkv][128]; the newest
// min(tail_len, T_b) tokens of sequence b come from the tail ring, rows
// past T_b (ragged batch, seq non-null) are zero.
hipError_t launch_dequant(const PlaneArgs &p, int batch, int T, const int32_t *seq, float *out,
                          hipStream_t stream);

hipError_t launch_transcode(const PlaneArgs &src, const PlaneArgs &dst, int batch, int T,
                            hipStream_t stream);

hipError_t launch_decode(const DecodeArgs &a, const float *q, float sm_scale, float *out,
                         hipStream_t stream);

// Status with detail for kvq_last_error (host).
kvq_status api_fail(kvq_status s, const char *detail);
kvq_status api_ok();

// Event timing of the split-K decode kernel (host side, not thread safe).
hipError_t timing_begin(int capacity);
hipError_t timing_end(double *total_ms, int *count);
// Elapsed milliseconds of each recorded pair (at most capacity), in launch order.
hipError_t timing_durations(float *ms, int capacity, int *count);
// Next free event pair (nulls when timing is off or the pool is used up);
// timing_commit() marks it used once the launch went through.
void timing_next(hipEvent_t *ev0, hipEvent_t *ev1);
void timing_commit();

// Split-K decode workgroups: waves per workgroup and workgroups resident
// per CU (the split policy sizes one round of workgroups from these).
constexpr int DECODE_WG_WAVES = 8;
// Completion counters at the start of every decode workspace, spread over
// DECODE_CNT_PAGES pages of 4 KB.
constexpr int DECODE_MAX_UNITS = 16384;
constexpr int DECODE_CNT_PAGES = 16;
constexpr size_t DECODE_CNT_BYTES = DECODE_MAX_UNITS * sizeof(unsigned);
static_assert(DECODE_CNT_BYTES == DECODE_CNT_PAGES * 4096, "counter pages are 4 KB");
constexpr int DECODE_WG_PER_CU = 1;

int decode_tile_tokens(int kcodec, int vcodec, int basis);
int decode_head_group(int G);
bool decode_lowrank_supported(int codec, int rank);
bool decode_pair_supported(int kcodec, int vcodec, int hg);

template <int HG>
hipError_t launch_decode_hg(const DecodeArgs &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace kvq
