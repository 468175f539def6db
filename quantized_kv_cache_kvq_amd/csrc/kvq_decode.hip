// Decode attention over the packed cache: the launch of the split-K decode
// kernel (kvq_decode_impl.hpp, kvq_decode_q.hpp; KVarN and low-rank body
// workgroups transform the raw query themselves) and its event-timing hook.
//
// The computation (forum thread on decode bandwidth, second post): scores
// s_t = sm_scale <q, k_t>, softmax over t, output sum_t p_t v_t; the cache is
// read once per step, so the step is bound by HBM bandwidth (same thread,
// first post).  One launch does all of it: workgroups own context splits of
// a (batch entry, kv head, head group), write (m, l, o) partials, and the
// workgroup that finishes a unit last merges the splits (M = max m_s,
// L = sum l_s 2^(m_s - M), o = sum o_s 2^(m_s - M) / L) after taking body
// partials back to the raw basis (inverse Hadamard and 1/w for KVarN, P_h
// for low rank).
#include <vector>

#include "kvq_decode_impl.hpp"

namespace kvq {

// --------------------------------------------------------------- launcher --

int decode_tile_tokens(int kcodec, int vcodec, int basis) {
  (void)kcodec; (void)vcodec; (void)basis;
  return 64;   // one wave tile; a split owns whole multiples of it
}

int decode_head_group(int G) {
  const int cands[] = {8, 6, 4, 2, 1};
  for (int c : cands)
    if (G % c == 0) return c;
  return 1;
}

extern template hipError_t launch_decode_hg<1>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_hg<2>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_hg<4>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_hg<6>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);
extern template hipError_t launch_decode_hg<8>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);

bool decode_lowrank_supported(int codec, int rank) { return decode_lowrank_supported_impl(codec, rank); }

bool decode_pair_supported(int kc, int vc, int hg) {
  if (!(hg == 1 || hg == 2 || hg == 4 || hg == 6 || hg == 8)) return false;
#define KVQ_PAIR_CHECK(K, V) if (kc == K && vc == V) return true;
  KVQ_DECODE_PAIRS(KVQ_PAIR_CHECK)
#undef KVQ_PAIR_CHECK
  return false;
}

// Optional event timing of the split-K decode kernel: one start/stop pair
// per decode call, stamped by that kernel's own dispatch.
namespace {
struct Timing {
  std::vector<hipEvent_t> ev;  // 2 per slot
  int used = 0;
  bool on = false;
};
Timing g_timing;
}  // namespace

void timing_next(hipEvent_t *ev0, hipEvent_t *ev1) {
  Timing &T = g_timing;
  const bool free = T.on && 2 * T.used < (int)T.ev.size();
  *ev0 = free ? T.ev[2 * T.used] : nullptr;
  *ev1 = free ? T.ev[2 * T.used + 1] : nullptr;
}

void timing_commit() {
  Timing &T = g_timing;
  if (T.on && 2 * T.used < (int)T.ev.size()) ++T.used;
}

hipError_t timing_begin(int capacity) {
  (void)timing_end(nullptr, nullptr);
  Timing &T = g_timing;
  T.ev.assign(2 * (size_t)capacity, nullptr);
  for (auto &e : T.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      e = nullptr;
      (void)timing_end(nullptr, nullptr);
      return r;
    }
  }
  T.used = 0;
  T.on = true;
  return hipSuccess;
}

hipError_t timing_durations(float *ms, int capacity, int *count) {
  Timing &T = g_timing;
  hipError_t err = hipSuccess;
  const int n = T.used < capacity ? T.used : capacity;
  for (int i = 0; i < n; ++i) {
    float x = 0.f;
    hipError_t r = hipEventSynchronize(T.ev[2 * i + 1]);
    if (r == hipSuccess) r = hipEventElapsedTime(&x, T.ev[2 * i], T.ev[2 * i + 1]);
    if (r != hipSuccess && err == hipSuccess) err = r;
    ms[i] = x;
  }
  *count = n;
  return err;
}

hipError_t timing_end(double *total_ms, int *count) {
  Timing &T = g_timing;
  double sum = 0.0;
  hipError_t err = hipSuccess;
  for (int i = 0; i < T.used; ++i) {
    float ms = 0.f;
    hipError_t r = hipEventSynchronize(T.ev[2 * i + 1]);
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, T.ev[2 * i], T.ev[2 * i + 1]);
    if (r != hipSuccess && err == hipSuccess) err = r;
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (count) *count = T.used;
  for (auto e : T.ev)
    if (e) (void)hipEventDestroy(e);
  T.ev.clear();
  T.used = 0;
  T.on = false;
  return err;
}

hipError_t launch_decode(const DecodeArgs &args, const float *q, float sm_scale, float *out,
                         hipStream_t stream) {
  DecodeArgs a = args;
  const float scale2 = sm_scale * LOG2E;
  // plain bodies scale the raw query themselves; KVarN and low-rank body
  // workgroups transform it first (rotation / projection), into LDS
  a.q_body = q;
  a.scale_body = scale2;
  a.q_tail = q;
  a.scale_tail = scale2;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  hipError_t r;
  hipEvent_t ev0, ev1;
  timing_next(&ev0, &ev1);
  switch (a.HG) {
    case 1: r = launch_decode_hg<1>(a, stream, ev0, ev1); break;
    case 2: r = launch_decode_hg<2>(a, stream, ev0, ev1); break;
    case 4: r = launch_decode_hg<4>(a, stream, ev0, ev1); break;
    case 6: r = launch_decode_hg<6>(a, stream, ev0, ev1); break;
    case 8: r = launch_decode_hg<8>(a, stream, ev0, ev1); break;
    default: r = hipErrorNotSupported;
  }
  if (r != hipSuccess) return r;
  if (ev0) timing_commit();
  (void)out;   // merged into a.out by each unit's last workgroup
  return hipGetLastError();
}

}  // namespace kvq
