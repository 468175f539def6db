/*
 * kvq.h - packed low-bit KV cache and single-query decode attention on
 * AMD Instinct MI355X (gfx950).  C ABI of libkvq.so.
 *
 * What the library computes (sources are the pages this format follows):
 *
 *  - Block codecs.  The BeeLlama.cpp v0.4.0 release notes (new standard KV
 *    cache types) name the family: q8/q6/q5/q4/q3/q2 in an absmax "_0" and a
 *    min-offset "_1" flavour.  A block is 32 consecutive channels of one
 *    token of one (batch, kv head) with one binary16 scale (plus one binary16
 *    min for _1):
 *      _0: d = RN16(amax/qmax), qmax = 2^(b-1)-1, q = clamp(rne(x/d), +-qmax)
 *      _1: m = RN16(min x), y = RN32(x-m), d = RN16(RN32(max x - m)/(2^b-1)),
 *          u = clamp(rne(y/d), 0, 2^b-1); value RN32(u*d + m)
 *    (all quotients exact, ties to even; d == 0 gives zero codes).
 *  - Precision tail (same release notes, precision-tail section): the newest
 *    tail_len tokens are also kept as binary16 in a ring (token t in slot
 *    t mod tail_len) and decode reads them from there; codes are written for
 *    every token at append time.
 *  - KVarN basis (same release notes, KVarN section; KV-COBRA explainer,
 *    jargon on the Hadamard rotation): stored coordinates are
 *    y = H (x * w) with w = 1/sigma per channel (caller-supplied) and H the
 *    unnormalised order-128 Sylvester Hadamard matrix.
 *  - Low-rank basis (KV-COBRA explainer: per-head rank and bits, rotation
 *    fused into the projection): stored coordinates are u = P_h^T x with a
 *    caller-supplied binary16 P_h (128 x rank_h), coded with a per-head codec
 *    on blocks of min(32, rank_h); attention runs in rank space.
 *  - Per-layer codecs and transcoding (VBR announcement thread, opening
 *    posts): each layer and each of K/V carries its own codec; a layer can be
 *    re-encoded to another codec as the session grows.
 *  - Decode attention (forum thread on decode bandwidth, second post): the
 *    newest query is dotted with every cached key, softmax over the scores,
 *    weighted sum of the cached values.  Query head h reads kv head
 *    h / (n_q_heads / n_kv_heads).
 *
 * Conventions for every entry point:
 *  - Every pointer in a descriptor is device memory owned by the caller,
 *    except kvq_plane.rank and kvq_plane.head_codec (host arrays).
 *  - The library never allocates, frees or synchronises; work is enqueued on
 *    `stream` (a hipStream_t, NULL = the default stream) and runs
 *    asynchronously.  Descriptors are read, never modified.
 *  - All checks run on the host before anything is enqueued: on any error
 *    nothing is launched and the status says why (detail in kvq_last_error).
 *    A failed launch returns KVQ_ERR_HIP.
 *  - Values that are NaN/Inf or large enough to overflow a binary16 scale
 *    (|x| > 65504*qmax) are outside the contract and not detected.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 2
#define KVQ_HEAD_DIM 128        /* the only supported head_dim */
#define KVQ_TILE_TOKENS 64      /* capacity and tail_len are multiples of this */
#define KVQ_MAX_LOWRANK_HEADS 32
/* Largest capacity and tail_len (tokens per plane).  Kernels address a
 * token inside one (batch, kv head) plane with 32-bit offsets: 2^24 rows of
 * at most 256 bytes (a binary16 row) stay below 2^32.  Larger layers are
 * rejected with KVQ_ERR_INVALID_ARG before anything is enqueued. */
#define KVQ_MAX_CAPACITY (1 << 24)

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = 1,    /* null pointer, bad shape, bad enum value */
    KVQ_ERR_UNSUPPORTED = 2,    /* valid but unsupported combination */
    KVQ_ERR_CAPACITY = 3,       /* n_tokens + n_new > capacity */
    KVQ_ERR_WORKSPACE = 4,      /* workspace missing or too small */
    KVQ_ERR_HIP = 5             /* a HIP launch failed */
} kvq_status;

typedef enum kvq_codec {
    KVQ_F16 = 0,
    KVQ_Q8_0 = 1, KVQ_Q6_0 = 2, KVQ_Q5_0 = 3, KVQ_Q4_0 = 4, KVQ_Q3_0 = 5, KVQ_Q2_0 = 6,
    KVQ_Q8_1 = 7, KVQ_Q6_1 = 8, KVQ_Q5_1 = 9, KVQ_Q4_1 = 10, KVQ_Q3_1 = 11, KVQ_Q2_1 = 12,
    KVQ_Q1_1 = 13,
    KVQ_NUM_CODECS = 14
} kvq_codec;

typedef enum kvq_basis {
    KVQ_BASIS_PLAIN = 0,        /* channels as given */
    KVQ_BASIS_HADAMARD = 1,     /* y = H (x * w)      (KVarN) */
    KVQ_BASIS_LOWRANK = 2       /* u = P_h^T x        (KV-COBRA style) */
} kvq_basis;

/*
 * One of K or V of one layer.
 *
 * Device layout (capacity C, B batch entries, Hkv kv heads; one "plane" per
 * (batch entry, kv head) in that order):
 *  - codes: each plane holds C rows; a row is one token's n stored
 *    coordinates (n = 128, or rank_h for LOWRANK) as a little-endian
 *    bitstream, coordinate e at bits [e*b, e*b+b) (_0 codes two's
 *    complement, _1 unsigned), or n binary16 values for KVQ_F16.  Rows are
 *    tiled by 64 tokens: with R the row size in bytes and c the largest of
 *    16, 8, 4, 2, 1 dividing R, chunk k (c bytes) of token t is at byte
 *    (t/64)*64*R + (k*64 + t%64)*c of the plane.  Planes are back to back
 *    (LOWRANK planes have per-head sizes, in (batch, head) order).
 *  - scales / mins: binary16 bit patterns, per plane [C][n/L] token-major
 *    (L = 32, or min(32, rank_h)); mins only for _1 codecs (NULL otherwise);
 *    both NULL for KVQ_F16.
 *  - tail: 16-bit rows (binary16 or bfloat16, kvq_layer.tail_format) of the
 *    raw (unrotated, unprojected) vectors, [B][Hkv] planes of tail_len rows
 *    in the same 64-token tiled layout (R = 256).  NULL when tail_len == 0.
 * Sizes: kvq_plane_bytes.
 */
typedef struct kvq_plane {
    int32_t codec;              /* kvq_codec (ignored for LOWRANK) */
    int32_t basis;              /* kvq_basis */
    void *codes;
    uint16_t *scales;
    uint16_t *mins;
    uint16_t *tail;
    const float *w;             /* HADAMARD: [Hkv][128] binary32 1/sigma */
    const uint16_t *proj;       /* LOWRANK: [Hkv][128][128] binary16, head h
                                   uses columns [0, rank[h]) */
    const int32_t *rank;        /* LOWRANK, host [Hkv]: 16, 32, 64 or 128 */
    const int32_t *head_codec;  /* LOWRANK, host [Hkv]: kvq_codec of head h
                                   (_0 or _1; not F16) */
} kvq_plane;

/* Element type of the precision-tail rows (release notes, precision-tail
 * section: the newest tokens are kept in BF16 or F16).  Both K and V tails of
 * a layer use it.  Conversions from binary32 round to nearest, ties to even. */
typedef enum kvq_tail_format {
    KVQ_TAIL_F16 = 0,           /* binary16 */
    KVQ_TAIL_BF16 = 1           /* bfloat16 (binary32 with 16 low bits dropped) */
} kvq_tail_format;

typedef struct kvq_layer {
    kvq_plane k, v;
    int32_t batch;              /* B >= 1 */
    int32_t n_kv_heads;         /* Hkv >= 1 (<= 32 for LOWRANK) */
    int32_t head_dim;           /* must be 128 */
    int32_t capacity;           /* rows per plane, multiple of 64, <= KVQ_MAX_CAPACITY */
    int32_t tail_len;           /* N, multiple of 64, 0 = no tail, <= KVQ_MAX_CAPACITY */
    int32_t n_tokens;           /* T tokens already cached, 0 <= T <= capacity */
    int32_t tail_format;        /* kvq_tail_format of both tails */
    const int32_t *seq_tokens;  /* NULL, or device [batch]: tokens of each
                                   sequence (ragged batch), each in
                                   [0, n_tokens]; n_tokens is then their
                                   maximum.  See the entry points. */
} kvq_layer;

/* Byte sizes of the device buffers of K (which = 0) or V (which = 1):
 * codes, scales, mins (0 when absent) and tail (0 when tail_len == 0).
 * Any output pointer may be NULL. */
kvq_status kvq_plane_bytes(const kvq_layer *layer, int32_t which, size_t *codes_bytes,
                           size_t *scales_bytes, size_t *mins_bytes, size_t *tail_bytes);

/* Append n_new >= 1 tokens at positions n_tokens .. n_tokens+n_new-1 (with
 * seq_tokens: sequence b at seq_tokens[b] .. seq_tokens[b]+n_new-1).
 * k_new, v_new: device binary32 [B][n_new][Hkv][128].  Writes body codes,
 * scales, mins of every new token and, when tail_len > 0, its 16-bit copy
 * into tail slot t mod tail_len (the newest token wins a slot).  The caller
 * advances n_tokens (and seq_tokens) afterwards.  KVQ_ERR_CAPACITY if
 * n_tokens + n_new exceeds capacity; a sequence position past the capacity
 * (a seq_tokens value above n_tokens breaks the contract) writes nothing. */
kvq_status kvq_quantize_append(const kvq_layer *layer, const float *k_new, const float *v_new,
                               int32_t n_new, void *stream);

/* Read back plane `which` (0 = K, 1 = V) as the binary32 vectors decode
 * attention attends over, in the raw (input) basis:
 * out[b][t][h][0..127] for t < n_tokens, float32 [batch][n_tokens][n_kv_heads]
 * [128] in device memory (caller-owned, written whole).  The newest
 * min(tail_len, n_tokens) tokens are their binary16 tail-ring copies
 * (release notes, precision-tail section); the others are decoded rows (q*d,
 * fma(u, d, m), or the binary16 value) taken back to the raw basis: KVarN
 * x = (H y / 128) / w (release notes, KVarN section; H H = 128 I), low rank
 * x = P_h u (KV-COBRA explainer; coordinates past rank_h are zero).  With
 * seq_tokens, rows t >= seq_tokens[b] of sequence b are written as zeros.
 * Decode's output equals plain softmax attention over these K and V up to
 * rounding.  n_tokens == 0 writes nothing.  A read-back and measurement
 * path, not tuned for speed. */
kvq_status kvq_dequantize(const kvq_layer *layer, int32_t which, float *out, void *stream);

/* Re-encode the body rows [0, n_tokens) of K and V from src's codecs to
 * dst's codecs in the same basis (VBR degrade step), out of place: dst's
 * codes/scales/mins are written, src is only read, the tails are untouched
 * (dst may share src's tail buffers).  src and dst must agree on batch,
 * n_kv_heads, capacity, tail_len, n_tokens, basis and w.  Every codec pair
 * is accepted; LOWRANK planes are not supported (KVQ_ERR_UNSUPPORTED).  A
 * ragged batch is transcoded over n_tokens rows for every sequence (rows
 * past a sequence's own count are re-encoded and stay unread). */
kvq_status kvq_transcode_layer(const kvq_layer *src, const kvq_layer *dst, void *stream);

/* One decode step of a layer in one call: append one new token per
 * sequence (k_new, v_new: device binary32 [B][1][Hkv][128], at position
 * n_tokens, or seq_tokens[b]) and decode attention over the cache with it
 * (n_tokens + 1 tokens, or seq_tokens[b] + 1).  Equal to
 * kvq_quantize_append(layer, k_new, v_new, 1) followed by
 * kvq_decode_attention on the layer with its counts advanced by one (the
 * forum thread on decode bandwidth, second post: each step stores the new
 * token's K and V and attends over all of them); the caller advances
 * n_tokens (and seq_tokens) afterwards.  For plain and KVarN layers with one
 * head group per kv head (n_q_heads / n_kv_heads in {1, 2, 4, 6, 8}) the
 * append runs inside the decode launch: the one workgroup whose tiles hold
 * the new token writes its rows before it reads; otherwise it is the two
 * launches.  Workspace and errors as kvq_decode_attention;
 * KVQ_ERR_CAPACITY when n_tokens + 1 exceeds capacity. */
kvq_status kvq_append_decode(const kvq_layer *layer, const float *k_new, const float *v_new,
                             const float *q, int32_t n_q_heads, float sm_scale, float *out,
                             void *ws, size_t ws_bytes, void *stream);

/* kvq_append_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The decode workspace is a
 * fixed 16 MiB device array inside the library (one per GPU, held until the
 * process ends); the call allocates and frees nothing.  The first call on a
 * GPU also enqueues a small kernel that clears the array's completion
 * counters; every completed call leaves them clear.  All calls on one GPU
 * share the array: calls that overlap in time on one GPU (on any streams)
 * race and must not be issued.  KVQ_ERR_WORKSPACE (nothing enqueued) when
 * the layer's step needs more than 16 MiB of workspace (the workspace
 * kvq_decode_workspace_bytes reports for the plan chosen; grows with
 * batch x query heads); other arguments and errors as kvq_append_decode. */
kvq_status kvq_append_decode_noalloc(const kvq_layer *layer, const float *k_new, const float *v_new,
                                     const float *q, int32_t n_q_heads, float sm_scale, float *out,
                                     void *stream);

/* Workspace needed by kvq_decode_attention for this layer's shapes and
 * capacity (independent of n_tokens), in bytes.  Its first 64 KiB hold
 * split-completion counters: zero-fill a workspace once before its first
 * use; every completed call leaves them zero again, and the rest of the
 * workspace needs no initialisation. */
size_t kvq_decode_workspace_bytes(const kvq_layer *layer, int32_t n_q_heads);

/* Decode attention of one query per head over the first n_tokens tokens.
 * q: device binary32 [B][n_q_heads][128]; out: device binary32
 * [B][n_q_heads][128] (raw basis).  Scores are sm_scale * <q, k>.
 * n_q_heads must be a multiple of n_kv_heads; n_tokens >= 1 and
 * batch * n_kv_heads * head groups <= 16384 (a head group is up to 8 query
 * heads of one kv head).  ws: device scratch of at least
 * kvq_decode_workspace_bytes bytes, zero-filled before its first use (see
 * there); calls sharing a workspace must not overlap in time.  One kernel
 * launch: the split that finishes its (batch, kv head, head group) last
 * merges the splits into out.  Tokens t >= n_tokens - tail_len are read
 * from the tail.  With seq_tokens, sequence b attends over its own
 * T_b = seq_tokens[b] tokens (tail: t >= T_b - tail_len); T_b == 0 gives a
 * zero output. */
kvq_status kvq_decode_attention(const kvq_layer *layer, const float *q, int32_t n_q_heads,
                                float sm_scale, float *out, void *ws, size_t ws_bytes,
                                void *stream);

/* As kvq_decode_attention with an explicit number of context splits per
 * (batch, kv head) for the quantised body (0 = the library's choice); the
 * result does not depend on it beyond floating-point rounding. */
kvq_status kvq_decode_attention_splits(const kvq_layer *layer, const float *q,
                                       int32_t n_q_heads, float sm_scale, float *out,
                                       void *ws, size_t ws_bytes, int32_t body_splits,
                                       void *stream);

/* VBR budget controller (VBR announcement thread, opening posts: the cache
 * stays at 16 bits while it fits, then layers move down a codec ladder in a
 * profiled per-layer order, never below a floor codec, within a VRAM budget;
 * any added KV can push a degrade).  Host-only policy; each step it returns
 * is carried out with kvq_transcode_layer.
 *
 * Layer l is stored in codec ladder[level[l]] (K and V alike).  Bytes of a
 * layer at n tokens: 2 * batch * n_kv_heads * n * (codes + scales + mins of
 * one 128-wide row) plus, when tail_len > 0, 2 * batch * n_kv_heads *
 * tail_len * 256 bytes of binary16 tail.  A degrade moves one layer one rung
 * down; the layer moved next is the one at the highest rung (smallest level)
 * still above `floor`, ties broken by `order` (a permutation of the layers,
 * first = degraded first).  Layers never move back up. */
typedef struct kvq_vbr_policy {
    int32_t n_layers;
    const int32_t *ladder;      /* host [ladder_len] kvq_codec, best first */
    int32_t ladder_len;
    int32_t floor;              /* lowest allowed ladder index */
    const int32_t *order;       /* host [n_layers] degrade order */
    int32_t batch, n_kv_heads, tail_len;
    long long budget_bytes;
} kvq_vbr_policy;

/* Bytes of the whole cache at `level` and n_tokens (-1 on bad arguments). */
long long kvq_vbr_bytes(const kvq_vbr_policy *pol, const int32_t *level, int32_t n_tokens);

/* Degrade steps that make n_tokens fit the budget.  level: host [n_layers],
 * in/out (updated to the plan).  steps: host [max_steps][3] receives
 * (layer, from codec, to codec) in the order to run them; *n_steps their
 * count.  KVQ_OK: fits.  KVQ_ERR_CAPACITY: does not fit even with every
 * layer at the floor (level and steps hold the floor plan).
 * KVQ_ERR_WORKSPACE: max_steps too small (the steps so far are valid).
 * KVQ_ERR_INVALID_ARG: bad policy, level or order; nothing changed. */
kvq_status kvq_vbr_plan(const kvq_vbr_policy *pol, int32_t n_tokens, int32_t *level,
                        int32_t *steps, int32_t max_steps, int32_t *n_steps);

/* KV-COBRA per-head rank and bit allocation (KV-COBRA explainer: C1 picks
 * rank and bits inside a head, C2 moves budget between heads until each
 * sits at the same marginal error; "Where the bits actually go" for the
 * accounting).  Host-only calibration step.
 *
 * spectra: host [n_heads][128] binary64 variances of each head's key
 * directions, largest first (eigenvalues of the key covariance).  A head
 * at (r, b) costs r*b bits per token and has error
 *   E = sum_{j >= r} spectra[j] + gamma / (2^b - 1)^2 * sum_{j < r} spectra[j]
 * (dropped variance plus the rounding noise of a b-bit quantiser on the
 * kept, Hadamard-flattened coordinates; gamma = 4/3 for a 4-sigma range).
 * Candidates are every (ranks[i], bits[k]); the total cost must not exceed
 * budget_bits (bits per token summed over heads, e.g. bpd * 128 * n_heads).
 * Outputs per head: out_rank, out_bits; *rounds: C2 exchange rounds after
 * the greedy fill; *total_error: the sum of E.  KVQ_ERR_CAPACITY when even
 * the cheapest candidates exceed the budget. */
kvq_status kvq_cobra_allocate(const double *spectra, int32_t n_heads, const int32_t *ranks,
                              int32_t n_ranks, const int32_t *bits, int32_t n_bits,
                              long long budget_bits, double gamma, int32_t *out_rank,
                              int32_t *out_bits, int32_t *rounds, double *total_error);

/* Measurement hook (not part of the cache format).  kvq_timing_begin
 * creates 2*capacity host-side hipEvents on the current device; each later
 * kvq_decode_attention* call records one pair on its stream, right before
 * and after its split-K attention kernel (the kernel that reads the cache),
 * until capacity pairs are used.  kvq_timing_end waits for the recorded
 * events, returns the summed elapsed milliseconds and the number of pairs,
 * destroys the events and stops recording (NULL outputs are allowed).  Not
 * thread safe: one timing session per process.  capacity must be in
 * [1, 1<<20]. */
kvq_status kvq_timing_begin(int32_t capacity);
kvq_status kvq_timing_end(double *total_ms, int32_t *count);
/* Elapsed milliseconds of each pair recorded so far in the current timing
 * session, in launch order (waits for them): ms_each[i] for i < *count,
 * *count = min(pairs recorded, capacity).  Recording continues. */
kvq_status kvq_timing_durations(float *ms_each, int32_t capacity, int32_t *count);

const char *kvq_status_string(kvq_status status);
/* Detail of the last error on the calling thread ("" if none). */
const char *kvq_last_error(void);
int32_t kvq_abi_version(void);
/* Hash of the sources the library was built from (16 hex digits, comments
 * and whitespace ignored; "unknown" when the build did not set it). */
const char *kvq_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
