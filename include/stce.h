/*
 * stce.h -- C ABI of the sampling-transform scoring core for AMD Instinct
 * MI355X (gfx950).
 *
 * The library scores replayed rollout tokens: for every row t (one scored
 * token) it computes the log-probability of the token that was sampled,
 * target[t], under the sampling program that produced it, and the gradient
 * of that log-probability with respect to the hidden state and the LM-head
 * weight.  The method is the one of togethercomputer/xorl pull request 74,
 * "Consolidate sampling-transform scoring on one shared chunked core;
 * implement top-k/top-p/min-p replay for generic ce_modes":
 *
 *   - "What this PR does" item 2: chunked projection, then temperature, then
 *     the pinned support program, then the selected logprob; a recompute
 *     closed-form VJP that keeps only per-row scalars between forward and
 *     backward, never a [tokens, vocab] activation.
 *   - item 1: the support program.  Temperature first; keys ordered by value,
 *     lower token id first among equal values; top-k keeps the first k;
 *     top-p keeps the shortest prefix whose probability mass reaches top_p,
 *     the crossing token included; min-p keeps tokens with probability at
 *     least min_p times that of the row maximum taken before any filter;
 *     top_p == 1 is the exact identity.  The filters act jointly on the one
 *     temperature-scaled, unfiltered distribution: each is a prefix of the
 *     same order and the support is the shortest of the three.
 *   - item 4: a target outside its row's support scores -inf with an exactly
 *     zero gradient; one actionable error for an unsupported operand dtype.
 *   - self-review pass: per-row temperature applied after the projection
 *     (s = fl32(z / T), correctly rounded); logprob clamped to <= 0;
 *     over-length metadata rejected, never truncated; weight gradients
 *     written once per vocabulary slice.
 *
 * Logits are computed in fp32 from bf16 (or fp32) operands and are never
 * rounded to bf16 (align "architecture v2: proposal", section 5.4 A: an fp32
 * head needs fp32 output, not fp32 compute).  The fp8 lane (STCE_DT_FP8)
 * scores an e4m3 head: its products take e4m3 operands, scaled back to fp32
 * logits (see stce_problem.weight_scale).  The backward forms
 * dz = g * (1[j == y] - q) / T with q the softmax on the support, rounds dz
 * to the operand dtype and runs the two gradient products on it (same
 * section: bf16 dlogits are what lets the dh product run on the matrix
 * cores).
 *
 * Conventions for every entry point
 *   - All array pointers are DEVICE pointers on the current HIP device,
 *     row-major and contiguous, owned by the caller.  The library allocates
 *     no device memory and keeps none between calls; scratch space is the
 *     caller's workspace (sizes from stce_workspace_bytes).
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *     enqueued on it; no call synchronizes it, so calls can be captured in
 *     a HIP graph.
 *   - Host-detectable errors (NULL required pointers, bad shapes,
 *     misaligned pointers, a workspace that is too small, an unsupported
 *     dtype) return a non-zero stce_status BEFORE anything is enqueued and
 *     write nothing.  stce_last_error() then holds a thread-local message.
 *   - Per-row value errors (temperature not finite or <= 0, top_k < 0,
 *     top_p outside (0, 1] or NaN, min_p outside [0, 1] or NaN, target
 *     outside [0, V)) are found on the device.  Such a row gets a NaN
 *     logprob and a zero gradient, and *dev_status (if not NULL) receives
 *     the first bad row: see STCE_STATUS_NONE.
 *   - Thread-safe.  Mutable state kept between calls, all of it per thread:
 *     the error string, the attached profile (stce_profile_attach), and, per
 *     device, one side stream of default priority and four timing-free events
 *     that the chunked forward and the fused step fork to and join from.  The
 *     stream and events are created on a thread's first multi-chunk call and
 *     kept for the life of the process (they are released when the process
 *     ends).  Calls that share a workspace must be ordered by the caller.
 */
#ifndef STCE_H
#define STCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STCE_DT_BF16 = 1, /* hidden and weight are bf16 (the fast path) */
  STCE_DT_F32 = 2,  /* hidden and weight are fp32 */
  STCE_DT_FP8 = 3   /* the fp8 lane: weight of e4m3 codes [V, H] (uint8) with
                       per-row fp32 scales stce_problem.weight_scale; hidden
                       bf16 [T, H], quantized per row by the library; H a
                       multiple of 16 */
} stce_dtype;

typedef enum {
  STCE_OK = 0,
  STCE_E_ARG = 1,         /* NULL pointer, bad shape, misalignment */
  STCE_E_UNSUPPORTED = 2, /* operand dtype or shape the library does not run */
  STCE_E_WORKSPACE = 3,   /* workspace smaller than stce_workspace_bytes */
  STCE_E_HIP = 4          /* a HIP runtime call failed (kernel launch) */
} stce_status;

/* dev_status value meaning "no bad row".  Otherwise the value is
 * (row << 8) | field, field being one of STCE_FIELD_*, for the smallest bad
 * row (and the smallest field code on that row). */
#define STCE_STATUS_NONE INT64_MAX
#define STCE_FIELD_TEMPERATURE 1
#define STCE_FIELD_TOP_K 2
#define STCE_FIELD_TOP_P 3
#define STCE_FIELD_MIN_P 4
#define STCE_FIELD_TARGET 5

/* stce_problem.flags */
#define STCE_PROBLEM_IGNORE_INDEX 1 /* targets equal to ignore_index mark inactive rows */
#define STCE_PROBLEM_PRE_GEMM_TEMPERATURE 2 /* one scalar temperature applied to the hidden
                                              states before the projection: see
                                              stce_problem.pre_gemm_temperature */
#define STCE_PROBLEM_BF16_LANE 4 /* the bf16 value lane (bf16 operands only), read from
                                    the xorl pull request's deduplication and review
                                    passes, where one model family runs its value
                                    program in bf16 from end to end and its logprob
                                    dtype is part of the family's contract: the
                                    projection's fp32 result is rounded to bf16,
                                    divided by the row's temperature in fp32 and
                                    rounded to bf16 again, s = bf16(fl32(bf16(z) / T));
                                    the support and log-sum-exps are taken on these
                                    keys, and the selected logprob is rounded to bf16
                                    (still written as fp32, so every value is exact in
                                    a bf16 tensor).  Gradients treat both roundings as
                                    identity: q comes from the bf16 keys.  Without a
                                    bf16 hidden/weight: STCE_E_UNSUPPORTED. */
#define STCE_PROBLEM_RECOMPUTE_ALL 8 /* the backward recomputes the keys of every row
                                        with a gradient, as xorl pull request 74's
                                        recompute closed-form VJP ("What this PR does"
                                        item 2) does, ignoring the support lists of
                                        the state (see STCE_STATE_BYTES_PER_ROW); the
                                        gradients are the same bit for bit when every
                                        listed row has a tile list (the rows then keep
                                        their places), else equal up to fp32 summation
                                        order.  No effect on the forward. */

/* Bytes of per-row state stce_forward writes and stce_backward reads.  A
 * state of T rows holds T 32-byte records (stce_row_info, in row order), then
 * T 64-byte lists of the vocabulary tiles (256 tokens each) that can hold the
 * row's support tokens: the tiles whose largest key reaches the row's last
 * support key, at most 31 of them (a count, then the tile indices in
 * increasing order; count 0 when there are more, on unfiltered rows, and when
 * the vocabulary has more than 65,535 tiles), then T 1024-byte support lists:
 * for a filtered row whose support has at most 128 tokens, its tokens as
 * (int32 token id, fp32 key) pairs in decreasing key order, increasing id
 * among equal keys (flag bit 5 of the record then set); zeros past the
 * support and on every other row.  The backward forms a
 * listed row's dz from those keys, and recomputes the keys of a sparse row
 * with a tile list on its tiles only.  No part is of size [T, V]. */
#define STCE_STATE_BYTES_PER_ROW 1120

typedef struct stce_problem {
  int64_t T;             /* rows (scored tokens), 1 <= T <= 2^22 - 64 (the products
                            address a [vocabulary, T] dz through 32-bit buffer
                            offsets) */
  int64_t H;             /* hidden size, >= 8, multiple of 8 */
  int64_t V;             /* vocabulary size, 1 <= V < 2^31 - 256 */
  int32_t dtype;         /* stce_dtype of hidden and weight */
  int32_t flags;         /* 0 or a combination of STCE_PROBLEM_* */
  const void *hidden;    /* [T, H], dtype; 16-byte aligned */
  const void *weight;    /* [V, H] (lm_head.weight layout), dtype; 16-byte aligned */
  const int64_t *target; /* [T] sampled token ids in [0, V) */
  const float *temperature; /* [T] finite > 0, or NULL = 1.0 for every row */
  const int32_t *top_k;  /* [T] >= 0; 0 or >= V = off; or NULL = off */
  const float *top_p;    /* [T] in (0, 1]; 1 = off; or NULL = off */
  const float *min_p;    /* [T] in [0, 1]; 0 = off; or NULL = off */
  int64_t chunk_rows;    /* forward rows per chunk; 0 = library default: T when
                            T <= 4,096, else two chunks (the first one's
                            selection runs beside the second one's projection)
                            of about T / 2 rows, a multiple of 256 chosen so
                            that the two projections' last waves of tiles
                            leave the fewest compute units idle (8,448 at
                            T = 16,384, V = 151,936); more, smaller chunks when
                            two chunk buffers of fp32 keys (4 C V bytes each)
                            would exceed 12 GB.  The forward workspace holds
                            two such buffers.  The fp8 lane: 256 n rows, n in
                            12 .. 16 the number of 256-token tiles whose
                            projection best fills whole waves of the 256
                            compute units (3,840 at V = 151,936). */
  int64_t vocab_slice;   /* backward vocabulary columns per slice; 0 = default */
  int64_t ignore_index;  /* with STCE_PROBLEM_IGNORE_INDEX: a target equal to it
                            (a value outside [0, V), e.g. -100) marks an inactive
                            row (nested-learning compute_teach_signal masks such
                            rows out): logprob 0, exactly zero gradient, no
                            error; its support and side outputs are still
                            computed.  Ignored otherwise. */
  float pre_gemm_temperature; /* with STCE_PROBLEM_PRE_GEMM_TEMPERATURE: the lane's
                            one scalar temperature Ts (finite, > 0), applied
                            before the product -- the scalar convention the
                            xorl pull request's self-review pass sets beside the
                            per-row post-GEMM one.  The library forms h', the
                            correctly rounded fp32 quotient h / Ts rounded to
                            the operand dtype (nearest, ties to even), and
                            scores s = fl32(h' W^T);
                            the gradients are those of that s with respect to h
                            and W (dz = g (1[j == y] - q), dW = dz^T h',
                            dH = (dz W) / Ts).  `temperature` must then be NULL
                            (the two conventions do not combine).  A power of
                            two such as Ts = 0.5 divides exactly, so it gives
                            the bits of the per-row convention with every row
                            at Ts (barring overflow and subnormals).  Ignored
                            without the flag.  Not with STCE_DT_FP8. */
  const float *weight_scale; /* STCE_DT_FP8 only (ignored otherwise): [V] fp32 scales
                            of the weight's rows, 4-byte aligned.  xorl pull
                            request 74, "What this PR does" item 4, refuses an
                            FP8 head and gives no formula for scoring one; this
                            lane is one reading of it.  The weight is OCP e4m3
                            ("e4m3fn": bias 7, 3 mantissa bits, largest finite
                            448, no infinities; the NaN codes 0x7F / 0xFF must
                            not occur) with W_deq[j, k] = weight_scale[j] *
                            W8[j, k].  Each hidden row is quantized the same way,
                            per row: a[t] = fl32(max_k |h[t, k]| / 448) (1 for
                            an all-zero row) and h8[t, k] = e4m3(clamp(fl32(h[t,
                            k] / a[t]), -448, 448)), nearest with ties to even
                            (stce_fp8_quantize_rows).  Logits z = fl32(fl32(acc
                            * weight_scale[j]) * a[t]) with acc the fp32
                            matrix-core sum of the e4m3 products; then the
                            temperature, support and logprob of the fp32 lane.
                            Gradients pass both quantizations unchanged
                            (straight through): dH = dz . W_deq and dW = dz^T .
                            h_deq with h_deq = a h8, both products on the
                            matrix cores with bf16 operands (dz, and the
                            dequantized W_deq and h_deq, rounded to bf16);
                            grad_hidden is bf16.  Neither the bf16 value lane,
                            the pre-GEMM temperature nor the fused policy step
                            take this lane. */
} stce_problem;

/* Per-row state size in bytes for T rows (STCE_STATE_BYTES_PER_ROW * T). */
size_t stce_state_bytes(int64_t T);

/* Workspace bytes needed by stce_forward (*fwd) and stce_backward (*bwd)
 * for this problem's shapes, dtype and chunking (pointers are not read).
 * Either output pointer may be NULL. */
stce_status stce_workspace_bytes(const stce_problem *prob, size_t *fwd, size_t *bwd);

/* The chunk and slice sizes the library will use for this problem: forward
 * rows per chunk and backward vocabulary columns per slice (the problem's
 * own values when non-zero, else the defaults).  Either pointer may be NULL. */
stce_status stce_schedule(const stce_problem *prob, int64_t *chunk_rows, int64_t *vocab_slice);

/* Forward (xorl pull request 74, "What this PR does" items 1, 2 and 4 and the
 * self-review pass: temperature first, the joint top-k / top-p / min-p
 * support, the selected logprob clamped to <= 0, -inf out of support):
 * logprob[t] = min(s[t, y_t] - logsumexp_{j in S_t} s[t, j], 0) if
 * y_t is in the support S_t, else -inf, with s = fl32(h W^T) / T per row
 * (or the keys of the convention prob->flags selects: scalar pre-GEMM
 * temperature, bf16 value lane, which also rounds logprob to bf16).
 * Writes logprob [T] fp32 and state [T * STCE_STATE_BYTES_PER_ROW bytes]
 * (support boundary, filtered log-sum-exp, flags, support tiles) for
 * stce_backward.  dev_status: one int64
 * (may be NULL).  ws: at least the forward workspace size, 256-byte
 * aligned. */
stce_status stce_forward(const stce_problem *prob, float *logprob, void *state,
                         int64_t *dev_status, void *ws, size_t ws_bytes, void *stream);

/* Forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results as stce_forward, bit for bit, with its
 * workspace in a static device array of the library (stce_noalloc_scratch_bytes()
 * = 64 MiB, one copy per device, held until the process ends) instead of a
 * caller workspace.  It calls no hipMalloc, hipFree or allocating routine
 * and creates no stream or event: one chunk buffer, every chunk's selection
 * on `stream` after its projection.  The chunk is prob->chunk_rows when that
 * workspace fits the array, else the largest that fits (the chunking changes
 * no bit of the result); a problem whose forward needs more than the array
 * with one row per chunk is rejected with STCE_E_WORKSPACE (its vocabulary
 * is then beyond ~12 million tokens).  Every call on a device shares that
 * device's array, which keeps the last call's contents (the forward writes
 * every byte it reads): calls that overlap on one device, on different
 * streams or threads, race and must be ordered by the caller. */
size_t stce_noalloc_scratch_bytes(void);
stce_status stce_forward_noalloc(const stce_problem *prob, float *logprob, void *state, int64_t *dev_status,
                                 void *stream);

/* Forward with side outputs of the same sweep (align "architecture v2:
 * proposal", section 5.4 A: the entropy comes from the forward's sweep, no
 * extra product).  Each pointer of `side` is a device array [T] fp32, or
 * NULL to skip it (`side` itself may be NULL: then this is stce_forward):
 *   lse_full[t]        = logsumexp_j s[t, j] over the whole row,
 *   entropy_full[t]    = -sum_j p_j log p_j, p = softmax(s[t, :]),
 *   entropy_support[t] = -sum_{j in S_t} q_j log q_j, q the filtered
 *                        distribution (softmax of s on the support),
 * in nats, on the fp32 keys s; rows with invalid metadata get NaN.  The
 * full-row entropy comes from per-tile sums of e^(s - max) (s - max) that the
 * projection epilogue forms only when an entropy is requested (a separate
 * instance of the epilogue whose mass arithmetic is the plain forward's, so
 * logprob and state are bitwise the same with and without the request; fp32
 * sums, fp64 combination); the support entropy is summed over the sorted
 * selection window when the support starts at the top of the order, else
 * in one more pass over the row.  Same workspace as stce_forward. */
typedef struct stce_side_outputs {
  float *lse_full;
  float *entropy_full;
  float *entropy_support;
} stce_side_outputs;
stce_status stce_forward_with_side(const stce_problem *prob, float *logprob, void *state,
                                   const stce_side_outputs *side, int64_t *dev_status, void *ws,
                                   size_t ws_bytes, void *stream);

/* Backward of sum_t grad_logprob[t] * logprob[t]: the recompute closed-form
 * VJP of xorl pull request 74, "What this PR does" item 2 (nothing of size
 * [T, V] kept from the forward; exactly zero gradient for out-of-support
 * rows, item 4; weight gradients written once per vocabulary slice,
 * self-review pass).  Reads the support from `state` and forms
 * dz = g (1[j == y] - q) / T on it (zero on rows whose target is out of
 * support or whose metadata is invalid; with the scalar pre-GEMM
 * temperature dz = g (1[j == y] - q) and the hidden gradient is divided by
 * Ts).  The keys q comes from are the forward's, bit for bit: a row whose
 * support the state lists takes them from that list, a row with a tile list
 * recomputes them on those vocabulary tiles only, every other row with a
 * gradient on every vocabulary slice (all rows with
 * STCE_PROBLEM_RECOMPUTE_ALL); the recompute runs the forward's product
 * main loop (same k order) and temperature step.  A filtered row whose
 * support holds at most 128 tokens adds its dz entries to dH and dW as
 * ordered sums; larger supports run the matrix-core products over their
 * vocabulary-major dz.  Writes
 *   grad_hidden [T, H] in the hidden dtype, bf16 for the fp8 lane
 *                (overwritten; NULL = skip) and
 *   grad_weight [V, H] fp32 (overwritten, or added to when
 *                accumulate_grad_weight != 0; NULL = skip).
 * `prob` must describe the same inputs as the forward that wrote `state`
 * (not checked).  ws: at least the backward workspace size. */
stce_status stce_backward(const stce_problem *prob, const float *grad_logprob, const void *state,
                          void *grad_hidden, float *grad_weight, int32_t accumulate_grad_weight,
                          int64_t *dev_status, void *ws, size_t ws_bytes, void *stream);

/* Parity entry: the fp32 keys s = fl32(h W^T) / T of rows [row0, row0 +
 * nrows) (or those of the convention prob->flags selects), written to
 * s_out [nrows, V], produced by the same projection kernel and temperature
 * step as stce_forward (same bits).  Needs the
 * forward workspace of the problem. */
stce_status stce_scaled_logits(const stce_problem *prob, int64_t row0, int64_t nrows, float *s_out,
                               void *ws, size_t ws_bytes, void *stream);

/* Parity entry: the recompute products of stce_backward, launched as
 * stce_backward launches them (same kernels, same vocabulary slices and
 * arguments), which in this call also write the fp32 keys they recompute
 * into keys_out [T, V] row-major; no gradient product runs.  The keys must
 * equal the forward's bit for bit (the recompute closed-form VJP of xorl pull
 * request 74, "What this PR does" item 2, takes its support from the state
 * and re-derives membership from these keys).  A row the backward recomputes
 * on its listed tiles only (a sparse row with a tile list, see
 * STCE_STATE_BYTES_PER_ROW) gets the keys of those tiles; its other entries
 * are not written, and neither is any key of a row whose support the state
 * lists (the backward recomputes none of them).  Every other row gets all V
 * keys.  Arguments and
 * workspace as stce_backward; keys_out is required. */
stce_status stce_recompute_keys(const stce_problem *prob, const float *grad_logprob, const void *state,
                                float *keys_out, void *ws, size_t ws_bytes, void *stream);

/* Parity entry: the support program and selected logprob applied to given
 * fp32 keys s [R, V] (row-major, 16-byte aligned, V a multiple of 4), with
 * the same selection kernel as
 * stce_forward.  Metadata pointers as in stce_problem (NULL = off), target
 * [R] required.  Writes logprob [R] (= min(s_y - lse_S, 0) or -inf) and
 * state [R * STCE_STATE_BYTES_PER_ROW bytes].  ws: at least
 * stce_support_workspace_bytes(R, V). */
stce_status stce_support_from_logits(const float *s, int64_t R, int64_t V, const int32_t *top_k,
                                     const float *top_p, const float *min_p, const int64_t *target,
                                     float *logprob, void *state, int64_t *dev_status, void *ws,
                                     size_t ws_bytes, void *stream);

/* Workspace bytes for stce_support_from_logits. */
size_t stce_support_workspace_bytes(int64_t R, int64_t V);

/* Decoding of the 32-byte per-row records of a state (for tests and
 * diagnostics).  A record holds: the boundary key (order-preserving uint32 image of
 * the last support token's fp32 key), the boundary token id, the support
 * size n (V for an unfiltered row, whose boundary is then 0 / V - 1), the
 * filtered and full log-sum-exp, the row maximum, the target's key (0 on
 * inactive ignore_index rows) and flags.  Reads the first `nrows` records of
 * a HOST copy of a state (its first nrows * 32 bytes). */
typedef struct stce_row_info {
  uint32_t key_thr;
  int32_t id_thr;
  int32_t n;
  uint32_t flags; /* bit 0 valid metadata, bit 1 filtered row, bit 2 target in support,
                     bit 3 inactive (ignore_index) row, bit 5 support listed in the state */
  float lse_support;
  float lse_full;
  float row_max;
  float target_key;
} stce_row_info;
stce_status stce_decode_state(const void *host_state, int64_t nrows, stce_row_info *out);

/* Diagnostics: per-launch HIP event timing.  While a profile is attached to
 * the calling thread, each kernel launch the library makes from that thread
 * records start[i] before and stop[i] after the launch on the call's stream
 * and stores the launch's kind (STCE_KERNEL_*) in kind[i], for
 * i = count++ while count < capacity (later launches are not recorded).
 * start/stop hold hipEvent_t handles created by the caller, who also reads
 * the elapsed times.  Pass NULL to detach.  Thread-local; never fails. */
#define STCE_KERNEL_VALIDATE 1
#define STCE_KERNEL_PROJECTION 2  /* forward logits product + keys epilogue */
#define STCE_KERNEL_SELECT 3      /* support program + selected logprob */
#define STCE_KERNEL_DLOGITS 4     /* backward recompute product + dlogits epilogue */
#define STCE_KERNEL_GRAD_WEIGHT 5 /* weight-gradient product of one slice */
#define STCE_KERNEL_GRAD_HIDDEN 6 /* hidden-gradient product of one slice */
#define STCE_KERNEL_TRANSPOSE 7
#define STCE_KERNEL_PARTIALS 8
#define STCE_KERNEL_POLICY_LOSS 9  /* per-row policy-gradient loss */
#define STCE_KERNEL_DZ_KEYS 10     /* fused step: dlogits from a chunk's stored keys */
#define STCE_KERNEL_SPLIT_SUM 11   /* fused step: sum of the hidden-gradient split partials */
#define STCE_KERNEL_PRESCALE 12    /* hidden states divided by the scalar pre-GEMM temperature */
#define STCE_KERNEL_CLASSIFY 13    /* backward: row classes (dense, sparse, empty) and their order */
#define STCE_KERNEL_SPARSE_DW 14   /* backward: weight-gradient rows from the sparse rows' dz entries */
#define STCE_KERNEL_SPARSE_DH 15   /* backward: hidden-gradient rows of the sparse and empty rows */
#define STCE_KERNEL_REPROJECT 16   /* forward: projection of the rows whose candidates could not decide */
#define STCE_KERNEL_QUANTIZE 17    /* fp8 lane: per-row e4m3 quantization of hidden rows */
#define STCE_KERNEL_TILE_LISTS 18  /* backward: per-tile lists of the rows whose keys are recomputed there */
#define STCE_KERNEL_TILE_RECOMPUTE 19 /* backward: recompute of those rows' keys on their listed tiles */
#define STCE_KERNEL_LISTED_ENTRIES 20 /* backward: dz entries of the rows whose support the state lists */
typedef struct stce_profile {
  int32_t capacity;
  int32_t count;
  void **start;
  void **stop;
  int32_t *kind;
} stce_profile;
stce_status stce_profile_attach(stce_profile *prof);

/* Policy-gradient token loss on the selected logprob (align "architecture
 * v2: proposal", section 5.4 A, "Why the in-chunk form works for this
 * loss").  With the ratio r = exp(logprob - old_logprob) and the advantage
 * A of each row, the loss-sign token coefficient c of
 * d loss / d z = c (softmax - onehot) is
 *   STCE_PG_CISPO: c = A * sg(min(r, 1 + eps_high))  (stop-gradient weight,
 *                  no lower bound; CISPO);
 *   STCE_PG_CLIP:  c = A * r * 1[not clipped]          (clipped surrogate,
 *                  clip-higher PPO / DAPO, ratio bounds 1 - eps_low and
 *                  1 + eps_high);
 * and the per-token losses are -A sg(min(r, 1 + eps_high)) logprob and
 * -min(r A, clip(r, 1 - eps_low, 1 + eps_high) A).  Writes, for t < T,
 *   loss[t]         = scale * loss_t,
 *   grad_logprob[t] = scale * d loss_t / d logprob_t  (= -scale * c), the
 *                     upstream gradient to pass to stce_backward, which
 *                     then yields the gradient of sum_t loss[t],
 *   ratio[t]        = r (NULL = skip).
 * A row whose logprob is -inf (target outside its support) gets loss 0,
 * gradient 0 and ratio 0; a NaN logprob (invalid row) gets a NaN loss and a
 * zero gradient.  Arithmetic is fp32.  All arrays are device pointers,
 * 4-byte aligned; `logprob` is typically stce_forward's output.  Host
 * errors: NULL pointers, an unknown objective, eps_low outside [0, 1),
 * eps_high negative or not finite, scale not finite. */
#define STCE_PG_CISPO 1
#define STCE_PG_CLIP 2
typedef struct stce_pg_params {
  int32_t objective;        /* STCE_PG_CISPO or STCE_PG_CLIP */
  float eps_low;            /* lower ratio bound 1 - eps_low (STCE_PG_CLIP only) */
  float eps_high;           /* upper ratio bound 1 + eps_high */
  float scale;              /* multiplies losses and gradients, e.g. 1 / a constant denominator */
  const float *advantages;  /* [T] */
  const float *old_logprob; /* [T] logprob of the target under the behaviour policy */
  const void *state;        /* [T * STCE_STATE_BYTES_PER_ROW] from the forward, or NULL: rows it marks inactive
                               (ignore_index) get loss 0, gradient 0 and ratio 0 */
} stce_pg_params;
stce_status stce_policy_loss(const stce_pg_params *pg, int64_t T, const float *logprob, float *loss,
                             float *grad_logprob, float *ratio, void *stream);

/* Fused head + policy-gradient step (align "architecture v2: proposal",
 * section 5.4 A: the "Fused" row of its GEMM-count table and "Why the
 * in-chunk form works for this loss").  The token coefficient needs only the
 * new logprob, which a chunk has just computed, so dlogits can be formed
 * from keys the forward's sweep keeps instead of a recompute.  Two paths:
 *   - with row classes, when the operands are bf16 and a filter is given
 *     (top_k, top_p or min_p not NULL), or on the fp8 lane: stce_forward
 *     (side outputs as in stce_forward_with_side, `side` may be NULL), the
 *     token loss, its gradient g and the ratio as in stce_policy_loss, then
 *     stce_backward of g, in one call on `stream`.  The sweep keeps each
 *     small support with its keys in the state (see
 *     STCE_STATE_BYTES_PER_ROW), from which the backward forms those rows'
 *     dlogits with no recompute; only the other rows are recomputed.  Every
 *     output is bitwise that of the unfused sequence on the same inputs;
 *   - dense, for fp32 operands or bf16 with no filter (every row's support
 *     is the whole vocabulary, so every row's dz is dense), per chunk of
 *     rows: the projection keeps the fp32 keys of every row of the chunk;
 *     the support program and logprob as in stce_forward; the token loss;
 *     dz = g (1[j == y] - q) / T from the stored keys, with the arithmetic
 *     of stce_backward's recompute (so equal to it bit for bit); the chunk's
 *     grad_hidden rows = dz . W (split over the vocabulary, fp32 partials
 *     summed in split order); the vocab-major dz of a group of consecutive
 *     chunks is kept (as many as 8 GB hold: all of them at the sizes below),
 *     and at a group's end grad_weight (+)= dz^T . h with the group's rows as
 *     the reduction.  2 products for a frozen head (logits, dH), 3 for a
 *     trainable one (plus dW), against 3 and 4 for stce_forward +
 *     stce_policy_loss + stce_backward; logprob, state and loss are bitwise
 *     those of the unfused sequence, the gradients differ from its only by
 *     fp32 summation order.
 * Outputs: logprob, state (as stce_forward), loss and ratio (as
 * stce_policy_loss; ratio may be NULL), and the gradients of sum_t loss[t]:
 * grad_hidden [T][H] in the hidden dtype (bf16 on the fp8 lane) and
 * grad_weight [V][H] fp32 (overwritten, or added to when
 * accumulate_grad_weight is nonzero); either may be NULL, both NULL =
 * forward and loss only.  pg->state is not read (the step's own state marks
 * inactive rows).  Workspace: 256-byte aligned device memory of
 * stce_fused_workspace_bytes (which path a problem takes depends only on its
 * dtype and which filter pointers are set).  With row classes: g [T], then
 * one region holding stce_forward's workspace and afterwards stce_backward's
 * (bytes == min_bytes; 7.1 GB at T = 16384, H = 5120, V = 151936).  Dense
 * (chunk: prob->chunk_rows rounded up to a multiple of 64, default 4096):
 * the fp32 keys of two chunks (a chunk's selection runs on a side stream of
 * the library's while the next chunk is projected, joined by event waits as
 * in stce_forward), the group's vocab-major dz (with bf16 operands the only
 * copy: the hidden gradient is formed transposed and reads it as it is;
 * fp32 also keeps a chunk's token-major copy), the transposed weight (and
 * for fp32 the transposed hidden), the split partials and, with the scalar
 * pre-GEMM temperature, h / Ts (11.9 GB at those sizes, 8.2 GB at its
 * minimum); a workspace between *min_bytes (one chunk per group) and *bytes
 * keeps as many chunks per group as it holds, which changes only the order
 * of dW's fp32 sums.  Host errors as stce_forward, stce_backward and
 * stce_policy_loss, and V must be below 2^29 (the dense path reads a chunk's
 * key rows through 32-bit buffer offsets). */
stce_status stce_fused_workspace_bytes(const stce_problem *prob, size_t *bytes, size_t *min_bytes);
stce_status stce_fused_policy_step(const stce_problem *prob, const stce_pg_params *pg, float *logprob,
                                   void *state, float *loss, float *ratio, const stce_side_outputs *side,
                                   void *grad_hidden, float *grad_weight, int32_t accumulate_grad_weight,
                                   int64_t *dev_status, void *ws, size_t ws_bytes, void *stream);

/* The fp8 lane's per-row quantization (stce_problem.weight_scale) of R rows
 * of bf16 x [R, H] (H a multiple of 16, 16-byte aligned): scales[r] =
 * fl32(max_k |x[r, k]| / 448) (1 for an all-zero row) and codes[r, k] =
 * e4m3(clamp(fl32(x[r, k] / scales[r]), -448, 448)), nearest with ties to
 * even.  The forward and backward apply it to the hidden rows; a caller may
 * use it to produce a weight's codes and scales from a bf16 weight.  codes
 * [R, H] uint8 (16-byte aligned) and scales [R] fp32 are the caller's.
 * Enqueued on `stream`; host errors as stce_forward.  R = 0 does nothing. */
stce_status stce_fp8_quantize_rows(const void *x, int64_t R, int64_t H, uint8_t *codes, float *scales,
                                   void *stream);

/* Human-readable name of a status code (static string). */
const char *stce_status_string(stce_status status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char *stce_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* STCE_H */
