/*
 * spffn.h -- C ABI of the neuron-sparse FFN library for AMD Instinct MI355X
 * (gfx950).
 *
 * What the library computes, per token and per FFN layer:
 *   1. a two-layer MLP predictor scores every FFN neuron and a threshold turns
 *      the scores into an active-neuron mask
 *        ("PowerInfer_x64: Neuron-Level Sparse Inference Makes Large Models
 *          Fly on Consumer GPUs", list item 2 "Prediction and Caching";
 *         "PowerInfer Guide: Exploiting Activation Sparsity for LLM AI",
 *          section 3 "Adaptive Online Neuron Predictors", predictor equation);
 *   2. the mask is compacted into an ascending list of active neuron indices
 *        (Guide, Step 3 "Fused PowerInfer Sparse FFN Module", and section 4
 *         "Neuron-Aware Sparse GPU Operators": the bitmask is decoded and only
 *         active indices are computed);
 *   3. only the active rows of W_up (and W_gate) are read, activated with
 *      ReLU (or ReLU(gate) * up), and only the matching columns of W_down are
 *      accumulated into the output
 *        (Guide, "The Hidden Inefficiency": FFN(x) = W_down (sigma(W_gate x)
 *         (*) (W_up x)); Step 3 for the non-gated ReLU form).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked [host].  Every call only
 *     enqueues work on `stream` (a hipStream_t passed as void*, NULL = the
 *     null stream) and returns; no call synchronises the host, and no call
 *     allocates or frees device memory.  Outputs and workspaces belong to the
 *     caller.  Weight pointers in a layer description are BORROWED: the caller
 *     keeps them alive and unchanged while any handle that refers to them is
 *     used.
 *   - Activations (x, y, h, logits) are fp32.  Masks are uint8 0/1 (the byte
 *     layout of a torch.bool tensor); any nonzero byte counts as set on input.
 *     Neuron indices are int32 and refer to STORED rows (after any load-time
 *     permutation).
 *   - Matrices are row-major.  W_down is stored TRANSPOSED as W_down_t
 *     [d_ffn, d], so neuron i's output column is one contiguous row.
 *   - Errors: argument, shape, dtype and workspace checks return a negative
 *     spffn_status before anything is enqueued; a failed kernel launch returns
 *     SPFFN_E_HIP.  spffn_last_error() gives the text of the calling thread's
 *     last failure.  Faults inside kernels surface at the caller's next
 *     synchronisation.  No C++ exception crosses this interface.
 *   - Calls that share a workspace must not overlap (use one stream per
 *     workspace).
 */
#ifndef SPFFN_H
#define SPFFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPFFN_OK = 0,
    SPFFN_E_ARG = -1,       /* null / misaligned pointer, bad enum, bad flag     */
    SPFFN_E_SHAPE = -2,     /* a size out of range or not a multiple it must be  */
    SPFFN_E_DTYPE = -3,     /* a storage type the call does not accept           */
    SPFFN_E_WORKSPACE = -4, /* workspace missing or smaller than required        */
    SPFFN_E_HIP = -5        /* a HIP runtime call or kernel launch failed        */
} spffn_status;

typedef enum {
    SPFFN_F32 = 0,  /* IEEE binary32                                           */
    SPFFN_F16 = 1,  /* IEEE binary16                                           */
    SPFFN_Q4_0 = 2, /* 4-bit blocks of 32 codes with an fp16 scale; on the GPU
                       in the split layout written by spffn_q4_0_repack       */
    SPFFN_FP8_E4M3 = 3 /* predictor weights only: OCP 8-bit floating point E4M3
                       (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
                       no infinities) codes with one fp32 scale per row:
                       weight[i][k] = e4m3(code[i][k]) * scale[i].  A matrix
                       [rows, cols] is one buffer: the codes, row-major, one
                       byte each, then the rows' fp32 scales.  The NaN codes
                       0x7F and 0xFF must not occur.                           */
} spffn_dtype;

typedef enum {
    SPFFN_RELU = 0,   /* non-gated: a_i = max(W_up[i] . x + b_i, 0)               */
    SPFFN_REGLU = 1,  /* gated:     a_i = max(W_gate[i] . x + b_i, 0) * (W_up[i] . x) */
    SPFFN_SWIGLU = 2  /* gated:     a_i = silu(W_gate[i] . x + b_i) * (W_up[i] . x),
                         silu(z) = z / (1 + e^-z).  SiLU is never exactly 0, so the
                         neurons left out are near zero rather than zero: the
                         sparse FFN approximates the dense one, by at most the
                         skipped |a_i| times their W_down column norms (Guide,
                         "The Hidden Inefficiency": SwiGLU activations have
                         near-zero magnitudes, not exact zeros).  "Active" for
                         profiling is a positive gate pre-activation.          */
} spffn_kind;

/* Maximum number of tokens per call (batch B). */
#define SPFFN_MAX_BATCH 16

/* [host] Description of one FFN layer and its predictor.
 *   w_gate    [d_ffn, d]  ReGLU only (NULL for ReLU)
 *   w_up      [d_ffn, d]
 *   w_down_t  [d_ffn, d]  W_down transposed
 *   b_act     fp32 [d_ffn] bias of the activated projection (gate for ReGLU,
 *             up for ReLU), or NULL for none
 *   p_w1 [r, d], p_b1 fp32 [r], p_w2 [d_ffn, r], p_b2 fp32 [d_ffn]
 *   tau       probability threshold in (0, 1): neuron i is predicted active
 *             when sigmoid(logit_i) > tau, evaluated as logit_i > t with
 *             t = ln(tau / (1 - tau)) computed once in binary64 and rounded to
 *             binary32 (sigmoid is increasing)
 *   dense_prefix  k in [0, d_ffn]: the first k stored neurons are always
 *             active, for every token, and the predictor does not score them
 *             (their p_w2 / p_b2 rows are never read; logits reported for
 *             them are +inf).  After the hot-first order these are the
 *             neurons that fire on every profiling token, so the hot set runs
 *             as a plain dense GEMV with no predictor bytes (Guide section 2,
 *             hot neurons placed where they are always at hand; section 4,
 *             neurons pre-grouped into blocks: the always-hot block).  0 is
 *             the plain predictor.
 * FFN weights are w_dtype (F32, F16 or Q4_0 split layout); predictor weights
 * are p_dtype (F32, F16 or FP8_E4M3: the x64 page's list item 2 and the
 * Guide's section 3 describe a small, low-rank predictor; 8-bit weights halve
 * its bytes, which are a third to four fifths of a decode step's).  Shapes:
 * F32 needs d % 4 == 0, F16 d % 8 == 0, Q4_0 d % 32 == 0; the predictor needs
 * d and r multiples of 4 (F32), 8 (F16) or 16 (FP8_E4M3).  Every weight
 * pointer must be 16-byte aligned. */
typedef struct {
    int32_t d, d_ffn, r;
    int32_t kind;     /* spffn_kind  */
    int32_t w_dtype;  /* spffn_dtype */
    int32_t p_dtype;  /* spffn_dtype */
    float tau;
    int32_t dense_prefix; /* always-active leading neurons, 0 for none */
    const void *w_gate;
    const void *w_up;
    const void *w_down_t;
    const float *b_act;
    const void *p_w1;
    const float *p_b1;
    const void *p_w2;
    const float *p_b2;
} spffn_layer_desc;

typedef struct spffn_layer spffn_layer; /* [host] opaque, immutable after create */
typedef struct spffn_model spffn_model; /* [host] opaque: an ordered layer stack  */

/* [host] Optional per-layer record of a decode step, for tests and timing.
 * Any member may be NULL.  h_in [L, B, d]: the residual stream entering each
 * layer; union_mask [sum_l d_ffn_l]: each layer's union mask, layers
 * concatenated; logits [sum_l B * d_ffn_l]: each layer's predictor logits
 * [B, d_ffn_l]; events [2 L]: hipEvent_t handles (owned by the caller)
 * that time each layer's largest kernel: on the single-token path the kernel
 * that streams predictor layer 2, gathers the gate/up rows and runs the down
 * projection, whose dispatch is timestamped into events 2l (start) and 2l+1
 * (end); on other paths the events are recorded on the stream around the FFN
 * kernels. */
typedef struct {
    float *h_in;
    uint8_t *union_mask;
    float *logits;
    void **events;
} spffn_trace;

/* ---- handles --------------------------------------------------------- */

/* Validate `desc` and build a layer handle (a small host struct; the weights
 * stay borrowed).  *out is set only on SPFFN_OK. */
spffn_status spffn_layer_create(const spffn_layer_desc *desc, spffn_layer **out);
void spffn_layer_destroy(spffn_layer *layer);

/* [host] The binary32 logit threshold t the layer compares against (NaN for
 * a NULL layer). */
float spffn_layer_threshold(const spffn_layer *layer);

/* An ordered stack of layers sharing one model width d.  `layers` is a host
 * array of L handles, which stay owned by the caller and must outlive the
 * model.  rms_eps is the epsilon of the gainless RMS normalisation applied to
 * the residual stream before every layer. */
spffn_status spffn_model_create(const spffn_layer *const *layers, int32_t n_layers,
                                float rms_eps, spffn_model **out);
void spffn_model_destroy(spffn_model *model);

/* Bytes of device workspace that spffn_predict / spffn_forward (layer) and
 * spffn_decode_step (model) need for a batch of B tokens; 0 on bad input.
 * The workspace must be 256-byte aligned.  Its first 256 bytes are a status
 * block (see spffn_workspace_status). */
size_t spffn_layer_workspace_bytes(const spffn_layer *layer, int32_t B);
size_t spffn_model_workspace_bytes(const spffn_model *model, int32_t B);

/* Workspace status.  The first int32 of every workspace counts the
 * down-projection workgroups of the single-token decode step whose bounded
 * in-launch wait ran out (see spffn_set_wait_limit): each such workgroup wrote
 * NaN partial sums and listed no rows, so a step with a nonzero count has a
 * NaN output and under-reports its layer counts.  The count accumulates over
 * every call that uses the workspace until it is cleared; a newly allocated
 * workspace holds no meaningful count until spffn_workspace_clear_status.
 * clear: zeroes the status block (ws_bytes >= 256), enqueued on `stream`
 * (a fill kernel, so it may be captured into a graph).
 * status: copies the count into *giveups (a device int32) on `stream`.
 * SPFFN_E_ARG for NULL or misaligned pointers, SPFFN_E_WORKSPACE for a
 * workspace smaller than its status block. */
spffn_status spffn_workspace_clear_status(void *ws, size_t ws_bytes, void *stream);
spffn_status spffn_workspace_status(const void *ws, size_t ws_bytes, int32_t *giveups,
                                    void *stream);

/* ---- the hot path ----------------------------------------------------- */

/* Threshold given logits: mask[i] = logits[i] > t for i < n (strict; NaN is
 * inactive).  Guide section 3 threshold; sigmoid replaced by its logit, as in
 * spffn_layer_desc. */
spffn_status spffn_threshold(const float *logits, int64_t n, float t, uint8_t *mask,
                             void *stream);

/* Compaction: idx[0 .. count) = the i < n with mask[i] != 0, ascending;
 * *count (device int32) = their number.  idx must hold n entries; entries at
 * and after count are left unspecified.  1 <= n < 2^31; mask 16-byte aligned
 * is fastest but not required.  Guide Step 3 (the active positions of the
 * mask) and section 4 (the activation bitmask decoded into indices). */
spffn_status spffn_compact(const uint8_t *mask, int32_t n, int32_t *idx, int32_t *count,
                           void *stream);

/* Predictor for B tokens x [B, d]:
 *   hid = ReLU(W1 x + b1), logits = W2 hid + b2, mask = logits > t
 * logits [B, d_ffn] (may be NULL), mask [B, d_ffn] (may be NULL) and
 * union_mask [d_ffn] = OR over the batch (may be NULL).  x64 page list item 2
 * (a 2-layer MLP predictor); Guide section 3. */
spffn_status spffn_predict(const spffn_layer *layer, const float *x, int32_t B, float *logits,
                           uint8_t *mask, uint8_t *union_mask, void *ws, size_t ws_bytes,
                           void *stream);

/* Neuron-sparse FFN of B tokens x [B, d] over one neuron set shared by the
 * batch, written to y [B, d]:
 *   y_b = sum over active i, ascending, of a_i(x_b) * W_down_t[i]
 * The set is, in order of precedence:
 *   mask != NULL            the set entries of mask [d_ffn] (compacted here);
 *   idx, count != NULL      idx[0 .. *count), ascending, each in [0, d_ffn),
 *                           count a device int32 <= d_ffn;
 *   all NULL                every neuron (the dense FFN, same kernels).
 * Guide "The Hidden Inefficiency" (FFN equation) and Step 3 (gather active
 * rows of W_up, activate, gather the matching columns of W_down, sum).  The
 * result does not depend on the run: no atomics carry data, and partial sums
 * are reduced in a fixed order. */
spffn_status spffn_forward(const spffn_layer *layer, const float *x, int32_t B,
                           const uint8_t *mask, const int32_t *idx, const int32_t *count,
                           float *y, void *ws, size_t ws_bytes, void *stream);

#define SPFFN_DECODE_DENSE 1 /* skip predictor and compaction; every neuron */

/* One decode step through the whole stack for B tokens, all on `stream`
 * with no host synchronisation.  For each layer l:
 *   n_b = h_b / sqrt(mean(h_b^2) + rms_eps)            (gainless RMS norm)
 *   M   = OR over b of the predicted mask of n_b        (union over the batch)
 *   h_b = h_b + FFN_l over M of n_b
 * x [B, d] is the input residual stream, h [B, d] receives the output (x == h
 * updates in place).  layer_counts [L] (device int32, may be NULL) receives
 * |M| per layer; trace may be NULL.  flags: 0 or SPFFN_DECODE_DENSE (every
 * neuron, no predictor: the dense baseline on the same kernels).  The
 * per-layer pipeline follows the Guide's section 3 latency-hiding pipeline
 * (predictor, then the fused neuron-sparse GEMV); the residual/normalisation
 * glue between layers is this library's reading, as the pages show one layer. */
spffn_status spffn_decode_step(const spffn_model *model, const float *x, float *h, int32_t B,
                               int32_t flags, int32_t *layer_counts, const spffn_trace *trace,
                               void *ws, size_t ws_bytes, void *stream);

/* [host] The logit threshold of a probability threshold tau in (0, 1):
 * ln(tau / (1 - tau)) evaluated in binary64 and rounded once to binary32 (the
 * same value a layer created with that tau compares against); NaN outside
 * (0, 1).  Guide section 3: a neuron is predicted active when
 * sigmoid(logit) > tau. */
float spffn_tau_threshold(float tau);

/* The decode step with a threshold per token and per layer instead of each
 * layer's tau: thresholds [L, B] (device fp32, row-major, binary32 LOGIT
 * thresholds, e.g. spffn_tau_threshold of a per-token tau) -- token b is
 * predicted active on neuron i of layer l when its logit > thresholds[l*B + b]
 * (strict; NaN logits are inactive), and each layer computes every token on
 * the union of the batch's per-token sets, as spffn_decode_step does.  The
 * mechanism of the Guide's "Production Engineering" section 2 (tuning
 * predictor thresholds: adaptive dynamic thresholding, which lowers tau for
 * sensitive tokens); the policy that picks the values is the caller's.
 * Other arguments and errors as spffn_decode_step (flags 0); SPFFN_E_ARG for
 * NULL or misaligned thresholds.  The array is read on the device while the
 * step runs, so the caller keeps it unchanged until the step completes. */
spffn_status spffn_decode_step_adaptive(const spffn_model *model, const float *x, float *h,
                                        int32_t B, const float *thresholds,
                                        int32_t *layer_counts, const spffn_trace *trace,
                                        void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * decode step as spffn_decode_step (same arguments and results, no trace),
 * with the kernels' workspace taken from a static device array of the
 * library instead of a caller buffer.  The array holds
 * SPFFN_NOALLOC_SCRATCH_BYTES (64 MiB, enough for every shape here up to
 * d = 12288, d_ffn = 49152 at B = 16); each GPU the library runs on keeps its
 * own copy until the process ends.  The call allocates nothing: its first call
 * on a device looks up that device's copy (hipGetSymbolAddress) and keeps the
 * address.  Every call on a GPU shares that GPU's array, which keeps the last
 * call's contents, so calls that overlap on one GPU (two streams, or a call
 * and a replay still in flight) race.  The give-up count of the bounded waits
 * (spffn_workspace_status) is not observable here; a give-up still shows as
 * NaN in h.  SPFFN_E_WORKSPACE when the model needs more scratch than the
 * array holds at this B (spffn_model_workspace_bytes); otherwise errors as
 * spffn_decode_step. */
#define SPFFN_NOALLOC_SCRATCH_BYTES (64u << 20)
spffn_status spffn_decode_step_noalloc(const spffn_model *model, const float *x, float *h,
                                       int32_t B, int32_t flags, int32_t *layer_counts,
                                       void *stream);

typedef struct spffn_graph spffn_graph; /* [host] opaque: a captured decode step */

/* Capture one spffn_decode_step (same arguments, no trace) into a HIP graph
 * for replay: a decode loop then issues one graph launch per token instead of
 * one launch per kernel.  The capture runs on a private stream of the
 * library's own and enqueues no device work; it records the pointers it is
 * given, so every replay reads x, writes h and layer_counts and uses ws at
 * those addresses, and the caller changes the input by writing into x between
 * replays.  The buffers must stay allocated while the graph exists, and two
 * replays in flight at once (or a replay and any other call using the same
 * ws) race.  Errors as spffn_decode_step, plus SPFFN_E_HIP when the runtime
 * cannot capture or instantiate.  *out is set only on SPFFN_OK. */
spffn_status spffn_decode_graph_create(const spffn_model *model, const float *x, float *h,
                                       int32_t B, int32_t flags, int32_t *layer_counts, void *ws,
                                       size_t ws_bytes, spffn_graph **out);

/* Enqueue one replay of the captured step on `stream` (hipStream_t). */
spffn_status spffn_graph_launch(const spffn_graph *graph, void *stream);

void spffn_graph_destroy(spffn_graph *graph);

/* ---- load-time utilities ---------------------------------------------- */

/* Activation profile over N tokens x [N, d] (N >= 1): counts[i] (device
 * int32 [d_ffn]) += the number of tokens with a positive pre-activation of
 * neuron i (W_gate for ReGLU, W_up for ReLU, plus bias).  Accumulates, so the
 * caller zeroes counts first.  Guide Step 1 "Offline Activation Profiler".
 * ws (device, 256-byte aligned, caller-owned) is optional: with at least
 * spffn_profile_workspace_bytes(layer) bytes, fp16 rows with d a multiple of
 * 512 are profiled on the matrix cores (the tokens split into fp16 halves, as
 * the batched decode does); otherwise, or with ws NULL, the vector kernels run.
 * A count can then differ only for tokens whose pre-activation is within
 * rounding of zero. */
spffn_status spffn_profile(const spffn_layer *layer, const float *x, int32_t N, int32_t *counts,
                           void *ws, size_t ws_bytes, void *stream);

/* Scratch bytes that let spffn_profile use the matrix cores (0 for NULL). */
size_t spffn_profile_workspace_bytes(const spffn_layer *layer);

/* Hot-first order of n neurons from their counts: perm[k] = the neuron of
 * rank k when sorted by count descending, ties by ascending index (a stable
 * order, so the result is unique).  Guide Step 1 sorts by descending count. */
spffn_status spffn_hot_first_order(const int32_t *counts, int32_t n, int32_t *perm,
                                   void *stream);

/* dst row k = src row perm[k] for k < rows; rows of row_bytes bytes (a
 * multiple of 4).  perm must be a permutation of 0..rows-1 (an entry outside
 * that range leaves its dst row unwritten).  src and dst must not overlap.  Applied at load to W_gate,
 * W_up, W_down_t, b_act, p_w2 and p_b2 together (the Guide's section 2
 * placement by neuron temperature, kept here as a storage order). */
spffn_status spffn_permute_rows(const void *src, void *dst, const int32_t *perm, int32_t rows,
                                int64_t row_bytes, void *stream);

/* 4-bit block split.  aos [rows, cols/32] blocks of 18 bytes: an fp16 scale
 * (2 bytes, little-endian), then 16 bytes where byte k holds code k in its
 * low nibble and code k+16 in its high nibble; weight = (code - 8) * scale.
 * soa (same total size, rows*cols/32*18 bytes, 16-byte aligned) receives the
 * codes of every block, 16 bytes each, row-major ([rows, cols/2] bytes, same
 * nibble order), followed by the scales ([rows, cols/32] fp16).  cols % 32
 * == 0.  The split layout is what SPFFN_Q4_0 weight pointers refer to. */
spffn_status spffn_q4_0_repack(const void *aos, void *soa, int32_t rows, int32_t cols,
                               void *stream);

/* ---- measurement ------------------------------------------------------ */

/* Read-bandwidth probe: reads every byte of buf [bytes] once with 16-byte
 * non-temporal loads (the access the decode kernels use for weights) and
 * folds the data into sink [SPFFN_STREAM_SINK_WORDS] (device uint32s: the
 * XOR of all sink words is the XOR of all 32-bit words of buf), so the loads
 * cannot be dropped.  Timed over a buffer much larger than the caches it
 * gives the read ceiling that the decode step's achieved bandwidth is
 * compared with.  bytes a positive multiple of 16; buf 16-byte aligned.
 * SPFFN_E_ARG / SPFFN_E_SHAPE otherwise. */
#define SPFFN_STREAM_SINK_WORDS 4096
spffn_status spffn_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/* [host] Test hook.  Inside the single-token decode step, the workgroups that
 * run a chunk's down projection wait (in the same launch) until the row groups
 * of that chunk have published their lists; the wait always ends, because
 * those row groups were dispatched before them and never wait, and it is also
 * bounded: after `polls` polls (default 2^18, far beyond any layer's run time)
 * the workgroup gives up and writes NaN partial sums, so the step yields NaN
 * instead of hanging, and it counts itself in the workspace status word
 * (spffn_workspace_status).  polls in [0, 2^24]; 0 makes every such workgroup give
 * up at once (for testing the give-up path).  Process-wide; applies to
 * launches enqueued after the call (a captured graph keeps the value it was
 * captured with).  SPFFN_E_ARG outside the range. */
spffn_status spffn_set_wait_limit(int32_t polls);

/* [host] Text of the calling thread's last non-OK status ("" if none). */
const char *spffn_last_error(void);

/* [host] Library version string. */
const char *spffn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPFFN_H */
