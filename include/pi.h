/*
 * pi.h -- C ABI of the predictor-gated, neuron-aware sparse FFN for MI355X (gfx950).
 *
 * One FFN layer of batch-1 / small-batch LLM decode, computed the way the
 * PowerInfer article describes it:
 *   - "Adaptive Sparsity Predictors" / online engine: a small predictor marks,
 *     for every token, the FFN neurons that will fire; only those are computed.
 *   - "Neuron Placement and Management": a table maps every kept neuron back to
 *     its position in the original matrix (here: an ascending int32 list).
 *   - "Neuron-aware Operator": the operator works on individual row vectors
 *     (up / gate projection) and column vectors (down projection) of the one
 *     dense matrix, reading the selected neurons in place with no conversion to
 *     a sparse format.
 * Weight-only int4 with one scale per group of 128 along the row follows the
 * Intel Extension for Transformers LLM Runtime page ("01 LLM Runtime").
 *
 * Conventions for every call below
 *   - All array pointers are DEVICE pointers owned by the caller.  The library
 *     keeps no pointer after a call returns and never allocates device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream: there is no host synchronisation, and
 *     device-side counts never travel to the host.
 *   - Arguments are validated on the host BEFORE any HIP call.  A call that
 *     fails validation enqueues nothing and leaves every output untouched.
 *     Launch failures return PI_ERR_HIP.  Faults during execution surface at
 *     the caller's next synchronisation on that stream.
 *   - Every call returns a status code; pi_last_error() gives a readable detail
 *     for the calling thread.  No C++ exception crosses this boundary.
 *   - fp16 values are passed as uint16_t bit patterns (IEEE binary16).
 *   - Calls on different streams may run concurrently only with distinct
 *     workspaces; calls sharing a workspace must be ordered on one stream.
 */
#ifndef PI_H
#define PI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------- */
#define PI_OK              0
#define PI_ERR_NULL        1  /* a required pointer is NULL                          */
#define PI_ERR_SHAPE       2  /* a size is out of range or inconsistent              */
#define PI_ERR_ALIGN       3  /* a pointer is not 16-byte aligned                    */
#define PI_ERR_DTYPE       4  /* unknown activation / weight format / mode enum      */
#define PI_ERR_UNSUPPORTED 5  /* valid request the library does not implement        */
#define PI_ERR_WORKSPACE   6  /* workspace missing, too small or misaligned          */
#define PI_ERR_HIP         7  /* a HIP runtime call failed                           */

/* ---- enums ------------------------------------------------------------------------ */
#define PI_ACT_RELU   0   /* h = max(W_up[i] . x, 0)                                   */
#define PI_ACT_REGLU  1   /* h = max(W_gate[i] . x, 0) * (W_up[i] . x)                 */
#define PI_W_F16      0   /* fp16 weights, [F, d] neuron-major                         */
#define PI_W_I4G128   1   /* int4: u8 [F, d/2] (even column in the low nibble, value
                             (u - 8) * scale) + fp16 scales [F, d/128], neuron-major  */
#define PI_PER_TOKEN  0   /* pi_compact: one index list per token                     */
#define PI_UNION      1   /* pi_compact: one list of the OR of the B token masks      */

#define PI_MAX_BATCH  32        /* tokens of one union pass (pi_predict / pi_sparse_ffn at B > 1) */
#define PI_MAX_BATCH_RUN 64     /* tokens per step of pi_batch_run and pi_batch_plan            */
#define PI_MAX_D_F16  8192    /* largest d of the fp16 batch-1 kernels                */
#define PI_MAX_D_I4   16384   /* largest d of the int4 batch-1 kernels                */

/* ---- descriptors -------------------------------------------------------------------- */

/* Low-rank activation predictor of one layer: l = (x W_p1) W_p2 + bias, with
 * W_p1 [d, r] and W_p2 [r, F].  Both factors are passed TRANSPOSED, so that every
 * predictor output is one contiguous row: w_p1t[j, :] is column j of W_p1 and
 * w_p2t[i, :] is column i of W_p2 -- neuron i's predictor weights, neuron-major like
 * the FFN matrices.  Neuron i is predicted active iff sigmoid(l_i) > threshold,
 * evaluated as l_i > ln(threshold / (1 - threshold)) in fp32 (strict; 0 for
 * threshold 0.5).  z = x W_p1 is accumulated and kept in fp32 (never rounded to
 * fp16).                                                                       */
#define PI_P_F16     0   /* predictor factors fp16                                      */
#define PI_P_I8G128  1   /* predictor factors int8 weight-only, one fp16 scale per group of
                            128 along each row: w = q * s (q the stored signed byte), the
                            per-group weight-only scheme of the LLM Runtime page ("Model
                            Quantization") at 8 bits.  Batch-1 paths only: pi_predict with
                            B = 1 and pi_decode_run's kernel schedules; d % 128 == 0 and
                            r % 128 == 0.                                                  */
typedef struct pi_pred_desc {
    const void*     w_p1t;  /* [r, d] row-major (= W_p1 transposed): fp16, or int8 (PI_P_I8G128) */
    const void*     w_p2t;  /* [F, r] row-major (= W_p2 transposed): fp16, or int8 (PI_P_I8G128) */
    const float*    bias;   /* fp32 [F]                                   */
    int32_t d;              /* model width, d % 8 == 0                    */
    int32_t r;              /* predictor rank, r % 8 == 0                 */
    int32_t F;              /* ffn width (neurons), F % 8 == 0            */
    float   threshold;      /* probability in (0, 1); 0.5 is the default  */
    int32_t pfmt;           /* PI_P_F16 (0, a zero-filled descriptor) or PI_P_I8G128      */
    const uint16_t* s_p1t;  /* PI_P_I8G128: fp16 [r, d/128] scales of w_p1t; else NULL     */
    const uint16_t* s_p2t;  /* PI_P_I8G128: fp16 [F, r/128] scales of w_p2t; else NULL     */
} pi_pred_desc;

/* FFN weights of one layer, every matrix neuron-major [F, d]: row i of
 * w_down is neuron i's output vector, stored contiguously.              */
typedef struct pi_ffn_desc {
    const void*     w_gate; /* PI_ACT_REGLU only (NULL for ReLU)                       */
    const void*     w_up;
    const void*     w_down;
    const uint16_t* s_gate; /* int4 only: fp16 [F, d/128] scales; NULL for fp16        */
    const uint16_t* s_up;
    const uint16_t* s_down;
    int32_t d;              /* fp16: d % 8 == 0, d <= PI_MAX_D_F16; int4: d % 128 == 0 */
    int32_t F;
    int32_t act;            /* PI_ACT_*                                                */
    int32_t wfmt;           /* PI_W_*                                                  */
    int32_t nhot;           /* neurons [0, nhot) form the layer's hot block (0: none; a
                               zero-filled descriptor has none).  PowerInfer, "Neuron Placement
                               and Management" and its hot/cold split: the neurons that fire on
                               most tokens are laid out together (pi_place_neurons_hot) and, in
                               pi_decode_run's split schedule, computed densely -- their up/gate
                               rows read alongside the predictor, without waiting for it -- while
                               the cold rest is gathered from the predicted set.  Only the
                               results of predicted-active neurons reach y, so the output is
                               that of the same layer without a hot block.  Other calls ignore
                               it.  0 <= nhot <= 8 * ceil(F / 64).                          */
} pi_ffn_desc;

/* ---- status / info ------------------------------------------------------------------ */
const char* pi_status_string(int status);   /* static string, never NULL                */
const char* pi_last_error(void);            /* thread-local detail of the last failure  */
int         pi_version(void);               /* major * 10000 + minor * 100 + patch      */

/* ---- workspace -------------------------------------------------------------------------
 * Bytes of device workspace needed by pi_predict / pi_sparse_ffn / pi_ffn_down /
 * pi_ffn_dense_ref_gpu for any batch 1..B_max, and (when both descriptors are
 * given) by pi_decode_run.  Either descriptor may be NULL.
 * The workspace holds partial sums, the predictor's z, the activations h and
 * self-resetting arrival counters.  It must be 256-byte aligned and zero-filled
 * once before first use (pi_workspace_init, or any zero fill); every kernel
 * leaves its counters at zero when it completes.  Returns 0 on invalid input.  */
size_t pi_workspace_bytes(const pi_pred_desc* pred, const pi_ffn_desc* ffn, int B_max);

/* Zero-fills the workspace with a kernel on `stream` (no hipMemset). */
int pi_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* ---- pi_predict --------------------------------------------------------------------------
 * PowerInfer, "Adaptive Sparsity Predictors": evaluate the layer's predictor on
 * the B tokens x (fp16 [B, d]) and mark the neurons predicted to fire.
 *   logits : fp32 [B, F] or NULL       -- l for every neuron (diagnostics)
 *   mask   : u32 [B, ceil(F/32)]       -- bit (i % 32) of word i / 32 = neuron i active;
 *                                         bits at positions >= F are 0
 *   idx    : int32 [B, F] or NULL      -- with count: token b's active neuron ids in
 *   count  : int32 [B]   or NULL          ascending order in idx[b*F .. b*F+count[b])
 *                                         (the neuron table, "Neuron Placement and
 *                                         Management"); entries past count are not written
 * idx and count must both be given or both be NULL.  1 <= B <= PI_MAX_BATCH.
 * B > 1 takes an fp16 predictor with r * d * 2 < 2^31 bytes (PI_ERR_UNSUPPORTED
 * otherwise).                                                                       */
int pi_predict(const pi_pred_desc* pred, const uint16_t* x, int B,
               float* logits, uint32_t* mask, int32_t* idx, int32_t* count,
               void* ws, size_t ws_bytes, void* stream);

/* ---- pi_compact ----------------------------------------------------------------------------
 * PowerInfer, "Neuron Placement and Management": the engine keeps a neuron table that
 * maps every neuron it computes to its original position in the weight matrix.  Here
 * the table is the ascending list of the set bits of a predicted-active mask.
 * Turns masks (u32 [B, ceil(F/32)], as written by pi_predict) into ascending
 * neuron-id lists.  PI_PER_TOKEN: idx int32 [B, F], count int32 [B].
 * PI_UNION: the OR of the B masks -> idx int32 [F], count int32 [1] (the table of the
 * batch's union, which the B > 1 sparse FFN runs over).
 * Mask bits at positions >= F are ignored.  Needs no workspace (ws may be NULL).
 * Errors: PI_ERR_NULL (mask, idx or count NULL), PI_ERR_SHAPE (F <= 0, B outside
 * 1..PI_MAX_BATCH), PI_ERR_DTYPE (mode), PI_ERR_HIP.                                          */
int pi_compact(const uint32_t* mask, int B, int F, int mode,
               int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);

/* ---- pi_sparse_ffn ---------------------------------------------------------------------------
 * PowerInfer, "Neuron-aware Operator": y = sum over listed neurons i of
 * h_i * W_down[i, :], with h_i from the rows W_up[i] (and W_gate[i]) only.
 *   x          : fp16 [B, d]
 *   idx, count : device neuron list (ascending, ids < F) and its length (int32 [1]);
 *                the list is read on the device, never on the host
 *   token_mask : B == 1: must be NULL.  B > 1: u32 [B, ceil(F/32)] per-token masks;
 *                idx/count then hold their union (pi_compact PI_UNION) and token b
 *                only receives the neurons set in its own mask
 *   y          : fp32 [B, d], overwritten (an empty list gives exactly 0)
 * Accumulation is fp32; B > 1 runs on MFMA with h rounded to fp16 and takes fp16
 * weights only (int4 at B > 1 returns PI_ERR_UNSUPPORTED).  The B > 1 path keeps H in
 * the workspace (2 KB per 32 neurons of F) with the down product's partial sums
 * (up to 16 * 32 * d fp32); pi_workspace_bytes with B_max > 1 includes both.           */
int pi_sparse_ffn(const pi_ffn_desc* ffn, const uint16_t* x, int B,
                  const int32_t* idx, const int32_t* count, const uint32_t* token_mask,
                  float* y, void* ws, size_t ws_bytes, void* stream);

/* ---- the two batch-1 operators on their own ----------------------------------------------
 * pi_sparse_ffn at B == 1 is exactly pi_ffn_up followed by pi_ffn_down; each
 * enqueues one kernel, so callers can time or schedule them separately.
 * PowerInfer, "Neuron-aware Operator": the row operator reads single row vectors
 * of the up (and gate) projection, the column operator single output vectors of
 * the down projection.
 *   pi_ffn_up   : h[k] = act(W_up[idx[k]] . x [, W_gate[idx[k]] . x]) for k < count;
 *                 h fp32 [F] (entries from count on are not written).  Needs no
 *                 workspace.
 *   pi_ffn_down : y = sum over k < count of h[k] * W_down[idx[k], :]; y fp32 [d],
 *                 overwritten.  Uses the workspace for its partial sums.
 * Ids outside [0, F) contribute nothing; count is clamped to F.                        */
int pi_ffn_up(const pi_ffn_desc* ffn, const uint16_t* x, const int32_t* idx,
              const int32_t* count, float* h, void* stream);
int pi_ffn_down(const pi_ffn_desc* ffn, const int32_t* idx, const int32_t* count,
                const float* h, float* y, void* ws, size_t ws_bytes, void* stream);

/* ---- pi_decode_run: native batch-1 decode-stream executor ------------------------------
 * Enqueues nsteps consecutive decode steps on `stream` from native code.  Step
 * i uses token x[(s0 + i) % T] (x fp16 [T, d]) and the layer of replica
 * (s0 + i) % nrep (preds[nrep], ffns[nrep]: layers of one shape, e.g. the layers
 * of a model or byte-identical copies).  A step is the computation of
 * pi_predict + pi_sparse_ffn at batch 1 (PowerInfer online engine): predictor,
 * strict threshold, the neuron table, the row operator on the predicted-active
 * up/gate rows and the column operator on their down rows.  Steps run strictly one
 * after another: a step starts only when the previous step's y is complete.
 *   mode PI_RUN_FUSED: two kernels per step (predictor stage 1; then one block per
 *        64-neuron tile: its logits, mask words, up/gate rows and down rows, whose column
 *        sums are the tile's partial row: ceil(F/64) partial rows of d per step).
 *   mode PI_RUN_SPLIT: three kernels per step (predictor stage 1; logits + mask + up/gate
 *        rows per tile; down projection from the mask over ranges of neurons: at most 32
 *        partial rows of d per step, whatever the shape).
 *   mode PI_RUN_KERNELS: PI_RUN_FUSED where ceil(F/64) * d <= 2^20, else PI_RUN_SPLIT
 *        (a layer with a hot block always runs split).
 *   mode PI_RUN_AUTO: as PI_RUN_KERNELS.
 *   (Mode 1 is not assigned.)
 * y of the kernel schedules: every block that owns a share of the step's neurons stores its
 * d column sums as one fp32 partial row in the workspace (no atomics); a later kernel sums
 * the rows into y in an order fixed by the number of rows and d alone.  So y is fp32 with
 * relative (not absolute) rounding: each partial sum and each addition of the reduction
 * rounds once in fp32, whatever the scale of x or of the weights; NaN and Inf propagate as
 * in any fp32 sum (a non-finite h or weight of a listed neuron makes the affected columns of
 * y non-finite); a run is bit-identical to itself, and a step's y does not depend on the
 * steps before it.  The fused and split schedules group the sums differently and agree to
 * fp32 rounding.
 * mask u32 [ceil(F/32)], idx int32 [F] + count int32 [1] (both NULL or both set)
 * and y fp32 [d] hold the LAST step's results.  The summation order of z differs
 * from pi_predict's, so logits agree to fp32 rounding, not bit for bit.
 * events: NULL, or 2 hipEvent_t: events[0] is recorded on the stream before the
 * first launch and events[1] after the last, so their elapsed time is the run's.
 * kernel_events: NULL, or 2*nsteps hipEvent_t: kernel 2
 * of step i (the tile kernel, the one that moves the most bytes) is launched with
 * kernel_events[2i] / [2i+1] attached to its own start / end, so their elapsed time is
 * that kernel's execution time.  Attaching them slows the run down; time a run without
 * them.                                                                               */
#define PI_RUN_AUTO        0
#define PI_RUN_KERNELS     2
#define PI_RUN_FUSED       3
#define PI_RUN_SPLIT       4
int pi_decode_run(const pi_pred_desc* preds, const pi_ffn_desc* ffns, int nrep,
                  const uint16_t* x, int T, long long s0, int nsteps, int mode,
                  uint32_t* mask, int32_t* idx, int32_t* count, float* y,
                  void* const* events, void* const* kernel_events,
                  void* ws, size_t ws_bytes, void* stream);

/* ---- pi_decode_run_noalloc ---------------------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  pi_decode_run in one of its kernel schedules
 * (PI_RUN_AUTO, PI_RUN_KERNELS, PI_RUN_FUSED, PI_RUN_SPLIT) with no workspace argument: its
 * scratch (z, h and the down projection's partial rows) lives in a static device array of
 * PI_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the process
 * ends.  The call allocates nothing (no hipMalloc, no allocating library routine); the caller
 * still owns x and the outputs.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents (nothing in it needs to start at zero): calls that overlap on one
 * GPU -- different streams or threads -- race, so the caller orders them.
 * Scratch a layer needs: 256-aligned (16384 + 4 r) + 256-aligned (4 F) + 4 d P bytes, with
 * P = ceil(F/64) for the fused schedule and the split schedule's range count (at most 32 for
 * int4 rows, 64 for fp16 rows) otherwise; a layer that needs more than PI_NOALLOC_SCRATCH_BYTES
 * is rejected with
 * PI_ERR_WORKSPACE before any HIP call.
 * Every other argument, output, check and error is that of pi_decode_run.                  */
#define PI_NOALLOC_SCRATCH_BYTES (4u << 20)
int pi_decode_run_noalloc(const pi_pred_desc* preds, const pi_ffn_desc* ffns, int nrep,
                          const uint16_t* x, int T, long long s0, int nsteps, int mode,
                          uint32_t* mask, int32_t* idx, int32_t* count, float* y,
                          void* const* events, void* const* kernel_events, void* stream);

/* ---- pi_ffn_dense_ref_gpu ------------------------------------------------------------------
 * The dense FFN that skipping has to reproduce: PowerInfer ("Neuron-aware Operator"; the
 * online engine's "skip the inactive neurons") computes only the predicted-active
 * neurons, and the result equals the layer's full FFN whenever every neuron that would
 * fire is in the predicted set.  This call computes that full FFN over all F neurons (no
 * predictor, no skipping) with the same numerics as pi_sparse_ffn: the GPU reference of
 * the "all neurons listed = dense" and "true support = dense" identities, and the
 * dense-time baseline.  x fp16 [B, d]; y fp32 [B, d], overwritten.  The workspace holds
 * its down projection's partial sums (pi_workspace_bytes with a NULL predictor).
 * Errors: those of pi_sparse_ffn's descriptor checks, PI_ERR_WORKSPACE, PI_ERR_HIP.     */
int pi_ffn_dense_ref_gpu(const pi_ffn_desc* ffn, const uint16_t* x, int B, float* y,
                         void* ws, size_t ws_bytes, void* stream);

/* ---- neuron placement ----------------------------------------------------------------------
 * PowerInfer, "Neuron Placement and Management" (with its offline profiling of how often each
 * neuron fires): neurons are laid out by activation frequency, and a neuron table maps every
 * placed neuron back to its position in the original matrices.  On one GPU the layout serves
 * the balance of the batch-1 kernels, which give each block 64 consecutive neurons: the
 * neurons, ranked by profiled activation count, are dealt over those 64-neuron tiles in
 * serpentine order (ranks 0 .. T-1 to tiles 0 .. T-1, the next T ranks to tiles T-1 .. 0,
 * and so on; the last tile holds F - 64 (T - 1)), so every tile expects about the same number
 * of active neurons.  Placement permutes rows only: predictor logits, masks, the FFN output y
 * and the active sets (mapped back through the table) are those of the original layer.
 *
 * pi_place_neurons (host only, no HIP call): counts int32 [F] on the host, >= 0 (activation
 * counts of a calibration run); perm int32 [F] on the host, written: placed position p holds
 * original neuron perm[p].  Ties rank by ascending original index.  Errors: PI_ERR_NULL,
 * PI_ERR_SHAPE (F <= 0 or a negative count); perm untouched on error.                       */
int pi_place_neurons(const int32_t* counts, int F, int32_t* perm);

/* Applies a placement to one per-neuron array on `stream`: row i of dst (row_bytes bytes) is
 * row perm[i] of src, for i < n.  src and dst are device buffers of n rows and must not
 * overlap; perm is a device int32 [n] permutation of 0 .. n-1 (a row whose entry lies
 * outside [0, n) is zero-filled).  Use it for W_up, W_gate, W_down (fp16 [F, d]; int4
 * u8 [F, d/2] and scales fp16 [F, d/128]), W2t (fp16 [F, r], the transposed W_p2) and the
 * bias (fp32 [F], row_bytes 4).  Errors: PI_ERR_NULL, PI_ERR_SHAPE (n <= 0, row_bytes == 0),
 * PI_ERR_HIP.                                                                                */
int pi_permute_rows(const void* src, void* dst, const int32_t* perm, int n, size_t row_bytes,
                    void* stream);

/* The hot/cold layout (PowerInfer: power-law activation locality; "Neuron Placement and
 * Management"): the neurons that fire on at least hot_rate of the ntok profiled tokens (counts
 * as pi_count_active accumulates them, 0 <= counts[i] <= ntok) form the hot block at placed
 * positions [0, *nhot), hottest first (ties by ascending original index), at most
 * 8 * ceil(F / 64) of them; the cold rest, by descending count, is dealt in serpentine order
 * over the tiles' remaining positions.  Set the layer's pi_ffn_desc.nhot to *nhot and apply
 * perm with pi_permute_rows; pi_map_ids names original neurons as for pi_place_neurons.
 * Host only, no HIP call.  perm int32 [F] and nhot are host pointers, written on success.
 * Errors: PI_ERR_NULL, PI_ERR_SHAPE (F or ntok <= 0, a count outside 0..ntok, hot_rate outside
 * (0, 1]).                                                                                   */
int pi_place_neurons_hot(const int32_t* counts, int F, int ntok, float hot_rate, int32_t* perm,
                         int32_t* nhot);

/* PowerInfer, offline phase ("LLM Profiler"): the profiler runs requests through the model and
 * records which neurons fire in every layer; the placement above ranks neurons by those counts.
 * Here the profiling statistic on the device: counts[i] += the number of the B masks (u32
 * [B, ceil(F/32)], as pi_predict writes them) in which neuron i is set, for i < F.  counts is
 * a device int32 [F] accumulator owned by the caller (zero it before the first batch); a
 * profiling run calls pi_predict and then this on each batch of calibration tokens, on one
 * stream.  Mask bits at positions >= F are ignored.  Needs no workspace.
 * Errors: PI_ERR_NULL, PI_ERR_SHAPE (F <= 0, B outside 1..PI_MAX_BATCH), PI_ERR_HIP.       */
int pi_count_active(const uint32_t* mask, int B, int F, int32_t* counts, void* stream);

/* The neuron table: out[b, k] = perm[idx[b, k]] for k < count[b] (rows of F entries), so the
 * active list of a placed layer names original neurons (in placed order, not ascending).
 * idx, count (int32 [B]) and out are device buffers; an id outside [0, F) maps to -1; out
 * may be idx itself.  1 <= B <= PI_MAX_BATCH.  Errors: PI_ERR_NULL, PI_ERR_SHAPE, PI_ERR_HIP. */
int pi_map_ids(const int32_t* idx, const int32_t* count, int B, int F, const int32_t* perm,
               int32_t* out, void* stream);

/* ---- batch-size dispatch ------------------------------------------------------------------
 * Efficient, VRAM-Constrained xLM Inference on Clients, "Methodology" (planning phase): a
 * roofline time estimate picks, for each number of tokens per step, one of several schedules
 * prepared in advance.  Here the two schedules of the sparse FFN of B tokens on one GPU:
 *   PI_BATCH_TOKENS  every token through the batch-1 operators with its own list
 *                    (pi_sparse_ffn at B = 1, once per token): m n d w bytes per token;
 *   PI_BATCH_UNION   one pass over the union of the B lists on MFMA (pi_compact PI_UNION,
 *                    then pi_sparse_ffn at B): m U d w bytes for the B tokens together.
 * m = 2 (ReLU) or 3 (ReGLU) matrices, w = bytes per weight.  With rate[i] the probability that
 * neuron i is predicted active for one token (activation counts of a calibration run over
 * its number of tokens) and tokens drawn independently:
 *   n = sum_i rate[i],   U = sum_i (1 - (1 - rate[i])^B).
 * Each schedule's time is a fixed cost per step or per token (its kernel launches) plus its
 * bytes over its measured fraction of hbm_gbs (figures measured on MI355X, stated with the
 * implementation).  B = 1 and int4 weights (no union path) give PI_BATCH_TOKENS.  More than
 * PI_MAX_BATCH tokens run as ceil(B / 32) union passes of near-equal size (e.g. 64 = 32 + 32,
 * 33 = 17 + 16), each priced on its own group's union; u_mean is then the mean union of a pass.
 * Host only, no HIP call.  rate: host float [F], each in [0, 1].  Errors: PI_ERR_NULL,
 * PI_ERR_SHAPE (B outside 1..PI_MAX_BATCH_RUN, a rate outside [0, 1], hbm_gbs <= 0), and the
 * descriptor checks of pi_sparse_ffn; *plan untouched on error.                             */
#define PI_BATCH_TOKENS 0
#define PI_BATCH_UNION  1
#define PI_BATCH_AUTO   2   /* pi_batch_run: the cheaper of the two, estimated as below      */
typedef struct {
    double n_mean;       /* expected active neurons per token                    */
    double u_mean;       /* expected size of the union of B tokens' lists        */
    double t_tokens_us;  /* estimated time of PI_BATCH_TOKENS for the B tokens    */
    double t_union_us;   /* estimated time of PI_BATCH_UNION (B > 1, fp16)        */
    int32_t choice;      /* PI_BATCH_TOKENS or PI_BATCH_UNION: the smaller time  */
} pi_batch_plan_t;
int pi_batch_plan(const pi_ffn_desc* ffn, int B, const float* rate, double hbm_gbs,
                  pi_batch_plan_t* plan);

/* ---- pi_batch_run: native small-batch decode executor ----------------------------------------
 * The client-inference page's planning step (a schedule per number of tokens, chosen by a roofline
 * estimate) executed inside the library, around PowerInfer's online engine.  Enqueues nsteps
 * steps on `stream`; step i decodes the B tokens x[(s0 + i) % T] (x fp16 [T, B, d]) through the
 * layer of replica (s0 + i) % nrep (as pi_decode_run), every token with its own predicted
 * neurons, in one of two schedules:
 *   PI_BATCH_TOKENS: every token through pi_decode_run's kernel schedule, one after another;
 *   PI_BATCH_UNION:  ceil(B / 32) passes of near-equal groups, each the batch predictor (per-token
 *                    masks, and their union), the union's neuron table, and the union FFN on MFMA
 *                    where each token only receives the neurons of its own mask (fp16 weights and
 *                    predictor; B = 1 runs PI_BATCH_TOKENS);
 *   PI_BATCH_AUTO:   the cheaper of the two by pi_batch_plan's estimate from rate (host float [F],
 *                    activation rates of a profile) and hbm_gbs, with the predictor's bytes
 *                    (2 d r + 2 r F) added once per token to the first and once per pass to the
 *                    second.
 * 1 <= B <= PI_MAX_BATCH_RUN.  mask u32 [B, ceil(F/32)] and y fp32 [B, d] hold the last step's
 * per-token masks and outputs.  events: NULL or 2 hipEvent_t recorded around the enqueued work;
 * kernel_events: NULL or 2 nsteps hipEvent_t recorded around each step's union FFN (the union
 * schedule in one pass only, 2 <= B <= PI_MAX_BATCH; PI_ERR_SHAPE otherwise).
 * Workspace: pi_workspace_bytes(pred, ffn, min(B, 32)) with both descriptors given (B_max > 1
 * includes the union list), zero-filled once.  Errors: PI_ERR_NULL, PI_ERR_SHAPE, PI_ERR_ALIGN,
 * PI_ERR_DTYPE (schedule), PI_ERR_UNSUPPORTED (the union schedule on int4 weights or an int8
 * predictor), PI_ERR_WORKSPACE, PI_ERR_HIP; all but the last before any HIP call.           */
int pi_batch_run(const pi_pred_desc* preds, const pi_ffn_desc* ffns, int nrep, const uint16_t* x,
                 int T, int B, long long s0, int nsteps, int schedule, const float* rate,
                 double hbm_gbs, uint32_t* mask, float* y, void* const* events,
                 void* const* kernel_events, void* ws, size_t ws_bytes, void* stream);

/* ---- the attention side: head-sparse q/k/v and output projections ------------------------
 * PowerInfer, "Adaptive Sparsity Predictors": every layer has a second predictor, for the
 * self-attention block, and only the neurons it predicts are computed; "Neuron-aware Operator":
 * their rows and columns are read in place.  The attention block's neurons are its heads (head h
 * owns d_head rows each of W_q, W_k, W_v and d_head rows of W_o^T).  The head predictor is
 * pi_predict with a pi_pred_desc of F = H (its factors W_a1 [d, r] and W_a2 [r, H] passed
 * transposed as for the MLP predictor, H % 8 == 0); its mask (one bit per head, strict
 * l > theta) drives the two calls below, and its index list is the head table.  The attention
 * core over the KV cache is not part of this library: its per-head output o is an input here.
 *
 * Weights (fp16, head-major, caller-owned device memory):
 *   w_qkv [H, 3, d_head, d]: head h's q rows, then its k rows, then its v rows, each row of d;
 *   w_o   [H, d_head, d]:    head h's rows of W_o^T (y = sum_h sum_c o[h, c] w_o[h, c, :]).
 * 8 <= d <= PI_ATTN_MAX_D with d % 8 == 0; 1 <= H <= PI_ATTN_MAX_HEADS; 1 <= d_head.        */
#define PI_ATTN_MAX_HEADS 1024
#define PI_ATTN_MAX_D 16384
typedef struct pi_attn_desc {
    const void* w_qkv;
    const void* w_o;
    int32_t d;
    int32_t H;
    int32_t dh;             /* d_head */
} pi_attn_desc;

/* Bytes of device workspace pi_attn_out needs (reusable across calls on one stream; zero-fill
 * it once with pi_workspace_init: its arrival counters start at zero and are left at zero).
 * 0 on an invalid descriptor.                                                                */
size_t pi_attn_workspace_bytes(const pi_attn_desc* a);

/* q, k and v of the predicted heads: qkv fp32 [H, 3, d_head] (device) gets, for every head h
 * whose bit is set in head_mask (u32 [ceil(H/32)], device, as pi_predict writes it),
 * qkv[h, m, c] = w_qkv[h, m, c, :] . x (fp32 accumulation), and 0 for every other head.
 * x: fp16 [d], device, 16-byte aligned.  Errors: PI_ERR_NULL, PI_ERR_SHAPE, PI_ERR_ALIGN before
 * any HIP call; PI_ERR_HIP.                                                                  */
int pi_attn_qkv(const pi_attn_desc* a, const uint16_t* x, const uint32_t* head_mask, float* qkv,
                void* stream);

/* The output projection over the predicted heads: y fp32 [d] (device) =
 * sum over the heads h of the head table, c < d_head, of o[h, c] w_o[h, c, :], summed in a
 * fixed order (bitwise reproducible).  heads int32 [*count] and count (device) are the table
 * pi_predict writes (ascending head ids; ids outside [0, H) contribute nothing, a count above
 * H is taken as H).  o: fp32 [H, d_head], device; only the listed heads' values are read.  An
 * empty table gives y = 0.  ws: pi_attn_workspace_bytes(a) bytes, 256-byte aligned.
 * Errors: PI_ERR_NULL, PI_ERR_SHAPE, PI_ERR_ALIGN, PI_ERR_WORKSPACE before any HIP call;
 * PI_ERR_HIP.                                                                                */
int pi_attn_out(const pi_attn_desc* a, const float* o, const int32_t* heads, const int32_t* count,
                float* y, void* ws, size_t ws_bytes, void* stream);

/* nsteps attention-side decode steps enqueued on `stream`: step i takes token t = (s0 + i) % T
 * (x fp16 [T, d], device) through the replica (s0 + i) % nrep: the head predictor (pi_predict
 * of preds[rep], F = H, fp16 factors) writes mask u32 [ceil(H/32)], the ascending head table idx
 * int32 [H] and count [1]; pi_attn_qkv writes qkv fp32 [H, 3, d_head]; pi_attn_out projects
 * o[t] (o fp32 [T, H, d_head], the attention core's output for token t) over those heads into
 * y fp32 [d].  The outputs hold the last step's.  events: NULL or 2 hipEvent_t recorded around
 * the enqueued work; kernel_events: NULL or 2 nsteps hipEvent_t recorded around each step's
 * q/k/v kernel.  With H <= 64 the heads' logits are computed inside the q/k/v kernel (from the
 * same z and factors; the fp32 sum runs in another order than pi_predict's, so a head within
 * rounding of the threshold can be decided the other way); the outputs are the same arrays.
 * The output projection of a step stores fp32 partial rows that the next step's first kernel
 * (after the last step, a small kernel) sums into y in a fixed order, so y is bitwise that of
 * a one-step run of the last token.  Workspace: pi_workspace_bytes(pred, NULL, 1) +
 * pi_attn_workspace_bytes(a) bytes, zero-filled once.  Errors: PI_ERR_NULL, PI_ERR_SHAPE, PI_ERR_ALIGN, PI_ERR_UNSUPPORTED (an
 * int8 head predictor), PI_ERR_WORKSPACE before any HIP call; PI_ERR_HIP.                  */
int pi_attn_run(const pi_pred_desc* preds, const pi_attn_desc* attns, int nrep, const uint16_t* x,
                const float* o, int T, long long s0, int nsteps, uint32_t* mask, int32_t* idx,
                int32_t* count, float* qkv, float* y, void* const* events,
                void* const* kernel_events, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PI_H */
