/*
 * moe_gate.h -- C ABI of the MI355X (gfx950) MoE gate / dispatch / combine library.
 *
 * One data-parallel hot path of a mixture-of-experts layer on one GPU:
 *   (1) top-k gating over router logits,
 *   (2) the dispatch layout: per-expert counts, token-order slots, capacity drop,
 *   (3) the permute of activation rows into an expert-grouped buffer,
 *   (4) the weighted combine of each token's expert outputs,
 *   (5) the backward passes, and a replay of (3) from a saved layout.
 *
 * Sources, cited by page title and section:
 *   [DS-8195] DeepSpeed PR "MoE dispatch: fix silent Tutel + TP corruption, speed up
 *             native and Tutel paths": part 1 (per-route index/location/gate metadata
 *             as contiguous int32; capacity resolved once on the host), part 2 (the
 *             [e, c, m] buffer), part 3 (index dispatch/combine, fp32 accumulation in
 *             combine), the review comment on fast_cumsum_sub_one (slot = cumsum - 1).
 *   [DS-8213] DeepSpeed PR "Add an opt-in DeepEP transport for the AutoEP expert
 *             all-to-all": first commit (replicate tokens before top-k expansion, group
 *             arrivals by expert, reduce the weighted sum in combine, backward = the
 *             dual operation replayed on the forward handle), review-fix commits
 *             (weights keep their gradient; rows and weights counted from one source;
 *             the row count comes from the handle without a device-to-host read), the
 *             review threads on combine weights, on live handles after a later forward
 *             and on combine reading only the rows the handle describes.
 *   [AM-3684] NeMo Automodel PR "perf(moe): reuse the DeepEP dispatch layout on
 *             activation-checkpoint recompute": section 1 and "How" (a saved handle
 *             skips the layout on recompute; the replay must reproduce row counts;
 *             mis-routing must fail loudly, not silently).
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers unless stated otherwise. The caller owns
 *     every buffer, including the layout workspace; the library allocates nothing and
 *     keeps no device state between calls, apart from the static scratch array of
 *     moe_dispatch_layout_static_scratch (a fixed size per GPU, never allocated).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call
 *     that takes a stream only enqueues work on it and returns without waiting, except
 *     moe_layout_read, which synchronises the stream.
 *   - Host-side argument checks run before anything is enqueued. On failure nothing is
 *     enqueued, a status other than MOE_OK is returned and moe_last_error() gives a
 *     message (thread-local).
 *   - Routing problems found on the device never fault and never write out of bounds:
 *     the offending route is treated as dropped and a bit is set in the layout's flags
 *     word (MOE_FLAG_*), readable with moe_layout_read.
 *   - Activation rows of m elements must start on 16-byte boundaries and be a multiple
 *     of 16 bytes long (m * element size % 16 == 0); otherwise MOE_ERR_MISALIGNED.
 *   - Element types: MOE_F32, MOE_BF16 (bfloat16), MOE_F16 (IEEE half). Narrowing to
 *     bf16/f16 rounds to nearest even. Route weights, their gradients and logits are
 *     float32; expert projection weights are of the element type and their gradient
 *     float32 or the element type (moe_expert_gemm_wgrad).
 *   - Results are deterministic: no floating-point atomics; integer atomics only where
 *     the result does not depend on their order.
 */
#ifndef MOE_GATE_H
#define MOE_GATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 6

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,     /* null pointer, negative size, k outside [1, e], ... */
  MOE_ERR_UNSUPPORTED = 2,     /* beyond MOE_MAX_EXPERTS / MOE_MAX_TOPK / 32-bit row ids */
  MOE_ERR_WORKSPACE = 3,       /* layout workspace smaller than moe_layout_workspace_bytes */
  MOE_ERR_HANDLE_MISMATCH = 4, /* layout not built by moe_dispatch_layout, or sizes differ */
  MOE_ERR_MISALIGNED = 5,      /* row pointer or row length not 16-byte aligned */
  MOE_ERR_HIP = 6              /* the HIP runtime reported an error on enqueue */
} moe_status_t;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_F16 = 2 } moe_dtype_t;

/* Bits of the layout's device flags word. */
#define MOE_FLAG_EXPERT_OUT_OF_RANGE 1 /* a route named an expert outside [0, e) */
#define MOE_FLAG_DUPLICATE_EXPERT 2    /* a route repeated an earlier expert of its token */
#define MOE_FLAG_REPLAY_MISMATCH 4     /* a replay was handed routing that differs */

#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

/*
 * Layout handle: a plain host struct whose array members point into the caller's
 * workspace. It holds routing metadata only (never weights or activations). It is a
 * value: copy it freely; it stays valid while its workspace lives, and any number of
 * layouts may be live at once ([DS-8213] review thread on a backward that runs after
 * a later forward). Fields are filled by moe_dispatch_layout; treat them as read-only.
 *
 * Buffer layout ([DS-8195] parts 2-3, [DS-8213] first commit):
 *   capacity > 0: rows = e * capacity, the [e, capacity, m] buffer; expert x owns rows
 *                 [x*capacity, (x+1)*capacity); its first kept[x] rows hold its tokens in
 *                 token order, the rest are zero padding.
 *   capacity <= 0 (dropless): rows = s * k; expert x owns rows [offsets[x], offsets[x+1])
 *                 holding its tokens in token order; offsets[e] = number of valid routes
 *                 (= s*k unless routes were flagged invalid); rows from offsets[e] on are
 *                 zero padding. For a grouped GEMM, counts[x] = offsets[x+1]-offsets[x].
 * With a pad multiple P > 1 (dropless only), each segment [offsets[x], offsets[x+1]) is
 * counts[x] rounded up to a multiple of P rows, the rows after counts[x] being zero
 * padding, and rows = s*k + e*(P-1) (an upper bound: offsets[e] is the rows used).
 * `rows` is known on the host, so sizing the next buffer needs no device read
 * ([DS-8213] review-fix commit on the row count taken from the handle).
 */
typedef struct moe_layout {
  uint64_t magic;     /* set by moe_dispatch_layout */
  int32_t s, e, k;    /* tokens, experts, routes per token */
  int32_t capacity;   /* > 0: capacity per expert; 0: dropless */
  int32_t route_major;  /* slot order (moe_layout_options_t) */
  int32_t pad_multiple; /* dropless segment rounding (moe_layout_options_t) */
  int64_t rows;       /* buffer rows (host-known) */
  int32_t* counts;    /* [e]   valid routes per expert, before the capacity drop */
  int32_t* kept;      /* [e]   routes placed per expert: min(counts, capacity) */
  int32_t* offsets;   /* [e+1] first buffer row of each expert's segment */
  int32_t* dst;       /* [s*k] buffer row of route (t, j) at t*k+j, or -1 if not placed */
  int32_t* src;       /* [rows] token of each buffer row, or -1 for padding */
  int32_t* route_idx; /* [s*k] copy of the routing the layout was built from */
  uint64_t* checksum; /* [1]   sum over routes of (idx+1)*(t*k+j+1), modulo 2^64 */
  int32_t* flags;     /* [1]   MOE_FLAG_* bits */
  void* scratch;      /* internal */
  void* workspace;
  size_t workspace_bytes;
} moe_layout_t;

/*
 * Layout options (moe_dispatch_layout_ex). A NULL options pointer means the defaults
 * {route_major = 0, pad_multiple = 1}, which is what moe_dispatch_layout uses.
 *   route_major   0: a route's slot counts the earlier tokens that chose its expert
 *                    (token order over each token's routes).
 *                 1: slots are handed to every token's first route, then every token's
 *                    second route, ... so first choices win capacity before second ones
 *                    ([DS-8195] review comment on fast_cumsum_sub_one: per-route masks
 *                    mask1, mask2, ..., later routes offset by the earlier routes'
 *                    counts).
 *   pad_multiple  >= 1; dropless only (must be 1 with a capacity): each expert segment is
 *                 rounded up to a multiple of this many rows, for grouped GEMMs with
 *                 fixed row tiles ([AM-3684] section 1: a pad multiple fixed at
 *                 construction).
 */
typedef struct moe_layout_options {
  int32_t route_major;
  int32_t pad_multiple;
} moe_layout_options_t;

/* ABI version of the loaded library (MOE_ABI_VERSION it was built with). */
int moe_abi_version(void);

/* Message of the last failed call on this thread ("" if none). Never NULL. */
const char* moe_last_error(void);

/* Name of a status code. Never NULL. */
const char* moe_status_string(moe_status_t status);

/*
 * Bytes of device workspace a layout needs for (s, e, k, capacity); 0 if the sizes are
 * invalid or unsupported. The workspace must be 256-byte aligned. Host only.
 */
size_t moe_layout_workspace_bytes(int32_t s, int32_t e, int32_t k, int32_t capacity);

/* Workspace bytes for a layout built with options (NULL = defaults); 0 if invalid. */
size_t moe_layout_workspace_bytes_ex(int32_t s, int32_t e, int32_t k, int32_t capacity,
                                     const moe_layout_options_t* options);

/*
 * (1) Top-k gate ([DS-8195] part 1; softmax then top-k renormalised over the k).
 *   logits     [s, e] float32, row-major.
 *   topk_idx   [s, k] int32 out: the k experts with the largest logits, largest first,
 *              ties to the lower expert id (+0.0 and -0.0 are equal).
 *   topk_w     [s, k] float32 out: softmax over the k selected logits (equal to the full
 *              softmax renormalised over the selection), formed in float64 and rounded
 *              once to float32.
 *   Requires 1 <= k <= e, e <= MOE_MAX_EXPERTS, k <= MOE_MAX_TOPK, s >= 0.
 *   NaN logits give unspecified (but in-range, distinct) expert ids.
 */
moe_status_t moe_gate_topk(const float* logits, int32_t s, int32_t e, int32_t k,
                           int32_t* topk_idx, float* topk_w, void* stream);

/*
 * (5) Gate backward ([DS-8213] review-fix commit: the weights' gradient must reach the
 * router). grad_logits [s, e] float32 out:
 *   for selected expert idx[t,j]: w[t,j] * (grad_w[t,j] - sum_q w[t,q] * grad_w[t,q]),
 *   formed in float64 and rounded once; every other entry is 0. Entries of topk_idx
 *   outside [0, e) are skipped.
 */
moe_status_t moe_gate_topk_backward(const int32_t* topk_idx, const float* topk_w,
                                    const float* grad_w, int32_t s, int32_t e, int32_t k,
                                    float* grad_logits, void* stream);

/*
 * (2) Dispatch layout ([DS-8195] review comment on fast_cumsum_sub_one, parts 2-3;
 * [DS-8213] review thread on the per-expert prefix sum).
 *   topk_idx   [s, k] int32: expert of route (t, j).
 *   capacity   > 0: routes whose token-order slot in their expert is >= capacity are
 *              dropped; <= 0: dropless.
 *   workspace  device buffer of at least moe_layout_workspace_bytes(s, e, k, capacity)
 *              bytes, 256-byte aligned; it backs every array of *layout.
 *   layout     host out: filled on success (also before the device work completes).
 * The slot of route (t, j) is the number of tokens t' < t whose routes name the same
 * expert (column cumsum of the token x expert mask, minus one). Routes naming an expert
 * outside [0, e), or an expert an earlier route of the same token named, are invalid:
 * not counted, not placed, and flagged. Two kernels (one when the routes fit a single
 * 256-item tile), no host synchronisation.
 */
moe_status_t moe_dispatch_layout(const int32_t* topk_idx, int32_t s, int32_t e, int32_t k,
                                 int32_t capacity, void* workspace, size_t workspace_bytes,
                                 moe_layout_t* layout, void* stream);

/*
 * (2) Dispatch layout with options (host-side `options`, NULL = defaults): the same
 * contract as moe_dispatch_layout, with the slot order and segment padding above.
 * MOE_ERR_INVALID_ARG if pad_multiple < 1, or > 1 together with a capacity.
 */
moe_status_t moe_dispatch_layout_ex(const int32_t* topk_idx, int32_t s, int32_t e, int32_t k,
                                    int32_t capacity, const moe_layout_options_t* options,
                                    void* workspace, size_t workspace_bytes,
                                    moe_layout_t* layout, void* stream);

/*
 * Dispatch layout that allocates nothing and needs no scratch from the caller: for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). The same contract and results as
 * moe_dispatch_layout_ex, bit for bit, except where the tile tables live that only the
 * layout build itself uses (per-tile expert counts, checksums and flags): in a static
 * device array of the library, MOE_STATIC_SCRATCH_BYTES per GPU, held by each GPU the
 * library runs on until the process ends.
 *   workspace  as for moe_dispatch_layout_ex, but only the handle's arrays live in it:
 *              at least MOE_LAYOUT_HANDLE_BYTES(s, e, k, rows) bytes (the regions
 *              counts[e], kept[e], offsets[e+1], dst[s*k], src[rows], route copy[s*k]
 *              int32, checksum u64 and flags i32, each starting on a 256-byte
 *              boundary; rows = e*capacity, or s*k + e*(pad_multiple-1) dropless);
 *              moe_layout_workspace_bytes_ex is always enough. The handle it fills is
 *              used by every other call exactly like one from moe_dispatch_layout_ex.
 *   MOE_ERR_UNSUPPORTED if the tile tables of (s, e, k, options) exceed the static array
 *   (about 4 bytes per expert per 256 tokens, 256 routes route-major: e = 128 covers a
 *   million tokens); MOE_ERR_WORKSPACE if the workspace is below the handle's share.
 * The first call on a device looks up its copy of the array; later calls reuse it. No
 * allocation, no memset: every table entry the build reads it wrote earlier in the same
 * call. All calls on one GPU share its array, so two of these builds enqueued on
 * different streams of one GPU that overlap in time race; builds on one stream, and
 * every other entry point, are unaffected. The array used is that of the stream's device
 * (the current device for the null stream).
 */
#define MOE_STATIC_SCRATCH_BYTES (2u << 20)
#define MOE_LAYOUT_ALIGN_UP(n) ((((size_t)(n)) + 255u) / 256u * 256u)
#define MOE_LAYOUT_HANDLE_BYTES(s, e, k, rows)                                               \
  (2 * MOE_LAYOUT_ALIGN_UP(4 * (size_t)(e)) + MOE_LAYOUT_ALIGN_UP(4 * ((size_t)(e) + 1)) +   \
   2 * MOE_LAYOUT_ALIGN_UP(4 * (size_t)(s) * (size_t)(k)) + MOE_LAYOUT_ALIGN_UP(4 * (size_t)(rows)) + \
   MOE_LAYOUT_ALIGN_UP(8) + MOE_LAYOUT_ALIGN_UP(4))
moe_status_t moe_dispatch_layout_static_scratch(const int32_t* topk_idx, int32_t s, int32_t e,
                                                int32_t k, int32_t capacity,
                                                const moe_layout_options_t* options,
                                                void* workspace, size_t workspace_bytes,
                                                moe_layout_t* layout, void* stream);

/*
 * (3) Dispatch ([DS-8195] part 3; [DS-8213] first commit): out[dst[t,j]] = x[t] for every
 * placed route, a bit copy; padding rows are written as zero. Each token row is read
 * once and written to its k destinations.
 *   x    [s, m] of dtype;  out  [layout->rows, m] of dtype.
 */
moe_status_t moe_dispatch(const moe_layout_t* layout, const void* x, int32_t m,
                          moe_dtype_t dtype, void* out, void* stream);

/*
 * (5) Dispatch replayed from a saved layout ([AM-3684] section 1, "How"): the same
 * buffer as moe_dispatch, without rebuilding the layout. If topk_idx is not NULL it is
 * compared route by route with the routing the layout was built from, and any
 * difference sets MOE_FLAG_REPLAY_MISMATCH in the layout's flags (the copy is still
 * made from the saved layout). The bit is never cleared by a later replay: it stays set
 * until the layout is built again in that workspace.
 */
moe_status_t moe_dispatch_replay(const moe_layout_t* layout, const int32_t* topk_idx,
                                 const void* x, int32_t m, moe_dtype_t dtype, void* out,
                                 void* stream);

/*
 * (3') Dispatch with the weights applied before the experts ([DS-8213] review thread on
 * combine weights and the commit that applies them before or after the expert MLP,
 * score_apply): out[dst[t,j]] = topk_w[t,j] * x[t], a float32 product rounded to dtype;
 * padding rows are zero. The combine that follows is then unweighted (moe_combine with
 * topk_w = NULL).
 */
moe_status_t moe_dispatch_weighted(const moe_layout_t* layout, const void* x,
                                   const float* topk_w, int32_t m, moe_dtype_t dtype, void* out,
                                   void* stream);

/*
 * (5') Backward of moe_dispatch_weighted: grad_x[t] = sum over placed routes j, in order,
 * of topk_w[t,j] * grad_out[dst[t,j]] (float32, separate multiply and add, rounded once to
 * dtype); grad_w[t,j] = <grad_out[dst[t,j]], x[t]> accumulated in float64 and rounded once
 * (0 for a dropped route).
 */
moe_status_t moe_dispatch_weighted_backward(const moe_layout_t* layout, const void* grad_out,
                                            const void* x, const float* topk_w, int32_t m,
                                            moe_dtype_t dtype, void* grad_x, float* grad_w,
                                            void* stream);

/*
 * Weights renormalised over each token's kept routes after the capacity drop (the other
 * reading of where the renormalisation sits): w_out[t,j] = topk_w[t,j] / S_t for routes
 * the layout placed, S_t the float64 sum of those weights in route order; 0 for dropped
 * routes, and for all of a token's routes if none was placed. Rounded once to float32.
 * topk_w and w_out are [s, k] float32 and may not overlap.
 */
moe_status_t moe_renormalize_kept(const moe_layout_t* layout, const float* topk_w, float* w_out,
                                  void* stream);

/*
 * Backward of moe_renormalize_kept, given the original weights: with u = w / S over the
 * placed routes, grad_w[t,i] = (grad_out[t,i] - sum_q u_q grad_out[t,q]) / S for placed i
 * and 0 otherwise (float64, sums in route order, rounded once).
 */
moe_status_t moe_renormalize_kept_backward(const moe_layout_t* layout, const float* topk_w,
                                           const float* grad_out, float* grad_w, void* stream);

/*
 * (4) Weighted combine ([DS-8195] part 3: fp32 accumulation; [DS-8213] first commit and
 * the review thread on combine weights: the weights are applied here):
 *   y[t] = sum over placed routes j = 0..k-1, in that order, of topk_w[t,j] * E[dst[t,j]],
 *   each product and each sum rounded to float32 (no fused multiply-add), rounded once
 *   to dtype. Dropped routes add nothing; a token with no placed route gets a zero row.
 *   Only rows the layout points at are read ([DS-8213] review on combine and rows).
 *   expert_out [layout->rows, m];  topk_w [s, k] float32, or NULL for an unweighted sum
 *   (after moe_dispatch_weighted);  y [s, m].
 */
moe_status_t moe_combine(const moe_layout_t* layout, const void* expert_out,
                         const float* topk_w, int32_t m, moe_dtype_t dtype, void* y,
                         void* stream);

/*
 * (5) Combine backward ([DS-8213] first commit: dispatch and combine are adjoint, so this is
 * a weighted dispatch; review-fix commit: the weights' gradient is returned):
 *   grad_expert_out[dst[t,j]] = topk_w[t,j] * grad_y[t] (float32 product, rounded to
 *   dtype); rows no route points at are zero.
 *   grad_w[t,j] = sum_m grad_y[t,m] * E[dst[t,j],m], accumulated in float64 and rounded
 *   once to float32; 0 for a dropped route.
 *   grad_y [s, m];  expert_out [rows, m];  grad_expert_out [rows, m];  grad_w [s, k] f32.
 */
moe_status_t moe_combine_backward(const moe_layout_t* layout, const void* grad_y,
                                  const void* expert_out, const float* topk_w, int32_t m,
                                  moe_dtype_t dtype, void* grad_expert_out, float* grad_w,
                                  void* stream);

/*
 * (5) Dispatch backward ([DS-8213] first commit: the dispatch's adjoint, an unweighted combine):
 *   grad_x[t] = sum over placed routes j, in order, of grad_out[dst[t,j]], float32
 *   accumulation, rounded once to dtype.
 *   grad_out [rows, m];  grad_x [s, m].
 */
moe_status_t moe_dispatch_backward(const moe_layout_t* layout, const void* grad_out,
                                   int32_t m, moe_dtype_t dtype, void* grad_x, void* stream);

/*
 * Grouped expert GEMM over the layout's segments, with the dispatch fused into its
 * operand loads ([DS-8213] review-fix commit: the grouped GEMM takes its row groups from
 * offsets = cumsum(counts) and ignores rows past them; first commit: arrivals are grouped
 * by expert for it). For expert x and each row r in [offsets[x], offsets[x] + kept[x]):
 *   out[r, :] = A(r) @ weights[x]^T,  A(r) = a[src[r]] if gather (a = x [s, m]: the
 *   permuted buffer is never materialised) else a[r] (a = a dispatched buffer [rows, m]).
 * Products of dtype operands are accumulated in float32 on the matrix cores (summation
 * order unspecified), optionally multiplied by the route's weight topk_w[t,j] for the
 * route placed at r (a float32 product; weights applied after the experts), and rounded
 * once to dtype. Rows no route fills are zero. Output for gather = 1 and gather = 0 on
 * the dispatched buffer is bitwise identical.
 *   weights [e, n, m] of dtype (output x input features, row-major);  out [rows, n].
 *   dtype bf16 or f16 (MOE_ERR_UNSUPPORTED otherwise); m and n multiples of 8;
 *   a, weights and out 16-byte aligned; a and out may not overlap; topk_w [s, k] float32
 *   or NULL (no scaling).
 */
moe_status_t moe_expert_gemm(const moe_layout_t* layout, const void* a, int32_t gather,
                             const void* weights, int32_t m, int32_t n, moe_dtype_t dtype,
                             const float* topk_w, void* out, void* stream);

/*
 * Input-row gradient of moe_expert_gemm ([DS-8213] first commit: the backward replays the
 * forward's grouping on the same handle; review-fix commit: the groups are the offsets'
 * segments). For expert x and each row r in [offsets[x], offsets[x] + kept[x]):
 *   grad_a[r, :] = grad_out[r, :] @ weights[x]
 * products accumulated in float32 on the matrix cores (order unspecified), rounded once
 * to dtype; rows no route fills are zero. The gradient of the token rows x (for the
 * gathered forward) is moe_dispatch_backward of grad_a.
 *   grad_out [rows, n];  weights [e, n, m];  grad_a [rows, m];  all of dtype (bf16 or f16,
 *   MOE_ERR_UNSUPPORTED otherwise); m and n multiples of 8; 16-byte aligned; grad_out and
 *   grad_a may not overlap.
 */
moe_status_t moe_expert_gemm_dgrad(const moe_layout_t* layout, const void* grad_out,
                                   const void* weights, int32_t m, int32_t n, moe_dtype_t dtype,
                                   void* grad_a, void* stream);

/*
 * Weight gradient of moe_expert_gemm, with the dispatch fused into its operand loads
 * ([DS-8213] review-fix commit: the groups are the offsets' segments; first commit: the
 * backward replays the forward's grouping). For every expert x:
 *   grad_w[x] = sum over the rows r in [offsets[x], offsets[x] + kept[x]) of
 *               outer(grad_out[r], A(r)),      A(r) = a[src[r]] if gather else a[r],
 * an [n, m] matrix (the layout of moe_expert_gemm's weights); experts with no placed row
 * get zeros. Products of dtype operands are accumulated in float32 on the matrix cores
 * (summation order unspecified); the float32 sums are stored as they are
 * (grad_w_dtype = MOE_F32) or rounded once to dtype (grad_w_dtype = dtype: the same sums,
 * narrowed to nearest even, for callers that keep gradients in the weights' type).
 *   a: x [s, m] (gather = 1) or a dispatched buffer [rows, m] (gather = 0), dtype;
 *   grad_out [rows, n] dtype (the gradient of moe_expert_gemm's output; rows outside the
 *   segments are not read);  grad_w [e, n, m] of grad_w_dtype, overwritten entirely.
 *   dtype bf16 or f16 (MOE_ERR_UNSUPPORTED otherwise); grad_w_dtype MOE_F32 or dtype
 *   (MOE_ERR_UNSUPPORTED otherwise); m and n multiples of 8; a, grad_out and grad_w
 *   16-byte aligned; grad_w may not overlap a or grad_out.
 */
moe_status_t moe_expert_gemm_wgrad(const moe_layout_t* layout, const void* a, int32_t gather,
                                   const void* grad_out, int32_t m, int32_t n, moe_dtype_t dtype,
                                   moe_dtype_t grad_w_dtype, void* grad_w, void* stream);

/*
 * Read the layout's flags word and routing checksum into HOST memory. Synchronises
 * `stream` (debugging and tests; not for the hot path). Either output may be NULL.
 */
moe_status_t moe_layout_read(const moe_layout_t* layout, int32_t* flags_host,
                             uint64_t* checksum_host, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GATE_H */
