// Host-side launchers shared between the translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Device view of a layout: the handle's arrays plus the internal tile scratch.
struct LayoutView {
  int32_t s, e, k, capacity;  // capacity 0 = dropless
  int32_t route_major;        // 1: slots walk every token's first route, then second, ...
  int32_t pad_multiple;       // dropless segments rounded up to this many rows (>= 1)
  int64_t rows;
  int32_t ntiles;             // ceil(items / kTileTokens); items = s, or s*k route-major
  int32_t* counts;
  int32_t* kept;
  int32_t* offsets;
  int32_t* dst;
  int32_t* src;
  int32_t* route_idx;
  uint64_t* checksum;
  int32_t* flags;
  int32_t* tile_counts;       // [e, tile_row_length(ntiles)] per-tile valid-route counts
  uint64_t* tile_checksum;    // [ntiles]
  int32_t* tile_flags;        // [ntiles]
};

// Row length of the expert-major tile table: the tile count rounded up to a multiple
// of 4, so each row can be read with 16-byte loads.
inline int tile_row_length(int ntiles) { return (ntiles + 3) / 4 * 4; }

// Smallest supported compile-time route bound >= k (k in [1, 16]).
inline int route_bound(int k) { return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16; }

hipError_t launch_gate_topk(const float* logits, int s, int e, int k, int32_t* idx, float* w,
                            hipStream_t stream);
hipError_t launch_gate_topk_backward(const int32_t* idx, const float* w, const float* gw, int s,
                                     int e, int k, float* gl, hipStream_t stream);

hipError_t launch_layout(const int32_t* idx, const LayoutView& L, hipStream_t stream);

// Row movers. row_chunks = 16-byte chunks per row. `verify_idx` may be null.
hipError_t launch_dispatch(const LayoutView& L, const int32_t* verify_idx, const void* x,
                           int64_t row_chunks, void* out, hipStream_t stream);
// w == nullptr: unweighted sum (the dispatch backward).
hipError_t launch_combine(const LayoutView& L, const void* rows_in, const float* w,
                          int64_t row_chunks, int dtype, void* y, hipStream_t stream);
hipError_t launch_combine_backward(const LayoutView& L, const void* gy, const void* E,
                                   const float* w, int64_t row_chunks, int dtype, void* gE,
                                   float* gw, hipStream_t stream);
// Weights applied at dispatch: out[dst] = w * x (and its backward: a weighted combine of
// grad_out plus grad_w = <grad_out[dst], x>).
hipError_t launch_dispatch_weighted(const LayoutView& L, const void* x, const float* w,
                                    int64_t row_chunks, int dtype, void* out, hipStream_t stream);
hipError_t launch_dispatch_weighted_backward(const LayoutView& L, const void* grad_out,
                                             const void* x, const float* w, int64_t row_chunks,
                                             int dtype, void* gx, float* gw, hipStream_t stream);
// Weights renormalised over each token's kept routes, and the backward.
hipError_t launch_renormalize_kept(const LayoutView& L, const float* w, float* w_out,
                                   hipStream_t stream);
hipError_t launch_renormalize_kept_backward(const LayoutView& L, const float* w,
                                            const float* grad_out, float* grad_w,
                                            hipStream_t stream);

// Zero the rows of a [rows, rc chunks] buffer that no placed route fills.
hipError_t launch_zero_unfilled_rows(const LayoutView& L, void* out, int64_t row_chunks,
                                     hipStream_t stream);
// Grouped expert GEMM over the layout's segments: out[r] = A(r) @ w[x]^T for the placed
// rows r of expert x, A(r) = a[src[r]] if gather else a[r]; optional route weight per
// row (route_w may be null); unfilled rows zeroed. dtype bf16 or f16; m, n multiples of 8.
hipError_t launch_expert_gemm(const LayoutView& L, const void* a, bool gather, const void* w,
                              const float* route_w, int m, int n, int dtype, void* out,
                              hipStream_t stream);
// Weight gradient of the grouped expert GEMM: grad_w[x] = sum over expert x's placed rows
// r of outer(grad_out[r], A(r)), [e, n, m] in float32 (out_f32) or rounded once to dtype;
// zeros for experts with no rows.
hipError_t launch_expert_gemm_wgrad(const LayoutView& L, const void* a, bool gather,
                                    const void* grad_out, int m, int n, int dtype, bool out_f32,
                                    void* grad_w, hipStream_t stream);
// The grouped expert GEMM with weights stored [K][N] per expert (each K row contiguous
// along N), on placed rows a[r] (no gather, no route weight): out[r] = a[r] @ w[x], [rows,
// N] of dtype; unfilled rows zeroed. dtype bf16 or f16; K, N multiples of 8.
hipError_t launch_expert_gemm_kn(const LayoutView& L, const void* a, const void* w, int K, int N,
                                 int dtype, void* out, hipStream_t stream);
int64_t expert_gemm_kn_grid(const LayoutView& L, int N);  // its workgroups (0 if none)
// Workgroups the grouped expert GEMM launches for these sizes (0 if none).
int64_t expert_gemm_grid(const LayoutView& L, int n);

}  // namespace moe
