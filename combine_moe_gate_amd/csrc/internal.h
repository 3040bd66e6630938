// Host-side launchers shared between the translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Device view of a layout: the handle's arrays plus the internal tile scratch.
struct LayoutView {
  int32_t s, e, k, capacity;  // capacity 0 = dropless
  int64_t rows;
  int32_t ntiles;             // ceil(s / kTileTokens)
  int32_t* counts;
  int32_t* kept;
  int32_t* offsets;
  int32_t* dst;
  int32_t* src;
  int32_t* route_idx;
  uint64_t* checksum;
  int32_t* flags;
  int32_t* tile_counts;       // [ntiles, e] per-tile valid-route counts
  uint64_t* tile_checksum;    // [ntiles]
  int32_t* tile_flags;        // [ntiles]
};

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

}  // namespace moe
