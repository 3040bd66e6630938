// Row movers on gfx950: dispatch (and its replay), weighted combine, and the two
// backward passes.
//
// All four are HBM-bound row gathers/scatters, not contractions, so there is no MFMA
// here. Every kernel is token-major: one wave64 per token, the token's k route rows
// named by the layout (dst) and kept in scalar registers. Each lane moves 16-byte
// chunks (global_load/store_dwordx4), chunk c of a row at lane c mod 64, so a wave
// touches 1 KiB of a row per step, fully coalesced.
//
//   dispatch          x[t] read once, written to its k rows (DeepSpeed PR "Add an
//                     opt-in DeepEP transport for the AutoEP expert all-to-all", first
//                     commit: tokens are taken before top-k expansion and replicated).
//   combine           the k rows of a token loaded together, then summed in route
//                     order in float32 with separate multiply and add, rounded once
//                     (DeepSpeed PR "MoE dispatch: fix silent Tutel + TP corruption,
//                     speed up native and Tutel paths", part 3: fp32 accumulation; PR
//                     8213's review thread on combine weights: the weights are applied).
//   dispatch backward the same kernel without weights (the gradient of a dispatch is a
//                     combine, PR 8213 first commit).
//   combine backward  grad_y[t] read once; for each route the weighted copy goes to the
//                     route's row and the dot product with the expert row accumulates
//                     in float64 (the gradient of a combine is a dispatch, plus the
//                     weights' gradient of PR 8213's review-fix commit).
//
// Rows that no route points at (capacity padding, or rows past the last valid route)
// are zero-filled by a grid-stride tail loop in the kernels that write [rows, m]
// buffers. No floating-point atomics anywhere: results are deterministic.
#include "internal.h"
#include "moe_device.h"

namespace moe {

// Grid-stride loop over the buffer rows that no placed route fills; each wave zeroes
// whole rows.
__device__ __forceinline__ void zero_unfilled_rows(chunk_t* __restrict__ out, int64_t rc,
                                                   int capacity, int e, int32_t rows,
                                                   const int32_t* __restrict__ kept,
                                                   const int32_t* __restrict__ offsets) {
  const int lane = lane_id();
  const int32_t wave = blockIdx.x * kWavesPerBlock + wave_in_block();
  const int32_t nwaves = gridDim.x * kWavesPerBlock;
  const int32_t begin = capacity > 0 ? 0 : offsets[e];
  const chunk_t z = chunk_t{0u, 0u, 0u, 0u};
  for (int32_t r = begin + wave; r < rows; r += nwaves) {
    bool pad = true;
    if (capacity > 0) {
      const int32_t x = r / capacity;
      pad = (r - x * capacity) >= kept[x];
    }
    if (pad) {
      chunk_t* o = out + static_cast<size_t>(r) * rc;
      for (int64_t c = lane; c < rc; c += kWave) o[c] = z;
    }
  }
}

template <int KMAX>
__device__ __forceinline__ void load_dst(const int32_t* __restrict__ dst, int t, int k,
                                         int (&d)[KMAX]) {
#pragma unroll
  for (int j = 0; j < KMAX; ++j) d[j] = (j < k) ? dst[static_cast<size_t>(t) * k + j] : -1;
}

// ---------------------------------------------------------------------------------
// dispatch

template <int KMAX>
__global__ __launch_bounds__(kBlock) void dispatch_kernel(
    const chunk_t* __restrict__ x, const int32_t* __restrict__ dst,
    const int32_t* __restrict__ verify_idx, const int32_t* __restrict__ route_idx,
    int32_t* __restrict__ flags, int s, int k, int64_t rc, chunk_t* __restrict__ out,
    int capacity, int e, int32_t rows, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ offsets) {
  constexpr int U = 4;  // chunks in flight per lane
  const int lane = lane_id();
  const int t = blockIdx.x * kWavesPerBlock + wave_in_block();
  if (t < s) {
    int d[KMAX];
    load_dst<KMAX>(dst, t, k, d);
    if (verify_idx != nullptr) {
      const size_t o = static_cast<size_t>(t) * k + lane;
      const bool bad = lane < k && verify_idx[o] != route_idx[o];
      if (__ballot(bad) != 0ull && lane == 0) atomicOr(flags, 4);
    }
    const chunk_t* xr = x + static_cast<size_t>(t) * rc;
    for (int64_t c0 = lane; c0 < rc; c0 += U * kWave) {
      chunk_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * kWave;
        if (c < rc) v[u] = *(xr + c);
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (d[j] >= 0) {
          chunk_t* o = out + static_cast<size_t>(d[j]) * rc;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + u * kWave;
            if (c < rc) o[c] = v[u];
          }
        }
      }
    }
  }
  zero_unfilled_rows(out, rc, capacity, e, rows, kept, offsets);
}

// ---------------------------------------------------------------------------------
// combine (weighted) and dispatch backward (unweighted)

template <int DT, int KMAX, bool WEIGHTED>
__global__ __launch_bounds__(kBlock) void combine_kernel(const chunk_t* __restrict__ rows_in,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ dst,
                                                         int s, int k, int64_t rc,
                                                         chunk_t* __restrict__ y) {
  constexpr int N = ChunkElems<DT>::value;
  const int lane = lane_id();
  const int t = blockIdx.x * kWavesPerBlock + wave_in_block();
  if (t >= s) return;
  int d[KMAX];
  load_dst<KMAX>(dst, t, k, d);
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    wt[j] = (WEIGHTED && j < k) ? w[static_cast<size_t>(t) * k + j] : 1.0f;

  chunk_t* yr = y + static_cast<size_t>(t) * rc;
  for (int64_t c = lane; c < rc; c += kWave) {
    chunk_t v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (d[j] >= 0) v[j] = *(rows_in + static_cast<size_t>(d[j]) * rc + c);
    float acc[N];
#pragma unroll
    for (int n = 0; n < N; ++n) acc[n] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (d[j] >= 0) {
        float f[N];
        unpack<DT>(v[j], f);
#pragma unroll
        for (int n = 0; n < N; ++n)
          acc[n] = WEIGHTED ? __fadd_rn(acc[n], __fmul_rn(wt[j], f[n])) : __fadd_rn(acc[n], f[n]);
      }
    }
    yr[c] = pack<DT>(acc);
  }
}

// ---------------------------------------------------------------------------------
// combine backward: grad_E rows and grad_w

template <int DT, int KMAX>
__global__ __launch_bounds__(kBlock) void combine_backward_kernel(
    const chunk_t* __restrict__ gy, const chunk_t* __restrict__ E, const float* __restrict__ w,
    const int32_t* __restrict__ dst, int s, int k, int64_t rc, chunk_t* __restrict__ gE,
    float* __restrict__ gw, int capacity, int e, int32_t rows,
    const int32_t* __restrict__ kept, const int32_t* __restrict__ offsets) {
  constexpr int N = ChunkElems<DT>::value;
  const int lane = lane_id();
  const int t = blockIdx.x * kWavesPerBlock + wave_in_block();
  if (t < s) {
    int d[KMAX];
    load_dst<KMAX>(dst, t, k, d);
    float wt[KMAX];
    double part[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      wt[j] = (j < k) ? w[static_cast<size_t>(t) * k + j] : 0.0f;
      part[j] = 0.0;
    }
    const chunk_t* gr = gy + static_cast<size_t>(t) * rc;
    for (int64_t c = lane; c < rc; c += kWave) {
      float g[N];
      unpack<DT>(*(gr + c), g);
      chunk_t v[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (d[j] >= 0) v[j] = *(E + static_cast<size_t>(d[j]) * rc + c);
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (d[j] >= 0) {
          float f[N], o[N];
          unpack<DT>(v[j], f);
#pragma unroll
          for (int n = 0; n < N; ++n) {
            // float32 x float32 is exact in float64, so the fma rounds only the sum
            part[j] = fma(static_cast<double>(g[n]), static_cast<double>(f[n]), part[j]);
            o[n] = __fmul_rn(wt[j], g[n]);
          }
          gE[static_cast<size_t>(d[j]) * rc + c] = pack<DT>(o);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const double tot = wave_sum(part[j]);
        if (lane == 0) gw[static_cast<size_t>(t) * k + j] = d[j] >= 0 ? static_cast<float>(tot) : 0.0f;
      }
    }
  }
  zero_unfilled_rows(gE, rc, capacity, e, rows, kept, offsets);
}

// ---------------------------------------------------------------------------------
// launchers

static int row_grid(const LayoutView& L, bool writes_rows) {
  int64_t g = (static_cast<int64_t>(L.s) + kWavesPerBlock - 1) / kWavesPerBlock;
  if (writes_rows && L.capacity > 0) {
    // enough waves for the zero padding even when there are few tokens
    int64_t pad = (L.rows + kWavesPerBlock - 1) / kWavesPerBlock;
    if (pad > 2048) pad = 2048;
    if (g < pad) g = pad;
  }
  return static_cast<int>(g);
}

template <int KMAX>
static void dispatch_k(const LayoutView& L, const int32_t* verify_idx, const void* x,
                       int64_t rc, void* out, int grid, hipStream_t stream) {
  dispatch_kernel<KMAX><<<grid, kBlock, 0, stream>>>(
      static_cast<const chunk_t*>(x), L.dst, verify_idx, L.route_idx, L.flags, L.s, L.k, rc,
      static_cast<chunk_t*>(out), L.capacity, L.e, static_cast<int32_t>(L.rows), L.kept, L.offsets);
}

hipError_t launch_dispatch(const LayoutView& L, const int32_t* verify_idx, const void* x,
                           int64_t rc, void* out, hipStream_t stream) {
  const int grid = row_grid(L, true);
  if (grid == 0) return hipSuccess;
  switch (route_bound(L.k)) {
    case 1: dispatch_k<1>(L, verify_idx, x, rc, out, grid, stream); break;
    case 2: dispatch_k<2>(L, verify_idx, x, rc, out, grid, stream); break;
    case 4: dispatch_k<4>(L, verify_idx, x, rc, out, grid, stream); break;
    case 8: dispatch_k<8>(L, verify_idx, x, rc, out, grid, stream); break;
    default: dispatch_k<16>(L, verify_idx, x, rc, out, grid, stream); break;
  }
  return hipGetLastError();
}

template <int DT, int KMAX>
static void combine_k(const LayoutView& L, const void* in, const float* w, int64_t rc, void* y,
                      int grid, hipStream_t stream) {
  if (w != nullptr)
    combine_kernel<DT, KMAX, true><<<grid, kBlock, 0, stream>>>(
        static_cast<const chunk_t*>(in), w, L.dst, L.s, L.k, rc, static_cast<chunk_t*>(y));
  else
    combine_kernel<DT, KMAX, false><<<grid, kBlock, 0, stream>>>(
        static_cast<const chunk_t*>(in), nullptr, L.dst, L.s, L.k, rc, static_cast<chunk_t*>(y));
}

template <int DT>
static void combine_dt(const LayoutView& L, const void* in, const float* w, int64_t rc, void* y,
                       int grid, hipStream_t stream) {
  switch (route_bound(L.k)) {
    case 1: combine_k<DT, 1>(L, in, w, rc, y, grid, stream); break;
    case 2: combine_k<DT, 2>(L, in, w, rc, y, grid, stream); break;
    case 4: combine_k<DT, 4>(L, in, w, rc, y, grid, stream); break;
    case 8: combine_k<DT, 8>(L, in, w, rc, y, grid, stream); break;
    default: combine_k<DT, 16>(L, in, w, rc, y, grid, stream); break;
  }
}

hipError_t launch_combine(const LayoutView& L, const void* in, const float* w, int64_t rc,
                          int dtype, void* y, hipStream_t stream) {
  const int grid = row_grid(L, false);
  if (grid == 0) return hipSuccess;
  switch (dtype) {
    case kF32: combine_dt<kF32>(L, in, w, rc, y, grid, stream); break;
    case kBF16: combine_dt<kBF16>(L, in, w, rc, y, grid, stream); break;
    default: combine_dt<kF16>(L, in, w, rc, y, grid, stream); break;
  }
  return hipGetLastError();
}

template <int DT, int KMAX>
static void combine_bwd_k(const LayoutView& L, const void* gy, const void* E, const float* w,
                          int64_t rc, void* gE, float* gw, int grid, hipStream_t stream) {
  combine_backward_kernel<DT, KMAX><<<grid, kBlock, 0, stream>>>(
      static_cast<const chunk_t*>(gy), static_cast<const chunk_t*>(E), w, L.dst, L.s, L.k, rc,
      static_cast<chunk_t*>(gE), gw, L.capacity, L.e, static_cast<int32_t>(L.rows), L.kept,
      L.offsets);
}

template <int DT>
static void combine_bwd_dt(const LayoutView& L, const void* gy, const void* E, const float* w,
                           int64_t rc, void* gE, float* gw, int grid, hipStream_t stream) {
  switch (route_bound(L.k)) {
    case 1: combine_bwd_k<DT, 1>(L, gy, E, w, rc, gE, gw, grid, stream); break;
    case 2: combine_bwd_k<DT, 2>(L, gy, E, w, rc, gE, gw, grid, stream); break;
    case 4: combine_bwd_k<DT, 4>(L, gy, E, w, rc, gE, gw, grid, stream); break;
    case 8: combine_bwd_k<DT, 8>(L, gy, E, w, rc, gE, gw, grid, stream); break;
    default: combine_bwd_k<DT, 16>(L, gy, E, w, rc, gE, gw, grid, stream); break;
  }
}

hipError_t launch_combine_backward(const LayoutView& L, const void* gy, const void* E,
                                   const float* w, int64_t rc, int dtype, void* gE, float* gw,
                                   hipStream_t stream) {
  const int grid = row_grid(L, true);
  if (grid == 0) return hipSuccess;
  switch (dtype) {
    case kF32: combine_bwd_dt<kF32>(L, gy, E, w, rc, gE, gw, grid, stream); break;
    case kBF16: combine_bwd_dt<kBF16>(L, gy, E, w, rc, gE, gw, grid, stream); break;
    default: combine_bwd_dt<kF16>(L, gy, E, w, rc, gE, gw, grid, stream); break;
  }
  return hipGetLastError();
}

}  // namespace moe
