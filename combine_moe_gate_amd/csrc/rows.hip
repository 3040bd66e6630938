// Row movers on gfx950: dispatch (and its replay), weighted combine, and the two
// backward passes.
//
// All four are HBM-bound row gathers/scatters, not contractions, so there is no MFMA
// here. Work is token-major: workgroup t owns token t (its k destination rows come
// from the layout's dst and live in scalar registers). A row of rc 16-byte chunks is
// cut into ng groups of 64*U chunks; the workgroup's waves (up to eight) take the
// groups in turn, lane l moving chunks l, l+64, ... of a group (global_load/store_dwordx4,
// fully coalesced). With U = 1 and eight waves, an 8 KiB row is one group per wave:
// measured 1.5-3.5% faster than four waves of two groups (or of U = 2) on 4-8 KiB rows. The first group a token visits is rotated by the token id, so that
// the waves in flight spread over all offsets within rows instead of all reading
// the same offset of 8 KiB-aligned rows at once (measured: +20-30% on a 512 MiB
// buffer).
//
//   dispatch          x[t] read once, written to its k rows (DeepSpeed PR "Add an
//                     opt-in DeepEP transport for the AutoEP expert all-to-all", first
//                     commit: tokens are taken before top-k expansion and replicated).
//   combine           a token's k rows loaded together, summed in route order in
//                     float32 with separate multiply and add, rounded once (DeepSpeed
//                     PR "MoE dispatch: fix silent Tutel + TP corruption, speed up
//                     native and Tutel paths", part 3: fp32 accumulation; PR 8213's
//                     review thread on combine weights: the weights are applied).
//   dispatch backward the same kernel without weights (dispatch and combine are adjoint,
//                     PR 8213 first commit).
//   combine backward  grad_y[t] read once (normal loads, like x in dispatch: measured
//                     faster than nontemporal ones); each route gets the weighted copy in its row
//                     and the dot product with its expert row accumulates in float64,
//                     per wave, then across the workgroup's waves through LDS in a
//                     fixed order (the combine's adjoint, plus the weights' gradient of
//                     PR 8213's review-fix commit).
//
//   weighted dispatch the combine backward's scatter without the dot: out[dst] = w * x
//                     (the weights applied before the experts; PR 8213's score_apply).
//   its backward      the weighted combine of grad_out, plus grad_w = <grad_out[dst], x>
//                     accumulated like the combine backward's dot.
//
// Stores: every row kernel writes with the sc1 (device-scope) bit, without the
// nontemporal hint, so its rows are written through the XCD's L2 into the Infinity Cache,
// which keeps them until they are evicted and the next kernel can read them from there.
// Measured on MI355X against nontemporal (streaming) stores, each kernel alone after a
// 1 GiB cache flush: faster for the dispatch, the combine and the combine backward on
// every workload (on the 8192-token, 4096-wide Zipf batch: dispatch 87 against 119 us,
// combine 100 against 106, combine backward 178 against 209). Back to back in one step,
// where a kernel also pays for evicting the lines the previous one left, the two are
// within a few percent either way. The gathered rows of the combine and its backward are
// loaded with the nontemporal hint (they are read once).
//
// Rows that no route points at (the tail of each expert segment: capacity or pad rows,
// and rows past the last segment) are zero-filled by extra workgroups after the token
// workgroups, in the kernels that write [rows, m] buffers. No floating-point atomics:
// results are deterministic.
#include "internal.h"
#include "moe_device.h"

namespace moe {

constexpr int kRowBlock = 512;                   // threads per workgroup of the row kernels
constexpr int kRowWaves = kRowBlock / kWave;

template <bool NT>
__device__ __forceinline__ chunk_t load_chunk(const chunk_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// One 16-byte row chunk stored with the sc1 bit (no clang builtin names that cache
// policy, hence the vector store written out; it only reads its operands).
__device__ __forceinline__ void store_chunk(chunk_t* p, const chunk_t& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}


// How a row is cut into groups and how many waves share a token.
struct RowSplit {
  int64_t rc;   // 16-byte chunks per row
  int64_t ng;   // groups of 64*U chunks per row
  int wpb;      // waves per workgroup (one token per workgroup)
};

// The token owned by this workgroup's wave `wv` visits groups gi = wv, wv+wpb, ...;
// group gi maps to g = (gi + t) mod ng.
__device__ __forceinline__ int64_t rotated_group(int64_t gi, int64_t t, int64_t ng) {
  int64_t g = gi + t % ng;
  return g >= ng ? g - ng : g;
}

// Workgroups past the s token workgroups zero the rows that no placed route fills:
// segment x in [0, e) has rows [offsets[x] + kept[x], offsets[x+1]) unfilled (capacity
// or pad rows), each (segment, sub-stride) pair being one work item so that a few long
// gaps still spread over many waves; then every padding wave strides over the tail
// [offsets[e], rows), which is long when a padded layout's row bound is far above
// the rows in use.
__device__ __forceinline__ void zero_unfilled_rows(chunk_t* __restrict__ out, int64_t rc, int s,
                                                   int e, int32_t rows,
                                                   const int32_t* __restrict__ kept,
                                                   const int32_t* __restrict__ offsets) {
  const int lane = lane_id();
  const int wpb = blockDim.x >> 6;
  const int32_t wave = (blockIdx.x - s) * wpb + wave_in_block();
  const int32_t nwaves = (gridDim.x - s) * wpb;
  const int32_t R = nwaves > e ? nwaves / e : 1;
  const chunk_t z = {0u, 0u, 0u, 0u};
  for (int32_t item = wave; item < e * R; item += nwaves) {
    const int32_t x = item % e, sub = item / e;
    const int32_t r1 = offsets[x + 1];
    for (int32_t r = offsets[x] + kept[x] + sub; r < r1; r += R) {
      chunk_t* o = out + static_cast<size_t>(r) * rc;
      for (int64_t c = lane; c < rc; c += kWave) store_chunk(o + c, z);
    }
  }
  for (int32_t r = offsets[e] + wave; r < rows; r += nwaves) {
    chunk_t* o = out + static_cast<size_t>(r) * rc;
    for (int64_t c = lane; c < rc; c += kWave) store_chunk(o + c, z);
  }
}

template <int KMAX>
__device__ __forceinline__ void load_dst(const int32_t* __restrict__ dst, int t, int k,
                                         int (&d)[KMAX]) {
#pragma unroll
  for (int j = 0; j < KMAX; ++j) d[j] = (j < k) ? dst[static_cast<size_t>(t) * k + j] : -1;
}

// ---------------------------------------------------------------------------------
// dispatch: normal loads of x (tokens are small and may be reread by a replay), cached
// stores of the buffer rows

template <int KMAX, int U>
__global__ __launch_bounds__(kRowBlock) void dispatch_kernel(
    const chunk_t* __restrict__ x, const int32_t* __restrict__ dst,
    const int32_t* __restrict__ verify_idx, const int32_t* __restrict__ route_idx,
    int32_t* __restrict__ flags, int s, int k, RowSplit sp, chunk_t* __restrict__ out,
    int capacity, int e, int32_t rows, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ offsets) {
  if (static_cast<int>(blockIdx.x) >= s) {
    zero_unfilled_rows(out, sp.rc, s, e, rows, kept, offsets);
    return;
  }
  const int lane = lane_id();
  const int wv = wave_in_block();
  const int t = blockIdx.x;
  int d[KMAX];
  load_dst<KMAX>(dst, t, k, d);
  if (verify_idx != nullptr && wv == 0) {
    const size_t o = static_cast<size_t>(t) * k + lane;
    const bool bad = lane < k && verify_idx[o] != route_idx[o];
    if (__ballot(bad) != 0ull && lane == 0) atomicOr(flags, 4);
  }
  const chunk_t* xr = x + static_cast<size_t>(t) * sp.rc;
  for (int64_t gi = wv; gi < sp.ng; gi += sp.wpb) {
    const int64_t c0 = rotated_group(gi, t, sp.ng) * (kWave * U) + lane;
    chunk_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave;
      if (c < sp.rc) v[u] = load_chunk<false>(xr + c);
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (d[j] >= 0) {
        chunk_t* o = out + static_cast<size_t>(d[j]) * sp.rc;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t c = c0 + u * kWave;
          if (c < sp.rc) store_chunk(o + c, v[u]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// combine (weighted), dispatch backward (unweighted) and the weighted dispatch's
// backward (weighted, plus the dot of each row with the token's own row): nontemporal
// loads of the k rows, one store per chunk

// Per-route float64 partials of one wave, summed across the workgroup's waves through
// LDS in wave order; lane j < k of wave 0 writes grad_w[t, j] (0 for a dropped route).
template <int KMAX>
__device__ __forceinline__ void reduce_route_dots(double (&part)[KMAX], const int (&d)[KMAX],
                                                  int t, int k, int wpb, float* __restrict__ gw,
                                                  double (*wave_part)[KMAX]) {
  const int lane = lane_id();
  const int wv = wave_in_block();
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      const double tot = wave_sum(part[j]);
      if (lane == 0) wave_part[wv][j] = tot;
    }
  }
  __syncthreads();
  if (wv == 0 && lane < k) {
    double tot = 0.0;
    for (int q = 0; q < wpb; ++q) tot += wave_part[q][lane];
    int dj = -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j == lane) dj = d[j];
    gw[static_cast<size_t>(t) * k + lane] = dj >= 0 ? static_cast<float>(tot) : 0.0f;
  }
}

template <int DT, int KMAX, bool WEIGHTED, bool WITH_DOT, int U>
__global__ __launch_bounds__(kRowBlock) void combine_kernel(const chunk_t* __restrict__ rows_in,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ dst,
                                                         int s, int k, RowSplit sp,
                                                         chunk_t* __restrict__ y,
                                                         const chunk_t* __restrict__ xdot,
                                                         float* __restrict__ gw) {
  constexpr int N = ChunkElems<DT>::value;
  __shared__ double wave_part[kRowWaves][KMAX];
  const int lane = lane_id();
  const int wv = wave_in_block();
  const int t = blockIdx.x;
  if (t >= s) return;
  int d[KMAX];
  load_dst<KMAX>(dst, t, k, d);
  float wt[KMAX];
  double part[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    wt[j] = (WEIGHTED && j < k) ? w[static_cast<size_t>(t) * k + j] : 1.0f;
    part[j] = 0.0;
  }

  chunk_t* yr = y + static_cast<size_t>(t) * sp.rc;
  const chunk_t* xr = WITH_DOT ? xdot + static_cast<size_t>(t) * sp.rc : nullptr;
  for (int64_t gi = wv; gi < sp.ng; gi += sp.wpb) {
    const int64_t c0 = rotated_group(gi, t, sp.ng) * (kWave * U) + lane;
    chunk_t v[U][KMAX];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (d[j] >= 0 && c < sp.rc)
          v[u][j] = load_chunk<true>(rows_in + static_cast<size_t>(d[j]) * sp.rc + c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave;
      if (c < sp.rc) {
        float xs[N];
        if constexpr (WITH_DOT) unpack<DT>(load_chunk<false>(xr + c), xs);
        float acc[N];
#pragma unroll
        for (int n = 0; n < N; ++n) acc[n] = 0.0f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (d[j] >= 0) {
            float f[N];
            unpack<DT>(v[u][j], f);
#pragma unroll
            for (int n = 0; n < N; ++n) {
              acc[n] = WEIGHTED ? __fadd_rn(acc[n], __fmul_rn(wt[j], f[n])) : __fadd_rn(acc[n], f[n]);
              if constexpr (WITH_DOT)
                part[j] = fma(static_cast<double>(xs[n]), static_cast<double>(f[n]), part[j]);
            }
          }
        }
        store_chunk(yr + c, pack<DT>(acc));
      }
    }
  }
  if constexpr (WITH_DOT) reduce_route_dots<KMAX>(part, d, t, k, sp.wpb, gw, wave_part);
}

// ---------------------------------------------------------------------------------
// weighted scatter: out[dst[t,j]] = w[t,j] * in[t] for every placed route, and with
// WITH_DOT also grad_w[t,j] = <in[t], E[dst[t,j]]>. The combine backward is the scatter
// of grad_y with the dot against the expert rows; the weighted dispatch is the scatter
// of x without it.

template <int DT, int KMAX, bool WITH_DOT, int U>
__global__ __launch_bounds__(kRowBlock) void weighted_scatter_kernel(
    const chunk_t* __restrict__ in, const chunk_t* __restrict__ E, const float* __restrict__ w,
    const int32_t* __restrict__ dst, int s, int k, RowSplit sp, chunk_t* __restrict__ out,
    float* __restrict__ gw, int e, int32_t rows, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ offsets) {
  constexpr int N = ChunkElems<DT>::value;
  __shared__ double wave_part[kRowWaves][KMAX];
  if (static_cast<int>(blockIdx.x) >= s) {
    zero_unfilled_rows(out, sp.rc, s, e, rows, kept, offsets);
    return;
  }
  const int lane = lane_id();
  const int wv = wave_in_block();
  const int t = blockIdx.x;
  int d[KMAX];
  load_dst<KMAX>(dst, t, k, d);
  float wt[KMAX];
  double part[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    wt[j] = (j < k) ? w[static_cast<size_t>(t) * k + j] : 0.0f;
    part[j] = 0.0;
  }
  const chunk_t* ir = in + static_cast<size_t>(t) * sp.rc;
  for (int64_t gi = wv; gi < sp.ng; gi += sp.wpb) {
    const int64_t c0 = rotated_group(gi, t, sp.ng) * (kWave * U) + lane;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave;
      if (c < sp.rc) {
        float g[N];
        // the token's own row: normal loads (measured faster than nontemporal ones)
        unpack<DT>(load_chunk<false>(ir + c), g);
        chunk_t v[KMAX];
        if constexpr (WITH_DOT) {
#pragma unroll
          for (int j = 0; j < KMAX; ++j)
            if (d[j] >= 0) v[j] = load_chunk<true>(E + static_cast<size_t>(d[j]) * sp.rc + c);
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (d[j] >= 0) {
            float o[N];
            if constexpr (WITH_DOT) {
              float f[N];
              unpack<DT>(v[j], f);
#pragma unroll
              for (int n = 0; n < N; ++n)
                // float32 x float32 is exact in float64, so the fma rounds only the sum
                part[j] = fma(static_cast<double>(g[n]), static_cast<double>(f[n]), part[j]);
            }
#pragma unroll
            for (int n = 0; n < N; ++n) o[n] = __fmul_rn(wt[j], g[n]);
            store_chunk(out + static_cast<size_t>(d[j]) * sp.rc + c, pack<DT>(o));
          }
        }
      }
    }
  }
  if constexpr (WITH_DOT) reduce_route_dots<KMAX>(part, d, t, k, sp.wpb, gw, wave_part);
}

// ---------------------------------------------------------------------------------
// launchers


static RowSplit make_split(int64_t rc, int U) {
  RowSplit sp;
  sp.rc = rc;
  sp.ng = (rc + kWave * U - 1) / (kWave * U);
  sp.wpb = static_cast<int>(sp.ng < kRowWaves ? sp.ng : kRowWaves);
  return sp;
}

// Workgroups that zero unfilled rows: enough for every capacity row or pad row; a few
// otherwise, where only flagged-invalid routes leave rows unfilled.
static int pad_blocks(const LayoutView& L, int wpb) {
  int64_t want = 16;
  if (L.capacity > 0) want = (L.rows + 8 * wpb - 1) / (8 * wpb);
  else if (L.pad_multiple > 1) want = (static_cast<int64_t>(L.e) * (L.pad_multiple - 1) + 8 * wpb - 1) / (8 * wpb);
  if (want < 16) want = 16;
  if (want > 4096) want = 4096;
  return L.s > 0 || L.rows > 0 ? static_cast<int>(want) : 0;
}

template <int KMAX, int U>
static void dispatch_k(const LayoutView& L, const int32_t* verify_idx, const void* x,
                       const RowSplit& sp, void* out, hipStream_t stream) {
  const int grid = L.s + pad_blocks(L, sp.wpb);
  if (grid == 0) return;
  dispatch_kernel<KMAX, U><<<grid, sp.wpb * kWave, 0, stream>>>(
      static_cast<const chunk_t*>(x), L.dst, verify_idx, L.route_idx, L.flags, L.s, L.k, sp,
      static_cast<chunk_t*>(out), L.capacity, L.e, static_cast<int32_t>(L.rows), L.kept,
      L.offsets);
}

template <int U>
static void dispatch_u(const LayoutView& L, const int32_t* verify_idx, const void* x,
                       const RowSplit& sp, void* out, hipStream_t stream) {
  switch (route_bound(L.k)) {
    case 1: dispatch_k<1, U>(L, verify_idx, x, sp, out, stream); break;
    case 2: dispatch_k<2, U>(L, verify_idx, x, sp, out, stream); break;
    case 4: dispatch_k<4, U>(L, verify_idx, x, sp, out, stream); break;
    case 8: dispatch_k<8, U>(L, verify_idx, x, sp, out, stream); break;
    default: dispatch_k<16, U>(L, verify_idx, x, sp, out, stream); break;
  }
}

hipError_t launch_dispatch(const LayoutView& L, const int32_t* verify_idx, const void* x,
                           int64_t rc, void* out, hipStream_t stream) {
  dispatch_u<1>(L, verify_idx, x, make_split(rc, 1), out, stream);
  return hipGetLastError();
}

// mode: 0 weighted combine, 1 unweighted sum, 2 weighted combine plus dots with xdot
template <int DT, int KMAX>
static void combine_k(const LayoutView& L, const void* in, const float* w, const RowSplit& sp,
                      void* y, const void* xdot, float* gw, int mode, hipStream_t stream) {
  const chunk_t* src = static_cast<const chunk_t*>(in);
  chunk_t* dsty = static_cast<chunk_t*>(y);
  const chunk_t* xd = static_cast<const chunk_t*>(xdot);
  if (mode == 0)
    combine_kernel<DT, KMAX, true, false, 1><<<L.s, sp.wpb * kWave, 0, stream>>>(src, w, L.dst, L.s, L.k, sp, dsty, nullptr, nullptr);
  else if (mode == 1)
    combine_kernel<DT, KMAX, false, false, 1><<<L.s, sp.wpb * kWave, 0, stream>>>(src, nullptr, L.dst, L.s, L.k, sp, dsty, nullptr, nullptr);
  else
    combine_kernel<DT, KMAX, true, true, 1><<<L.s, sp.wpb * kWave, 0, stream>>>(src, w, L.dst, L.s, L.k, sp, dsty, xd, gw);
}


template <int DT>
static void combine_dt(const LayoutView& L, const void* in, const float* w, const RowSplit& sp,
                       void* y, const void* xdot, float* gw, int mode, hipStream_t stream) {
  switch (route_bound(L.k)) {
    case 1: combine_k<DT, 1>(L, in, w, sp, y, xdot, gw, mode, stream); break;
    case 2: combine_k<DT, 2>(L, in, w, sp, y, xdot, gw, mode, stream); break;
    case 4: combine_k<DT, 4>(L, in, w, sp, y, xdot, gw, mode, stream); break;
    case 8: combine_k<DT, 8>(L, in, w, sp, y, xdot, gw, mode, stream); break;
    default: combine_k<DT, 16>(L, in, w, sp, y, xdot, gw, mode, stream); break;
  }
}

static hipError_t combine_any(const LayoutView& L, const void* in, const float* w, int64_t rc,
                              int dtype, void* y, const void* xdot, float* gw, int mode,
                              hipStream_t stream) {
  if (L.s == 0) return hipSuccess;
  const RowSplit sp = make_split(rc, 1);
  switch (dtype) {
    case kF32: combine_dt<kF32>(L, in, w, sp, y, xdot, gw, mode, stream); break;
    case kBF16: combine_dt<kBF16>(L, in, w, sp, y, xdot, gw, mode, stream); break;
    default: combine_dt<kF16>(L, in, w, sp, y, xdot, gw, mode, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const LayoutView& L, const void* in, const float* w, int64_t rc,
                          int dtype, void* y, hipStream_t stream) {
  return combine_any(L, in, w, rc, dtype, y, nullptr, nullptr, w != nullptr ? 0 : 1, stream);
}

hipError_t launch_dispatch_weighted_backward(const LayoutView& L, const void* grad_out,
                                             const void* x, const float* w, int64_t rc,
                                             int dtype, void* gx, float* gw, hipStream_t stream) {
  return combine_any(L, grad_out, w, rc, dtype, gx, x, gw, 2, stream);
}

template <int DT, int KMAX, bool WITH_DOT>
static void scatter_k(const LayoutView& L, const void* in, const void* E, const float* w,
                      const RowSplit& sp, void* out, float* gw, hipStream_t stream) {
  const int grid = L.s + pad_blocks(L, sp.wpb);
  if (grid == 0) return;
  weighted_scatter_kernel<DT, KMAX, WITH_DOT, 1><<<grid, sp.wpb * kWave, 0, stream>>>(
      static_cast<const chunk_t*>(in), static_cast<const chunk_t*>(E), w, L.dst, L.s, L.k, sp,
      static_cast<chunk_t*>(out), gw, L.e, static_cast<int32_t>(L.rows), L.kept, L.offsets);
}

template <int DT, bool WITH_DOT>
static void scatter_dt(const LayoutView& L, const void* in, const void* E, const float* w,
                       const RowSplit& sp, void* out, float* gw, hipStream_t stream) {
  switch (route_bound(L.k)) {
    case 1: scatter_k<DT, 1, WITH_DOT>(L, in, E, w, sp, out, gw, stream); break;
    case 2: scatter_k<DT, 2, WITH_DOT>(L, in, E, w, sp, out, gw, stream); break;
    case 4: scatter_k<DT, 4, WITH_DOT>(L, in, E, w, sp, out, gw, stream); break;
    case 8: scatter_k<DT, 8, WITH_DOT>(L, in, E, w, sp, out, gw, stream); break;
    default: scatter_k<DT, 16, WITH_DOT>(L, in, E, w, sp, out, gw, stream); break;
  }
}

template <bool WITH_DOT>
static hipError_t scatter_any(const LayoutView& L, const void* in, const void* E, const float* w,
                              int64_t rc, int dtype, void* out, float* gw, hipStream_t stream) {
  const RowSplit sp = make_split(rc, 1);
  switch (dtype) {
    case kF32: scatter_dt<kF32, WITH_DOT>(L, in, E, w, sp, out, gw, stream); break;
    case kBF16: scatter_dt<kBF16, WITH_DOT>(L, in, E, w, sp, out, gw, stream); break;
    default: scatter_dt<kF16, WITH_DOT>(L, in, E, w, sp, out, gw, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine_backward(const LayoutView& L, const void* gy, const void* E,
                                   const float* w, int64_t rc, int dtype, void* gE, float* gw,
                                   hipStream_t stream) {
  return scatter_any<true>(L, gy, E, w, rc, dtype, gE, gw, stream);
}

// Zero the unfilled rows of a buffer whose filled rows another kernel writes (the
// grouped expert GEMM's output).
__global__ __launch_bounds__(kRowBlock) void zero_rows_kernel(chunk_t* __restrict__ out, int64_t rc,
                                                           int e, int32_t rows,
                                                           const int32_t* __restrict__ kept,
                                                           const int32_t* __restrict__ offsets) {
  zero_unfilled_rows(out, rc, 0, e, rows, kept, offsets);
}

hipError_t launch_zero_unfilled_rows(const LayoutView& L, void* out, int64_t rc,
                                     hipStream_t stream) {
  const int grid = pad_blocks(L, kRowWaves);
  if (grid > 0)
    zero_rows_kernel<<<grid, kRowBlock, 0, stream>>>(static_cast<chunk_t*>(out), rc, L.e,
                                                  static_cast<int32_t>(L.rows), L.kept, L.offsets);
  return hipGetLastError();
}

hipError_t launch_dispatch_weighted(const LayoutView& L, const void* x, const float* w,
                                    int64_t rc, int dtype, void* out, hipStream_t stream) {
  return scatter_any<false>(L, x, nullptr, w, rc, dtype, out, nullptr, stream);
}

}  // namespace moe
