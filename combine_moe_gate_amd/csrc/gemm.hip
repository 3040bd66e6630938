// Grouped expert GEMM over a layout's segments, with the dispatch fused into its
// operand loads, on gfx950 matrix cores.
//
// For expert x and each placed row r of its segment [offsets[x], offsets[x] + kept[x]):
//     out[r, :] = A(r) @ W[x]^T,  A(r) = x[src[r]] (gathered) or a[r] (a dispatched buffer)
// with W [e, n, m] (output x input features). This is the consumer of the layout's
// per-expert offsets (DeepSpeed PR "Add an opt-in DeepEP transport for the AutoEP expert
// all-to-all", review-fix commit: the grouped GEMM takes its groups from the prefix sum);
// gathering A's rows straight from the token rows fuses the permute into the GEMM's
// prologue, so the [rows, m] buffer is never written or read.
//
// Tiling: a workgroup computes a 128 x 128 tile of one expert's rows x output features,
// K in steps of 32. Its four waves each own 64 x 64 as 2 x 2 MFMA tiles of 32 x 32
// (v_mfma_f32_32x32x16 bf16/f16, float32 accumulators). A and B tiles are staged in LDS
// K-contiguous (rows padded to 80 bytes), double-buffered, the next K step's global loads
// in flight while the current one is multiplied. Lane l of an MFMA reads row l%32,
// K elements 8*(l/32)..+7 of each operand (one ds_read_b128) and holds output rows
// 8*(v/4) + 4*(l/32) + v%4, column l%32 for v = 0..15.
//
// Workgroup order: tiles that share a row-block (the gathered A rows) are placed on one
// XCD (workgroups are dealt round-robin over the 8 XCDs), so those rows stay in that
// XCD's L2 while its workgroups sweep the output features.
#include "internal.h"
#include "moe_device.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;
constexpr int kGemmBK = 32;
constexpr int kGemmLdsK = kGemmBK + 8;  // padded LDS row, in elements (80 bytes)
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;

template <int DT>
__device__ __forceinline__ f32x16_t mfma_32x32x16(const chunk_t& a, const chunk_t& b, f32x16_t c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                   __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ uint16_t narrow(float v) {
  if constexpr (DT == kBF16) return static_cast<uint16_t>(f32x2_to_bf16x2_rne(v, 0.0f) & 0xffffu);
  else return static_cast<uint16_t>(f32_to_f16_rne(v));
}

// The row-block's expert: experts own ceil(kept[x] / 128) row-blocks each, in expert order.
// Wave 0 scans the per-expert block counts 64 experts at a time. Returns -1 past the end.
__device__ __forceinline__ void find_row_block(int rb, int e, const int32_t* __restrict__ kept,
                                               int* expert, int* rb_in) {
  const int lane = lane_id();
  int before = 0;
  *expert = -1;
  *rb_in = 0;
  for (int c0 = 0; c0 < e; c0 += kWave) {
    const int x = c0 + lane;
    const int nb = x < e ? (kept[x] + kGemmBM - 1) / kGemmBM : 0;
    int incl = nb;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    const int excl = incl - nb;
    const uint64_t hit = __ballot(x < e && rb >= before + excl && rb < before + incl);
    if (hit != 0ull) {
      const int owner = static_cast<int>(__builtin_ctzll(hit));
      *expert = c0 + owner;
      *rb_in = rb - before - __builtin_amdgcn_readlane(excl, owner);
      return;
    }
    before += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
}

template <int DT, bool GATHER, bool SCALE>
__global__ __launch_bounds__(kGemmThreads) void expert_gemm_kernel(
    const chunk_t* __restrict__ a, const chunk_t* __restrict__ wts,
    const float* __restrict__ route_w, const int32_t* __restrict__ dst,
    const int32_t* __restrict__ src, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ offsets, int e, int k, int m, int n, int row_blocks,
    int col_blocks, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kGemmBM * kGemmLdsK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kGemmBN * kGemmLdsK];
  __shared__ int32_t row_src[kGemmBM];
  __shared__ float row_scale[kGemmBM];
  __shared__ int32_t tile_info[2];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = wave_in_block();

  // workgroup -> (row-block, col-block); the col-blocks of a row-block share an XCD
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int rb = xcd + kXcds * (slot / col_blocks);
  const int cb = slot % col_blocks;
  if (rb >= row_blocks) return;  // uniform per workgroup
  if (wv == 0) {
    int x, rb_in;
    find_row_block(rb, e, kept, &x, &rb_in);
    if (lane == 0) {
      tile_info[0] = x;
      tile_info[1] = rb_in;
    }
  }
  __syncthreads();
  const int x = tile_info[0];
  if (x < 0) return;  // past the last row-block in use: uniform per workgroup
  const int rb_in = tile_info[1];
  const int row0 = offsets[x] + rb_in * kGemmBM;
  const int rem = kept[x] - rb_in * kGemmBM;
  const int nrows = rem < kGemmBM ? rem : kGemmBM;
  const int col0 = cb * kGemmBN;

  for (int i = tid; i < kGemmBM; i += kGemmThreads) {
    int sr = -1;
    float sc = 1.0f;
    if (i < nrows) {
      const int r = row0 + i;
      const int t = src[r];
      sr = GATHER ? t : r;
      if constexpr (SCALE) {
        for (int j = 0; j < k; ++j)
          if (dst[static_cast<size_t>(t) * k + j] == r) sc = route_w[static_cast<size_t>(t) * k + j];
      }
    }
    row_src[i] = sr;
    row_scale[i] = sc;
  }
  __syncthreads();

  const int kchunks = m / 8;  // 16-byte chunks per operand row
  const int nk = (m + kGemmBK - 1) / kGemmBK;
  const chunk_t zero = {0u, 0u, 0u, 0u};
  const chunk_t* wx = wts + static_cast<size_t>(x) * n * kchunks;

  // global -> register staging: each thread moves 2 chunks of A and 2 of B per K step
  chunk_t ra[2], rbv[2];
  auto load_tiles = [&](int kt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * kGemmThreads;
      const int row = c >> 2, kc = c & 3;
      const int kq = kt * (kGemmBK / 8) + kc;  // chunk index along K
      const int sr = row_src[row];
      ra[h] = (sr >= 0 && kq < kchunks) ? a[static_cast<size_t>(sr) * kchunks + kq] : zero;
      const int j = col0 + row;
      rbv[h] = (j < n && kq < kchunks) ? wx[static_cast<size_t>(j) * kchunks + kq] : zero;
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * kGemmThreads;
      const int row = c >> 2, kc = c & 3;
      *reinterpret_cast<chunk_t*>(&As[buf][row * kGemmLdsK + kc * 8]) = ra[h];
      *reinterpret_cast<chunk_t*>(&Bs[buf][row * kGemmLdsK + kc * 8]) = rbv[h];
    }
  };

  const int wm = wv >> 1, wn = wv & 1;  // this wave's 64 x 64 quarter
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.0f;

  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kGemmBK / 16; ++ks) {
      chunk_t fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        fa[i] = *reinterpret_cast<const chunk_t*>(&As[cur][row * kGemmLdsK + ks * 16 + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int col = wn * 64 + jj * 32 + (lane & 31);
        fb[jj] = *reinterpret_cast<const chunk_t*>(&Bs[cur][col * kGemmLdsK + ks * 16 + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = mfma_32x32x16<DT>(fa[i], fb[jj], acc[i][jj]);
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // epilogue: optional route weight (weights after the experts), one narrowing
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int col = col0 + wn * 64 + jj * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < nrows && col < n) {
          float f = acc[i][jj][v];
          if constexpr (SCALE) f = __fmul_rn(row_scale[row], f);
          out[static_cast<size_t>(row0 + row) * n + col] = narrow<DT>(f);
        }
      }
    }
  }
}

// An upper bound on the row-blocks in use, known on the host without reading the layout.
static int64_t row_block_bound(const LayoutView& L) {
  if (L.capacity > 0) return static_cast<int64_t>(L.e) * ((L.capacity + kGemmBM - 1) / kGemmBM);
  return (static_cast<int64_t>(L.s) * L.k + kGemmBM - 1) / kGemmBM + L.e;
}

int64_t expert_gemm_grid(const LayoutView& L, int n) {
  if (L.s == 0) return 0;
  const int64_t col_blocks = (n + kGemmBN - 1) / kGemmBN;
  return kXcds * col_blocks * ((row_block_bound(L) + kXcds - 1) / kXcds);
}

template <int DT, bool GATHER, bool SCALE>
static void gemm_launch(const LayoutView& L, const void* a, const void* w, const float* route_w,
                        int m, int n, void* out, hipStream_t stream) {
  const int64_t grid = expert_gemm_grid(L, n);
  if (grid == 0) return;
  const int col_blocks = (n + kGemmBN - 1) / kGemmBN;
  expert_gemm_kernel<DT, GATHER, SCALE><<<static_cast<unsigned>(grid), kGemmThreads, 0, stream>>>(
      static_cast<const chunk_t*>(a), static_cast<const chunk_t*>(w), route_w, L.dst, L.src, L.kept,
      L.offsets, L.e, L.k, m, n, static_cast<int>(row_block_bound(L)), col_blocks,
      static_cast<uint16_t*>(out));
}

template <int DT>
static void gemm_dt(const LayoutView& L, const void* a, bool gather, const void* w,
                    const float* route_w, int m, int n, void* out, hipStream_t stream) {
  if (gather) {
    if (route_w) gemm_launch<DT, true, true>(L, a, w, route_w, m, n, out, stream);
    else gemm_launch<DT, true, false>(L, a, w, route_w, m, n, out, stream);
  } else {
    if (route_w) gemm_launch<DT, false, true>(L, a, w, route_w, m, n, out, stream);
    else gemm_launch<DT, false, false>(L, a, w, route_w, m, n, out, stream);
  }
}

hipError_t launch_expert_gemm(const LayoutView& L, const void* a, bool gather, const void* w,
                              const float* route_w, int m, int n, int dtype, void* out,
                              hipStream_t stream) {
  if (L.s > 0) {
    if (dtype == kBF16) gemm_dt<kBF16>(L, a, gather, w, route_w, m, n, out, stream);
    else gemm_dt<kF16>(L, a, gather, w, route_w, m, n, out, stream);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // rows no route fills are zero
  return launch_zero_unfilled_rows(L, out, static_cast<int64_t>(n) * 2 / 16, stream);
}

}  // namespace moe
