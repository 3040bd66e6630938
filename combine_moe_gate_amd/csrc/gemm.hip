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
// Tiling: a workgroup of four waves (2 x 2) computes a BM x BN tile of one expert's rows
// x output features; each wave owns WM x WN as (WM/32) x (WN/32) MFMA tiles of 32 x 32
// (v_mfma_f32_32x32x16 bf16/f16, float32 accumulators). Both operands are K-contiguous
// in memory (token rows; weight rows), so each is staged in LDS as [rows][BK] with rows
// padded by 16 bytes (conflict-free 16-byte fragment reads), double-buffered: the next
// K step's global loads are in flight while the current step is multiplied. Lane l of
// an MFMA reads row l%32, K elements 8*(l/32)..+7 of each operand (one ds_read_b128)
// and holds output rows 8*(v/4) + 4*(l/32) + v%4, column l%32 for v = 0..15.
//
// Schedule: the expert weights dominate the traffic (e * n * m elements, far above the
// L2), so tiles are ordered to read each weight tile few times. The tiles of all experts
// are numbered expert by expert; inside an expert, in bands of kBandRows row-blocks,
// column-block by column-block, row-block fastest. Workgroups are dealt round-robin over
// the 8 XCDs, so workgroup b takes tile (b mod 8) * T8 + b / 8 (T8 = ceil(tiles / 8)):
// each XCD walks one contiguous stretch of that order, and the workgroups resident on
// it at once share each weight tile across the band's row-blocks and each row-block's
// rows across neighbouring column-blocks through that XCD's L2.
#include "internal.h"
#include "moe_device.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;
constexpr int kBandRows = 4;

// A K step is 64 elements: 8 chunks of 16 bytes per staged row, 128 bytes.
constexpr int kGemmBK = 64;
constexpr int kRowBytes = kGemmBK * 2;

template <int WM, int WN>
struct GemmShape {
  static constexpr int BM = 2 * WM, BN = 2 * WN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  // one direct-to-LDS load instruction moves 64 lanes x 16 bytes = 8 staged rows
  static constexpr int A_LOADS = BM / 8 / 4;  // per wave per stage
  static constexpr int B_LOADS = BN / 8 / 4;
  static constexpr int STAGE_BYTES = (BM + BN) * kRowBytes;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
};

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

// Inclusive wave scan of a non-negative int.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(v, o, kWave);
    if (lane >= o) v += y;
  }
  return v;
}

struct TileCoord {
  int expert, rb, cb;  // expert; row-block within its segment; column-block
};

// This workgroup's tile (expert = -1: none). Wave 0 only; uniform across the wave.
template <int BM>
__device__ __forceinline__ TileCoord find_tile(int b, int e, const int32_t* __restrict__ kept,
                                               int col_blocks) {
  const int lane = lane_id();
  TileCoord tc{-1, 0, 0};
  int total = 0;  // row-blocks in use
  for (int c0 = 0; c0 < e; c0 += kWave) {
    const int x = c0 + lane;
    const int nb = x < e ? (kept[x] + BM - 1) / BM : 0;
    total += __builtin_amdgcn_readlane(wave_inclusive_scan(nb), kWave - 1);
  }
  const int64_t tiles = static_cast<int64_t>(total) * col_blocks;
  const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
  const int64_t slot = b / kXcds;
  const int64_t t = (b % kXcds) * per_xcd + slot;
  if (slot >= per_xcd || t >= tiles) return tc;
  int before = 0;  // row-blocks of earlier experts
  for (int c0 = 0; c0 < e; c0 += kWave) {
    const int x = c0 + lane;
    const int nb = x < e ? (kept[x] + BM - 1) / BM : 0;
    const int incl = wave_inclusive_scan(nb);
    const int excl = incl - nb;
    const int64_t lo = static_cast<int64_t>(before + excl) * col_blocks;
    const int64_t hi = static_cast<int64_t>(before + incl) * col_blocks;
    const uint64_t hit = __ballot(x < e && t >= lo && t < hi);
    if (hit != 0ull) {
      const int owner = static_cast<int>(__builtin_ctzll(hit));
      const int R = __builtin_amdgcn_readlane(nb, owner);
      const int64_t first = static_cast<int64_t>(before + __builtin_amdgcn_readlane(excl, owner)) * col_blocks;
      const int u = static_cast<int>(t - first);
      const int band = u / (kBandRows * col_blocks);
      const int left = R - band * kBandRows;
      const int rows_in_band = left < kBandRows ? left : kBandRows;
      const int v = u - band * kBandRows * col_blocks;
      tc.expert = c0 + owner;
      tc.cb = v / rows_in_band;
      tc.rb = band * kBandRows + v % rows_in_band;
      return tc;
    }
    before += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return tc;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate that waits for LDS (lgkm) operations only: vmcnt 63, expcnt 7,
// lgkmcnt 0.
constexpr int kWaitLdsOnly = 0xC07F;

// Stage one K step of rows into LDS with direct-to-LDS loads: instruction q of wave w
// fills staged rows [(w * LOADS + q) * 8, +8), lane l writing row lane/8, slot lane%8.
// Slot p of staged row R holds chunk p ^ (R % 8) of the step (an XOR swizzle, so the
// fragment reads below hit eight different bank groups); lane l therefore loads chunk
// (l % 8) ^ (l / 8). Returns whether this lane's chunk lies past the row end (then it
// loaded the row's first chunk and its slot must be cleared once the load has landed).
template <int LOADS>
__device__ __forceinline__ bool stage_rows(const chunk_t* const (&row)[LOADS], int kt, int c_lane,
                                           int kchunks, char* lds_rows) {
  const int kq = kt * (kGemmBK / 8) + c_lane;
  const bool past = kq >= kchunks;
  const int off = past ? 0 : kq;
#pragma unroll
  for (int q = 0; q < LOADS; ++q)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(row[q] + off),
                                     (lds_void_t*)(lds_rows + q * 64 * 16), 16, 0, 0);
  return past;
}

template <int LOADS>
__device__ __forceinline__ void clear_slots(char* lds_rows, int lane) {
  const chunk_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < LOADS; ++q) *reinterpret_cast<chunk_t*>(lds_rows + q * 64 * 16 + lane * 16) = z;
}

// One workgroup per CU (its LDS stages take most of the CU's 160 KiB), one wave per SIMD:
// the register file is this wave's, so the schedule may keep two fragment sets live.
template <int DT, bool GATHER, bool SCALE, int WM, int WN>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void expert_gemm_kernel(
    const chunk_t* __restrict__ a, const chunk_t* __restrict__ wts,
    const float* __restrict__ route_w, const int32_t* __restrict__ dst,
    const int32_t* __restrict__ src, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ offsets, int e, int k, int m, int n, int col_blocks,
    uint16_t* __restrict__ out) {
  using S = GemmShape<WM, WN>;
  extern __shared__ __attribute__((aligned(1024))) char lds[];  // [2][BM + BN rows][128 B]
  __shared__ int32_t row_src[S::BM];
  __shared__ float row_scale[S::BM];
  __shared__ int32_t tile_info[3];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = wave_in_block();

  if (wv == 0) {
    const TileCoord tc = find_tile<S::BM>(blockIdx.x, e, kept, col_blocks);
    if (lane == 0) {
      tile_info[0] = tc.expert;
      tile_info[1] = tc.rb;
      tile_info[2] = tc.cb;
    }
  }
  __syncthreads();
  const int x = tile_info[0];
  if (x < 0) return;  // no tile: uniform per workgroup
  const int rb = tile_info[1];
  const int row0 = offsets[x] + rb * S::BM;
  const int rem = kept[x] - rb * S::BM;
  const int nrows = rem < S::BM ? rem : S::BM;
  const int col0 = tile_info[2] * S::BN;

  for (int i = tid; i < S::BM; i += kGemmThreads) {
    // rows past the segment repeat its first row: their products land only in output
    // rows that are never stored
    const int r = row0 + (i < nrows ? i : 0);
    const int t = src[r];
    float sc = 1.0f;
    if constexpr (SCALE) {
      for (int j = 0; j < k; ++j)
        if (dst[static_cast<size_t>(t) * k + j] == r) sc = route_w[static_cast<size_t>(t) * k + j];
    }
    row_src[i] = GATHER ? t : r;
    row_scale[i] = sc;
  }
  __syncthreads();

  const int kchunks = m / 8;  // 16-byte chunks per operand row
  const int nk = (m + kGemmBK - 1) / kGemmBK;
  const chunk_t* wx = wts + static_cast<size_t>(x) * n * kchunks;
  const int c_lane = (lane & 7) ^ (lane >> 3);  // the chunk this lane stages in every row

  // row starts of the staged rows this lane loads (columns past n repeat column n - 1:
  // they reach only output columns that are never stored)
  const chunk_t* a_rows[S::A_LOADS];
  const chunk_t* b_rows[S::B_LOADS];
#pragma unroll
  for (int q = 0; q < S::A_LOADS; ++q)
    a_rows[q] = a + static_cast<size_t>(row_src[(wv * S::A_LOADS + q) * 8 + (lane >> 3)]) * kchunks;
#pragma unroll
  for (int q = 0; q < S::B_LOADS; ++q) {
    const int j = col0 + (wv * S::B_LOADS + q) * 8 + (lane >> 3);
    b_rows[q] = wx + static_cast<size_t>(j < n ? j : n - 1) * kchunks;
  }
  auto stage_a = [&](int buf) { return lds + buf * S::STAGE_BYTES + wv * S::A_LOADS * 1024; };
  auto stage_b = [&](int buf) {
    return lds + buf * S::STAGE_BYTES + S::BM * kRowBytes + wv * S::B_LOADS * 1024;
  };
  auto issue = [&](int kt, int buf) {
    const bool pa = stage_rows<S::A_LOADS>(a_rows, kt, c_lane, kchunks, stage_a(buf));
    stage_rows<S::B_LOADS>(b_rows, kt, c_lane, kchunks, stage_b(buf));
    return pa;  // A and B rows share the chunk schedule
  };
  auto land = [&](bool past, int buf) {
    __builtin_amdgcn_s_waitcnt(0);
    if (past) {
      clear_slots<S::A_LOADS>(stage_a(buf), lane);
      clear_slots<S::B_LOADS>(stage_b(buf), lane);
    }
    __syncthreads();
  };

  const int wm = wv >> 1, wn = wv & 1;  // this wave's quarter of the tile
  f32x16_t acc[S::FM][S::FN];
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int jj = 0; jj < S::FN; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.0f;

  // fragment addresses: row (lane % 32) of each 32-row MFMA tile, chunk 2 ks + lane / 32,
  // found at slot chunk ^ (row % 8) = chunk ^ (lane % 8)
  const int a_frag = (wm * WM + (lane & 31)) * kRowBytes;
  const int b_frag = S::BM * kRowBytes + (wn * WN + (lane & 31)) * kRowBytes;
  int slot_off[kGemmBK / 16];
#pragma unroll
  for (int ks = 0; ks < kGemmBK / 16; ++ks) slot_off[ks] = ((2 * ks + (lane >> 5)) ^ (lane & 7)) * 16;

  land(issue(0, 0), 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    bool past = false;
    if (kt + 1 < nk) past = issue(kt + 1, cur ^ 1);
    const char* st = lds + cur * S::STAGE_BYTES;
    chunk_t fa[2][S::FM], fb[2][S::FN];
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
      fa[0][i] = *reinterpret_cast<const chunk_t*>(st + a_frag + i * 32 * kRowBytes + slot_off[0]);
#pragma unroll
    for (int jj = 0; jj < S::FN; ++jj)
      fb[0][jj] = *reinterpret_cast<const chunk_t*>(st + b_frag + jj * 32 * kRowBytes + slot_off[0]);
#pragma unroll
    for (int ks = 0; ks < kGemmBK / 16; ++ks) {
      const int c = ks & 1;
      // this step's fragments have landed before the next step's reads are issued, so
      // at most one step's reads (FM + FN <= 8) are ever outstanding and the wait for a
      // step never covers the reads of the one after it
      __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < kGemmBK / 16) {  // next k16 step's fragments, read under this step's MFMAs
#pragma unroll
        for (int i = 0; i < S::FM; ++i)
          fa[c ^ 1][i] = *reinterpret_cast<const chunk_t*>(st + a_frag + i * 32 * kRowBytes + slot_off[ks + 1]);
#pragma unroll
        for (int jj = 0; jj < S::FN; ++jj)
          fb[c ^ 1][jj] = *reinterpret_cast<const chunk_t*>(st + b_frag + jj * 32 * kRowBytes + slot_off[ks + 1]);
      }
      // keep those reads ahead of this step's MFMAs (the scheduler would otherwise sink
      // each read next to its first use and stall on it)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < S::FN; ++jj) acc[i][jj] = mfma_32x32x16<DT>(fa[c][i], fb[c][jj], acc[i][jj]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 1 < nk) land(past, cur ^ 1);
  }

  // epilogue: optional route weight (weights after the experts), one narrowing
#pragma unroll
  for (int i = 0; i < S::FM; ++i) {
#pragma unroll
    for (int jj = 0; jj < S::FN; ++jj) {
      const int col = col0 + wn * WN + jj * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < nrows && col < n) {
          float f = acc[i][jj][v];
          if constexpr (SCALE) f = __fmul_rn(row_scale[row], f);
          out[static_cast<size_t>(row0 + row) * n + col] = narrow<DT>(f);
        }
      }
    }
  }
}

// Tile shape chosen per launch: 256 x 256 tiles when experts average at least 512 rows
// (fewer LDS reads per MFMA), else 128 x 256 (less padding in short segments).
constexpr int kTallWM = 128, kTallWN = 128;
constexpr int kShortWM = 64, kShortWN = 128;

static bool use_tall(const LayoutView& L) {
  return L.capacity > 0 ? L.capacity >= 512 : static_cast<int64_t>(L.s) * L.k >= 512LL * L.e;
}

// An upper bound on the row-blocks in use, known on the host without reading the layout.
static int64_t row_block_bound(const LayoutView& L, int BM) {
  if (L.capacity > 0) return static_cast<int64_t>(L.e) * ((L.capacity + BM - 1) / BM);
  return (static_cast<int64_t>(L.s) * L.k + BM - 1) / BM + L.e;
}

int64_t expert_gemm_grid(const LayoutView& L, int n) {
  if (L.s == 0) return 0;
  const int BM = use_tall(L) ? 2 * kTallWM : 2 * kShortWM;
  const int BN = use_tall(L) ? 2 * kTallWN : 2 * kShortWN;
  const int64_t col_blocks = (n + BN - 1) / BN;
  const int64_t tiles = row_block_bound(L, BM) * col_blocks;
  return (tiles + kXcds - 1) / kXcds * kXcds;
}

template <int DT, bool GATHER, bool SCALE, int WM, int WN>
static hipError_t gemm_launch(const LayoutView& L, const void* a, const void* w,
                              const float* route_w, int m, int n, void* out, hipStream_t stream) {
  using S = GemmShape<WM, WN>;
  auto kern = expert_gemm_kernel<DT, GATHER, SCALE, WM, WN>;
  // dynamic LDS above the 64 KiB default needs the per-kernel limit raised (idempotent)
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS_BYTES);
  if (err != hipSuccess) return err;
  const int64_t grid = expert_gemm_grid(L, n);
  if (grid == 0) return hipSuccess;
  const int col_blocks = (n + S::BN - 1) / S::BN;
  kern<<<static_cast<unsigned>(grid), kGemmThreads, S::LDS_BYTES, stream>>>(
      static_cast<const chunk_t*>(a), static_cast<const chunk_t*>(w), route_w, L.dst, L.src, L.kept,
      L.offsets, L.e, L.k, m, n, col_blocks, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

template <int DT, bool GATHER, bool SCALE>
static hipError_t gemm_shape(const LayoutView& L, const void* a, const void* w,
                             const float* route_w, int m, int n, void* out, hipStream_t stream) {
  if (use_tall(L))
    return gemm_launch<DT, GATHER, SCALE, kTallWM, kTallWN>(L, a, w, route_w, m, n, out, stream);
  return gemm_launch<DT, GATHER, SCALE, kShortWM, kShortWN>(L, a, w, route_w, m, n, out, stream);
}

template <int DT>
static hipError_t gemm_dt(const LayoutView& L, const void* a, bool gather, const void* w,
                          const float* route_w, int m, int n, void* out, hipStream_t stream) {
  if (gather) {
    if (route_w) return gemm_shape<DT, true, true>(L, a, w, route_w, m, n, out, stream);
    return gemm_shape<DT, true, false>(L, a, w, route_w, m, n, out, stream);
  }
  if (route_w) return gemm_shape<DT, false, true>(L, a, w, route_w, m, n, out, stream);
  return gemm_shape<DT, false, false>(L, a, w, route_w, m, n, out, stream);
}

hipError_t launch_expert_gemm(const LayoutView& L, const void* a, bool gather, const void* w,
                              const float* route_w, int m, int n, int dtype, void* out,
                              hipStream_t stream) {
  if (L.s > 0) {
    const hipError_t err = dtype == kBF16 ? gemm_dt<kBF16>(L, a, gather, w, route_w, m, n, out, stream)
                                          : gemm_dt<kF16>(L, a, gather, w, route_w, m, n, out, stream);
    if (err != hipSuccess) return err;
  }
  // rows no route fills are zero
  return launch_zero_unfilled_rows(L, out, static_cast<int64_t>(n) * 2 / 16, stream);
}

}  // namespace moe
