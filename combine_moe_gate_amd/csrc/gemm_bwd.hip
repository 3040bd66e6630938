// Weight gradient of the grouped expert GEMM, with the dispatch fused into its operand
// loads, on gfx950 matrix cores.
//
// The forward computes out[r] = A(r) @ W[x]^T for the placed rows r of expert x's
// segment [offsets[x], offsets[x] + kept[x]). Its weight gradient is
//     grad_W[x] = sum over those rows r of outer(grad_out[r], A(r))        [n, m]
// a GEMM whose reduction runs over the segment's rows. A(r) = x[src[r]] is gathered
// straight from the token rows again, so neither pass materialises the [rows, m] buffer
// (DeepSpeed PR "Add an opt-in DeepEP transport for the AutoEP expert all-to-all":
// review-fix commit, the groups are the prefix sum's segments; first commit, the
// backward replays the forward's grouping).
//
// The sums are float32; they are stored as float32 or rounded once to the element type
// (gradients kept in the weights' own type, at half the bytes written).
//
// Tiling: a workgroup of 8 waves (2 along m x 4 along n, each 128 x 64 as 4 x 2 MFMA
// tiles of 32 x 32 x 16) computes a 256 x 256 tile of grad_W[x], reducing over the
// segment 64 rows at a time. The token rows are the MFMA's first operand, so each lane's
// accumulator holds four consecutive m of one row of grad_W. Both operands are stored
// row by row, contiguous along n (grad_out) or m (the token rows), so a K step is staged
// in LDS exactly as it sits in memory, [64 rows][256 elements] with each row padded to
// 576 bytes, and the MFMA fragments (8 consecutive rows of one column per lane) are read
// with gfx950's transposing LDS read, ds_read_b64_tr_b16. Within each 16-lane group it
// hands lane i column i % 4 of the 4-element pieces the group's lanes point at, taken
// from lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12: with lane j pointing at row
// k0 + j / 4, columns c0 + 4 (j % 4) .. + 3, lane i receives rows k0 .. k0 + 3 of column
// c0 + i. Two such reads make one fragment. A 576-byte pitch (64 mod 256) puts the four
// rows one read touches, and the two 16-column halves of a 32-lane pass, on distinct
// banks. Staging goes through registers (16-byte loads, 16-byte LDS writes), so rows past
// the segment are written as zeros directly. Two stages: the next step's loads are in
// flight while the current one is multiplied; the row map src is fetched one step
// further ahead. The finished tile leaves through LDS as whole rows, and the next tile's
// first loads are issued before its stores.
//
// Schedule: one workgroup per CU loops over tiles. The tiles of the experts with rows are
// numbered expert by expert (inside an expert in bands of 4 n-blocks, m-block major), and
// each XCD takes one contiguous stretch of that order holding an equal share of the work
// (a tile costs its number of K steps plus a fixed overhead), so the tiles resident on an
// XCD at once share operand slabs through its L2 and every XCD finishes together. The
// tiles of experts without rows only write zeros; they are split evenly over the XCDs
// and each CU interleaves its share between its multiplying tiles, so that the zero
// writes spread over every XCD's path to memory and over the whole run.
#include "gemm_common.h"
#include "internal.h"
#include "moe_device.h"

namespace moe {

constexpr int kWgTileN = 256, kWgTileM = 256;  // tile of grad_W: rows (n) x columns (m)
constexpr int kWgBK = 64;                // segment rows per K step
constexpr int kWgWM = 128, kWgWN = 64;   // per wave: along m (MFMA rows) x along n
constexpr int kWgThreads = 512;          // 8 waves: 2 along m x 4 along n
constexpr int kWgPitch = kWgTileM * 2 + 64; // bytes per staged row: 512 + 64 (64 mod 256)
constexpr int kWgOperandBytes = kWgBK * kWgPitch;
constexpr int kWgStageBytes = 2 * kWgOperandBytes;  // grad_out rows, then token rows
constexpr int kWgLdsBytes = 2 * kWgStageBytes;      // two stages: 147456 bytes
constexpr int kWgChunks = kWgBK * (kWgTileM / 8) / kWgThreads;  // 16-byte chunks per thread per operand
constexpr int kWgBandN = 4;              // n-blocks per band of the tile order
constexpr int kWgTileOverhead = 4;       // a tile's fixed cost, in K steps

static_assert(kWgTileM == kWgTileN, "both operands stage rows of the same width");
static_assert(kWgChunks == 4, "staging split");

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 read_tr(const char* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

struct WgTiles {
  int expert, nb, mb, nk;  // expert (-1: none), n-block, m-block, K steps
};

// The j-th expert, in expert order, among those with rows (with_rows) or without (-1 if
// there are fewer). Every lane of the wave calls it with the same arguments.
__device__ __forceinline__ int wg_nth_expert(int j, bool with_rows, const int32_t* __restrict__ kept, int e) {
  const int lane = lane_id();
  for (int c0 = 0; c0 < e; c0 += kWave) {
    const int x = c0 + lane;
    const bool hit = x < e && ((kept[x] > 0) == with_rows);
    const uint64_t b = __ballot(hit);
    const int cnt = __popcll(b);
    if (j < cnt) {
      const int below = __popcll(b & ((1ull << lane) - 1ull));
      return c0 + static_cast<int>(__builtin_ctzll(__ballot(hit && below == j)));
    }
    j -= cnt;
  }
  return -1;
}

// Tile t of the order of the experts with rows (with_rows) or of those without: each
// expert owns tiles_per_expert consecutive tiles; inside an expert, bands of kWgBandN
// n-blocks, m-block major, n-block fastest. nk = -1: no such tile.
__device__ __forceinline__ WgTiles wg_tile_of(int64_t t, bool with_rows, const int32_t* __restrict__ kept,
                                              int e, int tiles_per_expert, int n_blocks, int m_blocks) {
  WgTiles tc;
  const int jx = static_cast<int>(t / tiles_per_expert);
  tc.expert = wg_nth_expert(jx, with_rows, kept, e);
  const int u = static_cast<int>(t - static_cast<int64_t>(jx) * tiles_per_expert);
  const int band = u / (kWgBandN * m_blocks);
  const int left = n_blocks - band * kWgBandN;
  const int in_band = left < kWgBandN ? left : kWgBandN;
  const int v = u - band * kWgBandN * m_blocks;
  tc.mb = v / in_band;
  tc.nb = band * kWgBandN + v % in_band;
  tc.nk = tc.expert < 0 ? -1 : with_rows ? (kept[tc.expert] + kWgBK - 1) / kWgBK : 0;
  return tc;
}

// Inclusive wave scan of a non-negative 64-bit value, and its wave total.
__device__ __forceinline__ int64_t wave_inclusive_scan64(int64_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t y = __shfl_up(v, o, kWave);
    if (lane >= o) v += y;
  }
  return v;
}

// Tiles and work of expert x in the order of the experts with rows (lanes past e, and
// experts without rows: none): tiles_per_expert tiles, each costing its K steps plus a
// fixed overhead (the tile's store).
__device__ __forceinline__ void wg_expert_work(bool valid, int kx, int tiles_per_expert,
                                               int64_t* tiles, int64_t* per_tile) {
  const bool real = valid && kx > 0;
  *tiles = real ? tiles_per_expert : 0;
  *per_tile = real ? (kx + kWgBK - 1) / kWgBK + kWgTileOverhead : 0;
}

// First tile (in the order of the experts with rows) of XCD i's stretch: the first tile
// whose work starts at or after i / 8 of the total (uniform across the wave).
__device__ __forceinline__ int64_t wg_stretch_start(int i, int e, const int32_t* __restrict__ kept,
                                                    int tiles_per_expert) {
  const int lane = lane_id();
  int64_t total_cost = 0, total_tiles = 0;
  for (int c0 = 0; c0 < e; c0 += kWave) {
    const int x = c0 + lane;
    int64_t tiles, per;
    wg_expert_work(x < e, x < e ? kept[x] : 0, tiles_per_expert, &tiles, &per);
    total_cost += __shfl(wave_inclusive_scan64(tiles * per), kWave - 1, kWave);
    total_tiles += __shfl(wave_inclusive_scan64(tiles), kWave - 1, kWave);
  }
  if (i <= 0) return 0;
  if (i >= kXcds) return total_tiles;
  const int64_t target = (total_cost * i + kXcds - 1) / kXcds;
  int64_t cost_before = 0, tiles_before = 0;
  for (int c0 = 0; c0 < e; c0 += kWave) {
    const int x = c0 + lane;
    int64_t tiles, per;
    wg_expert_work(x < e, x < e ? kept[x] : 0, tiles_per_expert, &tiles, &per);
    const int64_t cost_incl = wave_inclusive_scan64(tiles * per);
    const int64_t tiles_incl = wave_inclusive_scan64(tiles);
    const int64_t lo = cost_before + cost_incl - tiles * per, hi = cost_before + cost_incl;
    const uint64_t hit = __ballot(tiles > 0 && target >= lo && target < hi);
    if (hit != 0ull) {
      const int owner = static_cast<int>(__builtin_ctzll(hit));
      const int64_t o_lo = __shfl(lo, owner, kWave), o_per = __shfl(per, owner, kWave);
      const int64_t o_first = tiles_before + __shfl(tiles_incl - tiles, owner, kWave);
      return o_first + (target - o_lo + o_per - 1) / o_per;
    }
    cost_before += __shfl(cost_incl, kWave - 1, kWave);
    tiles_before += __shfl(tiles_incl, kWave - 1, kWave);
  }
  return total_tiles;
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Output staging for the store: the finished tile passes through LDS so that it leaves
// as whole rows (16 bytes per lane, consecutive lanes on consecutive addresses). Stored
// straight from the MFMA accumulators, each instruction would write 32-byte pieces of 32
// different rows, which reaches HBM at about half the rate of whole lines. Float32 goes
// in two passes of 128 columns, 16-bit types in one; a staged row is 512 bytes, padded
// to 528 (16 mod 256) so the 16 rows one 16-byte LDS write touches hit distinct banks.
constexpr int kEpPitch = 512 + 16;
static_assert(256 * kEpPitch <= kWgLdsBytes, "output staging fits in the operand stages");

// Four consecutive gradients of one row: 16 bytes of float32, or 8 bytes rounded to the
// element type OUT.
template <int OUT>
__device__ __forceinline__ void put_row4(char* p, float v0, float v1, float v2, float v3) {
  if constexpr (OUT == kF32) {
    *reinterpret_cast<chunk_t*>(p) =
        chunk_t{__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3)};
  } else if constexpr (OUT == kBF16) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{f32x2_to_bf16x2_rne(v0, v1), f32x2_to_bf16x2_rne(v2, v3)};
  } else {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{f32_to_f16_rne(v0) | (f32_to_f16_rne(v1) << 16),
                                             f32_to_f16_rne(v2) | (f32_to_f16_rne(v3) << 16)};
  }
}

template <int DT, bool GATHER, int OUT>
__global__ __launch_bounds__(kWgThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void expert_gemm_wgrad_kernel(const chunk_t* __restrict__ a, const chunk_t* __restrict__ g,
                              const int32_t* __restrict__ src, const int32_t* __restrict__ kept,
                              const int32_t* __restrict__ offsets, int e, int m, int n,
                              void* __restrict__ gw) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];  // [2 stages][grad_out, rows][64][576 B]
  __shared__ int64_t stretch[4];  // this XCD's tiles with rows [0], [1]; zero tiles [2], [3]
  constexpr int kOutBytes = OUT == kF32 ? 4 : 2;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = wave_in_block();
  const int m_chunks = m / 8, n_chunks = n / 8;
  const int n_blocks = (n + kWgTileN - 1) / kWgTileN, m_blocks = (m + kWgTileM - 1) / kWgTileM;
  const int tiles_per_expert = n_blocks * m_blocks;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds, slots = gridDim.x / kXcds;

  if (wv == 0) {
    const int64_t t0 = wg_stretch_start(xcd, e, kept, tiles_per_expert);
    const int64_t t1 = wg_stretch_start(xcd + 1, e, kept, tiles_per_expert);
    int idle = 0;
    for (int c0 = 0; c0 < e; c0 += kWave) idle += __popcll(__ballot(c0 + lane < e && kept[c0 + lane] == 0));
    const int64_t zt = static_cast<int64_t>(idle) * tiles_per_expert;
    if (lane == 0) {
      stretch[0] = t0;
      stretch[1] = t1;
      stretch[2] = zt * xcd / kXcds;
      stretch[3] = zt * (xcd + 1) / kXcds;
    }
  }
  __syncthreads();
  // this CU's items: tiles with rows r0 + slot + i slots (i < n_real), zero tiles
  // z0 + slot + i slots (i < n_zero), interleaved in proportion
  const int64_t r0 = stretch[0], z0 = stretch[2];
  const int n_real = stretch[1] - r0 > slot ? static_cast<int>((stretch[1] - r0 - slot + slots - 1) / slots) : 0;
  const int n_zero = stretch[3] - z0 > slot ? static_cast<int>((stretch[3] - z0 - slot + slots - 1) / slots) : 0;
  auto item = [&](int ri, int zi) -> WgTiles {  // the item after ri tiles with rows and zi zero tiles
    if (ri < n_real && (zi >= n_zero || static_cast<int64_t>(ri) * n_zero <= static_cast<int64_t>(zi) * n_real))
      return wg_tile_of(r0 + slot + static_cast<int64_t>(ri) * slots, true, kept, e, tiles_per_expert,
                        n_blocks, m_blocks);
    if (zi < n_zero)
      return wg_tile_of(z0 + slot + static_cast<int64_t>(zi) * slots, false, kept, e, tiles_per_expert,
                        n_blocks, m_blocks);
    return WgTiles{-1, 0, 0, -1};
  };

  // staging: thread tid moves chunk (tid % 32) of rows tid / 32 + 16 h, h = 0..3
  const int s_chunk = tid % 32, s_row = tid / 32;
  // transposing fragment reads: lane j of 16-lane group q points at row 8 (q / 2) + j / 4,
  // columns 16 (q % 2) + 4 (j % 4) .. + 3 of each 32-wide MFMA tile
  const int q = lane >> 4, j = lane & 15;
  const int frag_off = (8 * (q >> 1) + (j >> 2)) * kWgPitch + (16 * (q & 1) + 4 * (j & 3)) * 2;
  const int wave_m = wv >> 2, wave_n = wv & 3;  // this wave's 128 (m) x 64 (n) part of the tile

  // Operand state of the tile whose first step sits in the staging registers.
  int seg0 = 0, rows_x = 0, nc = 0, mc = 0;
  chunk_t rg[kWgChunks], ra[kWgChunks];
  int rsrc[kWgChunks];  // token rows of the next step to load
  auto begin = [&](const WgTiles& tc) {
    seg0 = offsets[tc.expert];
    rows_x = kept[tc.expert];
    // column chunks this thread stages (past n / m: the last chunk, never stored)
    const int n_c = tc.nb * (kWgTileN / 8) + s_chunk, m_c = tc.mb * (kWgTileM / 8) + s_chunk;
    nc = n_c < n_chunks ? n_c : n_chunks - 1;
    mc = m_c < m_chunks ? m_c : m_chunks - 1;
  };
  auto fetch_src = [&](int kt) {
#pragma unroll
    for (int h = 0; h < kWgChunks; ++h) {
      const int i = kt * kWgBK + s_row + 16 * h;
      rsrc[h] = i < rows_x ? (GATHER ? src[seg0 + i] : seg0 + i) : -1;
    }
  };
  auto issue = [&](int kt) {
    const chunk_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < kWgChunks; ++h) {
      const int i = kt * kWgBK + s_row + 16 * h;
      const bool in = i < rows_x;
      rg[h] = in ? g[static_cast<size_t>(seg0 + i) * n_chunks + nc] : zero;
      ra[h] = rsrc[h] >= 0 ? a[static_cast<size_t>(rsrc[h]) * m_chunks + mc] : zero;
    }
  };
  auto publish = [&](int kt) {
    char* st = lds + (kt & 1) * kWgStageBytes;
#pragma unroll
    for (int h = 0; h < kWgChunks; ++h) {
      const int off = (s_row + 16 * h) * kWgPitch + s_chunk * 16;
      *reinterpret_cast<chunk_t*>(st + off) = rg[h];
      *reinterpret_cast<chunk_t*>(st + kWgOperandBytes + off) = ra[h];
    }
    __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
    stage_barrier();
  };

  chunk_t fa[2][4], fb[2][2];
  auto read_frags = [&](int kt, int ks, int fbuf) {
    const char* st = lds + (kt & 1) * kWgStageBytes + frag_off + ks * 16 * kWgPitch;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* p = st + kWgOperandBytes + (wave_m * kWgWM + i * 32) * 2;
      const uint2 lo = read_tr(p), hi = read_tr(p + 4 * kWgPitch);
      fa[fbuf][i] = chunk_t{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const char* p = st + (wave_n * kWgWN + jj * 32) * 2;
      const uint2 lo = read_tr(p), hi = read_tr(p + 4 * kWgPitch);
      fb[fbuf][jj] = chunk_t{lo.x, lo.y, hi.x, hi.y};
    }
  };

  int n_done_real = 0, n_done_zero = 0;
  WgTiles cur = item(0, 0);
  if (cur.nk > 0) {
    begin(cur);
    fetch_src(0);
    issue(0);
    if (cur.nk > 1) fetch_src(1);
  }
  while (cur.nk >= 0) {
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.0f;

    const int nk = cur.nk;
    if (nk > 0) {
      stage_barrier();  // every wave has read the previous tile's last stage
      publish(0);
      read_frags(0, 0, 0);
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) {
          issue(kt + 1);
          if (kt + 2 < nk) fetch_src(kt + 2);
        }
#pragma unroll
        for (int ks = 0; ks < kWgBK / 16; ++ks) {
          __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);  // this k16 step's fragments have landed
          __builtin_amdgcn_sched_barrier(0);
          if (ks + 1 < kWgBK / 16) {
            read_frags(kt, ks + 1, (ks + 1) & 1);
          } else if (kt + 1 < nk) {
            publish(kt + 1);  // step kt's buffer was read out before this barrier
            __builtin_amdgcn_sched_barrier(0);
            read_frags(kt + 1, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
              acc[i][jj] = mfma_32x32x16<DT>(fa[ks & 1][i], fb[ks & 1][jj], acc[i][jj]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // The next tile's first step goes out before this tile's global stores, so its
    // loads are not queued behind them (and, for a tile with rows, after the first
    // output pass has left the accumulators for LDS, which frees their registers).
    const int x = cur.expert;
    const int n0 = cur.nb * kWgTileN, m0 = cur.mb * kWgTileM;
    if (nk > 0) ++n_done_real;
    else ++n_done_zero;
    cur = item(n_done_real, n_done_zero);
    auto prefetch_next = [&]() {
      if (cur.nk > 0) {
        begin(cur);
        fetch_src(0);
        issue(0);
        if (cur.nk > 1) fetch_src(1);
      }
    };

    char* gx = static_cast<char*>(gw) + static_cast<size_t>(x) * n * m * kOutBytes;
    if (nk > 0) {
      // lane l holds, for MFMA tile (i, jj), grad_W row n = l % 32 of the tile's 32 x 32
      // block and its columns m 8 (v / 4) + 4 (l / 32) + v % 4: four consecutive m per
      // value group. Pass p stages MFMA row tiles i of [kEpI p, kEpI (p + 1)) of both
      // waves along m: staged column c is tile column (c / kEpSeg) 128 + p kEpSeg + c % kEpSeg.
      constexpr int kEpPasses = OUT == kF32 ? 2 : 1;
      constexpr int kEpI = 4 / kEpPasses;
      constexpr int kEpSeg = kEpI * 32;
      constexpr int kPerChunk = 16 / kOutBytes;
#pragma unroll
      for (int p = 0; p < kEpPasses; ++p) {
        stage_barrier();  // every wave is done with the LDS (operand stages or the previous pass)
#pragma unroll
        for (int ii = 0; ii < kEpI; ++ii) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int r = wave_n * kWgWN + jj * 32 + (lane & 31);
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
              const int c = wave_m * kEpSeg + ii * 32 + 8 * v4 + 4 * (lane >> 5);
              const f32x16_t& av = acc[p * kEpI + ii][jj];
              put_row4<OUT>(lds + r * kEpPitch + c * kOutBytes, av[4 * v4], av[4 * v4 + 1], av[4 * v4 + 2],
                            av[4 * v4 + 3]);
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
        stage_barrier();
        if (p == 0) prefetch_next();
        // thread tid moves 16-byte chunk tid % 32 of staged rows tid / 32 + 16 h
        const int r0 = tid >> 5, c = (tid & 31) * kPerChunk;
        const int col = m0 + (c / kEpSeg) * kWgWM + p * kEpSeg + c % kEpSeg;
        const char* lp = lds + r0 * kEpPitch + (tid & 31) * 16;
        char* gp = gx + (static_cast<size_t>(n0 + r0) * m + col) * kOutBytes;
        const size_t g_step = static_cast<size_t>(16) * m * kOutBytes;
        const int rows_left = n - n0 - r0;  // staged rows past n are not stored
#pragma unroll 4
        for (int h = 0; h < 256 / 16; ++h) {
          const chunk_t v = *reinterpret_cast<const chunk_t*>(lp + h * 16 * kEpPitch);
          if (col < m && 16 * h < rows_left) *reinterpret_cast<chunk_t*>(gp + h * g_step) = v;
        }
      }
    } else {  // an expert without rows: its gradient is zero
      prefetch_next();
      constexpr int kPerChunk = 16 / kOutBytes;  // elements per 16-byte store
      constexpr int kRowChunks = kWgTileM / kPerChunk;
      const chunk_t z = {0u, 0u, 0u, 0u};
      const int nrow = n - n0 < kWgTileN ? n - n0 : kWgTileN;
      const int ncol = m - m0 < kWgTileM ? m - m0 : kWgTileM;  // a multiple of 8
      for (int c = tid; c < nrow * kRowChunks; c += kWgThreads) {
        const int r = c / kRowChunks, col = (c % kRowChunks) * kPerChunk;
        if (col < ncol)
          __builtin_nontemporal_store(
              z, reinterpret_cast<chunk_t*>(gx + (static_cast<size_t>(n0 + r) * m + m0 + col) * kOutBytes));
      }
    }
  }
}

// Workgroups of the weight-gradient kernel: one per CU, a multiple of the XCD count.
static int wgrad_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < kXcds)
    cus = 256;
  return cus / kXcds * kXcds;
}

template <int DT, bool GATHER, int OUT>
static hipError_t wgrad_launch(const LayoutView& L, const void* a, const void* grad_out, int m,
                               int n, void* gw, hipStream_t stream) {
  auto kern = expert_gemm_wgrad_kernel<DT, GATHER, OUT>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kWgLdsBytes);
  if (err != hipSuccess) return err;
  kern<<<wgrad_grid(), kWgThreads, kWgLdsBytes, stream>>>(
      static_cast<const chunk_t*>(a), static_cast<const chunk_t*>(grad_out), L.src, L.kept,
      L.offsets, L.e, m, n, gw);
  return hipGetLastError();
}

template <int DT, int OUT>
static hipError_t wgrad_launch(const LayoutView& L, const void* a, bool gather, const void* grad_out,
                               int m, int n, void* gw, hipStream_t stream) {
  return gather ? wgrad_launch<DT, true, OUT>(L, a, grad_out, m, n, gw, stream)
                : wgrad_launch<DT, false, OUT>(L, a, grad_out, m, n, gw, stream);
}

hipError_t launch_expert_gemm_wgrad(const LayoutView& L, const void* a, bool gather,
                                    const void* grad_out, int m, int n, int dtype, bool out_f32,
                                    void* gw, hipStream_t stream) {
  if (dtype == kBF16)
    return out_f32 ? wgrad_launch<kBF16, kF32>(L, a, gather, grad_out, m, n, gw, stream)
                   : wgrad_launch<kBF16, kBF16>(L, a, gather, grad_out, m, n, gw, stream);
  return out_f32 ? wgrad_launch<kF16, kF32>(L, a, gather, grad_out, m, n, gw, stream)
                 : wgrad_launch<kF16, kF16>(L, a, gather, grad_out, m, n, gw, stream);
}

}  // namespace moe
