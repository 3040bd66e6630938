// Dispatch layout on gfx950: per-expert counts, token-order slots, capacity drop, and
// the route -> row (dst) and row -> token (src) maps.
//
// The slot of a route is the column cumsum of the token x expert mask minus one
// (DeepSpeed PR "MoE dispatch: fix silent Tutel + TP corruption, speed up native and
// Tutel paths", review comment on fast_cumsum_sub_one), i.e. the number of earlier
// tokens that chose the same expert. It is computed without sorting and without any
// order-dependent atomics, in three launches:
//
//   count  one workgroup per tile of 256 tokens: LDS histogram of the tile's valid
//          routes (integer atomic adds; the totals do not depend on their order), the
//          tile's share of the routing checksum and its flag bits.
//   scan   one workgroup: for every expert an exclusive scan over tiles (in place: the
//          tile counts become tile bases), the totals, kept = min(count, capacity), and
//          an exclusive scan over experts of the segment sizes (the dropless offsets;
//          with a capacity the segments are all `capacity` rows long).
//   place  one workgroup per tile again: each wave builds, per expert, a 64-bit mask
//          of its lanes (tokens) that chose it (LDS atomic OR: order-independent). The
//          slot of a route is then tile base + popcounts of the earlier waves' masks +
//          popcount of its own wave's mask below its lane. Writes dst, src and a copy
//          of the routing; rows no route fills get src = -1.
#include "internal.h"
#include "moe_device.h"

namespace moe {

// Load a token's k expert ids and decide which routes are valid: in [0, e) and not a
// repeat of an earlier route of the same token. Returns the flag bits raised.
template <int KMAX>
__device__ __forceinline__ int load_routes(const int32_t* __restrict__ idx, int t, int k, int e,
                                           int (&ids)[KMAX], bool (&ok)[KMAX]) {
  int flags = 0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) ids[j] = (j < k) ? idx[static_cast<size_t>(t) * k + j] : -1;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ok[j] = false;
    if (j < k) {
      const bool in_range = static_cast<unsigned>(ids[j]) < static_cast<unsigned>(e);
      bool dup = false;
#pragma unroll
      for (int q = 0; q < j; ++q) dup |= (ids[q] == ids[j]);
      if (!in_range) flags |= 1;
      else if (dup) flags |= 2;
      ok[j] = in_range && !dup;
    }
  }
  return flags;
}

template <int KMAX>
__global__ __launch_bounds__(kTileTokens) void layout_count_kernel(
    const int32_t* __restrict__ idx, int s, int e, int k, int32_t* __restrict__ tile_counts,
    uint64_t* __restrict__ tile_checksum, int32_t* __restrict__ tile_flags) {
  extern __shared__ int32_t hist[];  // [e]
  __shared__ uint64_t part_sum[kTileTokens / kWave];
  __shared__ int32_t part_flags[kTileTokens / kWave];
  for (int i = threadIdx.x; i < e; i += kTileTokens) hist[i] = 0;
  __syncthreads();

  const int t = blockIdx.x * kTileTokens + threadIdx.x;
  uint64_t cks = 0;
  int flags = 0;
  if (t < s) {
    int ids[KMAX];
    bool ok[KMAX];
    flags = load_routes<KMAX>(idx, t, k, e, ids, ok);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const uint64_t pos = static_cast<uint64_t>(t) * k + j + 1;
        cks += static_cast<uint64_t>(static_cast<int64_t>(ids[j]) + 1) * pos;
        if (ok[j]) atomicAdd(&hist[ids[j]], 1);
      }
    }
  }
  cks = wave_sum(cks);
  flags = wave_or(flags);
  if (lane_id() == 0) {
    part_sum[threadIdx.x >> 6] = cks;
    part_flags[threadIdx.x >> 6] = flags;
  }
  __syncthreads();
  int32_t* out = tile_counts + static_cast<size_t>(blockIdx.x) * e;
  for (int i = threadIdx.x; i < e; i += kTileTokens) out[i] = hist[i];
  if (threadIdx.x == 0) {
    uint64_t c = 0;
    int f = 0;
#pragma unroll
    for (int w = 0; w < kTileTokens / kWave; ++w) {
      c += part_sum[w];
      f |= part_flags[w];
    }
    tile_checksum[blockIdx.x] = c;
    tile_flags[blockIdx.x] = f;
  }
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(
    int e, int capacity, int ntiles, int32_t* __restrict__ tile_counts,
    const uint64_t* __restrict__ tile_checksum, const int32_t* __restrict__ tile_flags,
    int32_t* __restrict__ counts, int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
    uint64_t* __restrict__ checksum, int32_t* __restrict__ flags) {
  __shared__ int32_t wave_total[kScanThreads / kWave];
  __shared__ uint64_t wave_cks[kScanThreads / kWave];
  __shared__ int32_t wave_flags[kScanThreads / kWave];
  const int x = threadIdx.x;
  const int lane = lane_id(), wv = threadIdx.x >> 6;

  // per expert: exclusive scan over tiles, in place
  int32_t total = 0;
  if (x < e) {
    int32_t* col = tile_counts + x;
    int b = 0;
    for (; b + 4 <= ntiles; b += 4) {
      const int32_t c0 = col[static_cast<size_t>(b) * e], c1 = col[static_cast<size_t>(b + 1) * e];
      const int32_t c2 = col[static_cast<size_t>(b + 2) * e], c3 = col[static_cast<size_t>(b + 3) * e];
      col[static_cast<size_t>(b) * e] = total;
      col[static_cast<size_t>(b + 1) * e] = total + c0;
      col[static_cast<size_t>(b + 2) * e] = total + c0 + c1;
      col[static_cast<size_t>(b + 3) * e] = total + c0 + c1 + c2;
      total += c0 + c1 + c2 + c3;
    }
    for (; b < ntiles; ++b) {
      const int32_t c = col[static_cast<size_t>(b) * e];
      col[static_cast<size_t>(b) * e] = total;
      total += c;
    }
    counts[x] = total;
    kept[x] = capacity > 0 ? (total < capacity ? total : capacity) : total;
  }

  // exclusive scan over experts of the segment sizes
  int32_t seg = (x < e) ? (capacity > 0 ? capacity : total) : 0;
  int32_t incl = seg;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wave_total[wv] = incl;

  // routing checksum and flags over tiles
  uint64_t c = 0;
  int f = 0;
  for (int b = x; b < ntiles; b += kScanThreads) {
    c += tile_checksum[b];
    f |= tile_flags[b];
  }
  c = wave_sum(c);
  f = wave_or(f);
  if (lane == 0) {
    wave_cks[wv] = c;
    wave_flags[wv] = f;
  }
  __syncthreads();

  int32_t before = 0;
  for (int w = 0; w < wv; ++w) before += wave_total[w];
  if (x < e) {
    offsets[x] = before + incl - seg;
    if (x == e - 1) offsets[e] = before + incl;
  }
  if (x == 0) {
    uint64_t cc = 0;
    int ff = 0;
    for (int w = 0; w < kScanThreads / kWave; ++w) {
      cc += wave_cks[w];
      ff |= wave_flags[w];
    }
    *checksum = cc;
    *flags = ff;
  }
}

template <int KMAX>
__global__ __launch_bounds__(kTileTokens) void layout_place_kernel(
    const int32_t* __restrict__ idx, int s, int e, int k, int capacity, int32_t rows,
    const int32_t* __restrict__ tile_base, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ dst, int32_t* __restrict__ src,
    int32_t* __restrict__ route_idx) {
  extern __shared__ unsigned long long lane_masks[];  // [waves per tile][e]
  constexpr int kWaves = kTileTokens / kWave;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int tile = blockIdx.x;

  if (tile * kTileTokens < s) {  // uniform per workgroup
    for (int i = threadIdx.x; i < kWaves * e; i += kTileTokens) lane_masks[i] = 0ull;
    __syncthreads();

    const int t = tile * kTileTokens + threadIdx.x;
    int ids[KMAX];
    bool ok[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      ids[j] = -1;
      ok[j] = false;
    }
    if (t < s) {
      load_routes<KMAX>(idx, t, k, e, ids, ok);
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (ok[j]) atomicOr(&lane_masks[wv * e + ids[j]], 1ull << lane);
    }
    __syncthreads();

    if (t < s) {
      const unsigned long long below = (1ull << lane) - 1ull;
      const int32_t* base = tile_base + static_cast<size_t>(tile) * e;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          int d = -1;
          if (ok[j]) {
            const int x = ids[j];
            int r = base[x];
            for (int w = 0; w < wv; ++w) r += __popcll(lane_masks[w * e + x]);
            r += __popcll(lane_masks[wv * e + x] & below);
            if (capacity > 0)
              d = r < capacity ? x * capacity + r : -1;
            else
              d = offsets[x] + r;
          }
          const size_t o = static_cast<size_t>(t) * k + j;
          dst[o] = d;
          route_idx[o] = ids[j];
          if (d >= 0) src[d] = t;
        }
      }
    }
  }

  // rows no route fills: the tail of each capacity segment, or the dropless rows past
  // the last valid route
  const int32_t begin = capacity > 0 ? 0 : offsets[e];
  const int32_t stride = gridDim.x * kTileTokens;
  for (int32_t r = begin + blockIdx.x * kTileTokens + threadIdx.x; r < rows; r += stride) {
    if (capacity > 0) {
      const int32_t x = r / capacity;
      if (r - x * capacity >= kept[x]) src[r] = -1;
    } else {
      src[r] = -1;
    }
  }
}

template <int KMAX>
static hipError_t launch_layout_k(const int32_t* idx, const LayoutView& L, hipStream_t stream) {
  const int ntiles = L.ntiles;
  if (ntiles > 0) {
    layout_count_kernel<KMAX><<<ntiles, kTileTokens, L.e * sizeof(int32_t), stream>>>(
        idx, L.s, L.e, L.k, L.tile_counts, L.tile_checksum, L.tile_flags);
  }
  layout_scan_kernel<<<1, kScanThreads, 0, stream>>>(L.e, L.capacity, ntiles, L.tile_counts,
                                                     L.tile_checksum, L.tile_flags, L.counts,
                                                     L.kept, L.offsets, L.checksum, L.flags);
  int grid = ntiles;
  if (L.capacity > 0) {
    const int64_t pad_blocks = (L.rows + kTileTokens - 1) / kTileTokens;
    const int64_t want = pad_blocks < 1024 ? pad_blocks : 1024;
    if (grid < want) grid = static_cast<int>(want);
  }
  if (grid < 1) grid = 1;
  const size_t lds = static_cast<size_t>(kTileTokens / kWave) * L.e * sizeof(unsigned long long);
  layout_place_kernel<KMAX><<<grid, kTileTokens, lds, stream>>>(
      idx, L.s, L.e, L.k, L.capacity, static_cast<int32_t>(L.rows), L.tile_counts, L.kept,
      L.offsets, L.dst, L.src, L.route_idx);
  return hipGetLastError();
}

hipError_t launch_layout(const int32_t* idx, const LayoutView& L, hipStream_t stream) {
  switch (route_bound(L.k)) {
    case 1: return launch_layout_k<1>(idx, L, stream);
    case 2: return launch_layout_k<2>(idx, L, stream);
    case 4: return launch_layout_k<4>(idx, L, stream);
    case 8: return launch_layout_k<8>(idx, L, stream);
    default: return launch_layout_k<16>(idx, L, stream);
  }
}

}  // namespace moe
