// Dispatch layout on gfx950: per-expert counts, token-order slots, capacity drop, and
// the route -> row (dst) and row -> token (src) maps.
//
// The slot of a route is the column cumsum of the token x expert mask minus one
// (DeepSpeed PR "MoE dispatch: fix silent Tutel + TP corruption, speed up native and
// Tutel paths", review comment on fast_cumsum_sub_one), i.e. the number of earlier
// tokens that chose the same expert. It is computed without sorting and without any
// order-dependent atomics, in two launches over tiles of 256 tokens:
//
//   count  one workgroup per tile: LDS histogram of the tile's valid routes (integer
//          atomic adds; the totals do not depend on their order), the tile's share of
//          the routing checksum and its flag bits.
//   place  one workgroup per tile again. Each workgroup first derives what it needs
//          from the small, L2-resident tile tables: for every expert the sum over
//          earlier tiles (its tile base) and over all tiles (the count), then an
//          exclusive scan over experts of the segment sizes (the dropless offsets; with
//          a capacity every segment is `capacity` rows). Workgroup 0 publishes counts,
//          kept, offsets, checksum and flags. Then each wave builds, per expert, a
//          64-bit mask of its lanes (tokens) that chose it (LDS atomic OR: order-
//          independent); a route's slot is tile base + popcounts of the earlier waves'
//          masks + popcount of its own wave's mask below its lane. It writes dst, src
//          and a copy of the routing; rows no route fills get src = -1.
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

// Exclusive scan of one int per expert across the workgroup (e <= 1024 experts, each
// thread owning up to four consecutive experts). Returns the total.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t* __restrict__ vals, int e,
                                                        int32_t* __restrict__ wave_tot) {
  constexpr int kPer = 4;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int first = threadIdx.x * kPer;
  int32_t mine[kPer];
  int32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    mine[i] = (first + i < e) ? vals[first + i] : 0;
    sum += mine[i];
  }
  int32_t incl = sum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  int32_t before = 0, total = 0;
  for (int w = 0; w < kTileTokens / kWave; ++w) {
    if (w < wv) before += wave_tot[w];
    total += wave_tot[w];
  }
  int32_t run = before + incl - sum;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (first + i < e) vals[first + i] = run;
    run += mine[i];
  }
  __syncthreads();
  return total;
}

template <int KMAX>
__global__ __launch_bounds__(kTileTokens) void layout_place_kernel(
    const int32_t* __restrict__ idx, int s, int e, int k, int capacity, int32_t rows, int ntiles,
    const int32_t* __restrict__ tile_counts, const uint64_t* __restrict__ tile_checksum,
    const int32_t* __restrict__ tile_flags, int32_t* __restrict__ counts,
    int32_t* __restrict__ kept_out, int32_t* __restrict__ offsets_out, uint64_t* __restrict__ checksum,
    int32_t* __restrict__ flags, int32_t* __restrict__ dst, int32_t* __restrict__ src,
    int32_t* __restrict__ route_idx) {
  // LDS: per expert tile base, total and segment offset, then the per-wave lane masks
  extern __shared__ unsigned long long lds[];
  constexpr int kWaves = kTileTokens / kWave;
  __shared__ int32_t wave_tot[kWaves];
  __shared__ uint64_t wave_cks[kWaves];
  __shared__ int32_t wave_flg[kWaves];
  unsigned long long* lane_masks = lds;                                   // [kWaves][e]
  int32_t* base_s = reinterpret_cast<int32_t*>(lds + kWaves * e);          // [e]
  int32_t* total_s = base_s + e;                                           // [e]
  int32_t* off_s = total_s + e;                                            // [e + 1]
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int my_tile = tile < ntiles ? tile : ntiles;  // workgroups past the tiles: pad only

  // per expert: sum over earlier tiles and over all tiles
  for (int x = threadIdx.x; x < e; x += kTileTokens) {
    int32_t before = 0, all = 0;
    int b = 0;
    for (; b + 4 <= ntiles; b += 4) {
      const int32_t c0 = tile_counts[static_cast<size_t>(b) * e + x];
      const int32_t c1 = tile_counts[static_cast<size_t>(b + 1) * e + x];
      const int32_t c2 = tile_counts[static_cast<size_t>(b + 2) * e + x];
      const int32_t c3 = tile_counts[static_cast<size_t>(b + 3) * e + x];
      before += (b < my_tile ? c0 : 0) + (b + 1 < my_tile ? c1 : 0) + (b + 2 < my_tile ? c2 : 0) +
                (b + 3 < my_tile ? c3 : 0);
      all += c0 + c1 + c2 + c3;
    }
    for (; b < ntiles; ++b) {
      const int32_t c = tile_counts[static_cast<size_t>(b) * e + x];
      before += b < my_tile ? c : 0;
      all += c;
    }
    base_s[x] = before;
    total_s[x] = all;
    off_s[x] = capacity > 0 ? capacity : all;  // segment sizes, scanned below
  }
  __syncthreads();
  const int32_t seg_total = block_exclusive_scan(off_s, e, wave_tot);
  if (threadIdx.x == 0) off_s[e] = seg_total;
  __syncthreads();

  if (tile == 0) {  // publish the layout's per-expert arrays, checksum and flags
    for (int x = threadIdx.x; x < e; x += kTileTokens) {
      const int32_t c = total_s[x];
      counts[x] = c;
      kept_out[x] = capacity > 0 ? (c < capacity ? c : capacity) : c;
      offsets_out[x] = off_s[x];
    }
    if (threadIdx.x == 0) offsets_out[e] = off_s[e];
    uint64_t cks = 0;
    int f = 0;
    for (int b = threadIdx.x; b < ntiles; b += kTileTokens) {
      cks += tile_checksum[b];
      f |= tile_flags[b];
    }
    cks = wave_sum(cks);
    f = wave_or(f);
    if (lane == 0) {
      wave_cks[wv] = cks;
      wave_flg[wv] = f;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t c = 0;
      int ff = 0;
      for (int w = 0; w < kWaves; ++w) {
        c += wave_cks[w];
        ff |= wave_flg[w];
      }
      *checksum = c;
      *flags = ff;
    }
  }

  if (tile < ntiles) {  // uniform per workgroup
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
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          int d = -1;
          if (ok[j]) {
            const int x = ids[j];
            int r = base_s[x];
            for (int w = 0; w < wv; ++w) r += __popcll(lane_masks[w * e + x]);
            r += __popcll(lane_masks[wv * e + x] & below);
            if (capacity > 0)
              d = r < capacity ? x * capacity + r : -1;
            else
              d = off_s[x] + r;
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
  const int32_t begin = capacity > 0 ? 0 : off_s[e];
  const int32_t stride = gridDim.x * kTileTokens;
  for (int32_t r = begin + blockIdx.x * kTileTokens + threadIdx.x; r < rows; r += stride) {
    if (capacity > 0) {
      const int32_t x = r / capacity;
      const int32_t c = total_s[x];
      if (r - x * capacity >= (c < capacity ? c : capacity)) src[r] = -1;
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
  int grid = ntiles;
  if (L.capacity > 0) {
    const int64_t pad_blocks = (L.rows + kTileTokens - 1) / kTileTokens;
    const int64_t want = pad_blocks < 1024 ? pad_blocks : 1024;
    if (grid < want) grid = static_cast<int>(want);
  }
  if (grid < 1) grid = 1;
  const size_t lds = static_cast<size_t>(kTileTokens / kWave) * L.e * sizeof(unsigned long long) +
                     (3 * static_cast<size_t>(L.e) + 1) * sizeof(int32_t);
  layout_place_kernel<KMAX><<<grid, kTileTokens, lds, stream>>>(
      idx, L.s, L.e, L.k, L.capacity, static_cast<int32_t>(L.rows), ntiles, L.tile_counts,
      L.tile_checksum, L.tile_flags, L.counts, L.kept, L.offsets, L.checksum, L.flags, L.dst,
      L.src, L.route_idx);
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
