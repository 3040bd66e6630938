// Dispatch layout on gfx950: per-expert counts, slots, capacity drop, and the
// route -> row (dst) and row -> token (src) maps.
//
// The slot of a route is the column cumsum of the token x expert mask minus one
// (DeepSpeed PR "MoE dispatch: fix silent Tutel + TP corruption, speed up native and
// Tutel paths", review comment on fast_cumsum_sub_one): the number of routes to the
// same expert that come earlier. "Earlier" walks the routes as items:
//
//   token order  (default) item t = token t with its k routes; a token's routes never
//                share an expert, so the slot counts earlier tokens.
//   route major  item v = j*s + t holds the single route (t, j): every token's first
//                route comes before every second route (the per-route masks mask1,
//                mask2, ... of the same review comment, later columns offset by the
//                counts of earlier ones), so first choices win capacity.
//
// No sorting and no order-dependent atomics; two launches over tiles of 256 items (one
// when all items fit one tile: the place kernel then counts that tile itself, three when
// there are more than kScanTiles tiles):
//
//   count  one workgroup per tile: LDS histogram of the tile's valid routes (integer
//          atomic adds; the totals do not depend on their order), the tile's share of
//          the routing checksum and its flag bits.
//   scan   (more than kScanTiles tiles) one workgroup per expert turns its row of the
//          tile table into exclusive prefixes over the tiles, in place, and writes the
//          expert's total count: each place workgroup then reads one entry per expert
//          instead of the whole table, whose size grows with the batch.
//   place  one workgroup per tile again. Each workgroup first derives what it needs
//          from the small, L2-resident tile tables: for every expert the sum over
//          earlier tiles (its tile base) and over all tiles (the count), then an
//          exclusive scan over experts of the segment sizes (dropless: the count,
//          rounded up to the pad multiple; with a capacity: the capacity). Workgroup 0
//          publishes counts, kept, offsets, checksum and flags. Then each wave builds,
//          per expert, a 64-bit mask of its lanes (items) that chose it (LDS atomic OR:
//          order-independent); a route's slot is tile base + popcounts of the earlier
//          waves' masks + popcount of its own wave's mask below its lane. It writes
//          dst, src and a copy of the routing. Rows no route fills get src = -1.
#include "internal.h"
#include "moe_device.h"

namespace moe {

// The routes of one item. Token order: item t holds routes (t, 0..k-1); route major:
// item v holds the single route (v mod s, v div s). A route is valid if its expert is
// in [0, e) and no earlier route of the same token named it. Returns the flag bits.
template <int KMAX, bool RM>
__device__ __forceinline__ int load_item(const int32_t* __restrict__ idx, int item, int s, int k,
                                         int e, int& tok, int (&ids)[KMAX], bool (&ok)[KMAX],
                                         int64_t (&pos)[KMAX]) {
  int flags = 0;
  if constexpr (RM) {
    static_assert(KMAX == 1, "one route per item in route-major order");
    const int j = item / s;
    const int t = item - j * s;
    tok = t;
    const int64_t base = static_cast<int64_t>(t) * k;
    pos[0] = base + j;
    ids[0] = idx[pos[0]];
    const bool in_range = static_cast<unsigned>(ids[0]) < static_cast<unsigned>(e);
    bool dup = false;
    for (int q = 0; q < j; ++q) dup |= (idx[base + q] == ids[0]);
    if (!in_range) flags |= 1;
    else if (dup) flags |= 2;
    ok[0] = in_range && !dup;
  } else {
    tok = item;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      pos[j] = static_cast<int64_t>(item) * k + j;
      ids[j] = (j < k) ? idx[pos[j]] : -1;
    }
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
  }
  return flags;
}

template <int KMAX, bool RM>
__global__ __launch_bounds__(kTileTokens) void layout_count_kernel(
    const int32_t* __restrict__ idx, int s, int e, int k, int items, int ntp,
    int32_t* __restrict__ tile_counts, uint64_t* __restrict__ tile_checksum,
    int32_t* __restrict__ tile_flags) {
  extern __shared__ int32_t hist[];  // [e]
  __shared__ uint64_t part_sum[kTileTokens / kWave];
  __shared__ int32_t part_flags[kTileTokens / kWave];
  for (int i = threadIdx.x; i < e; i += kTileTokens) hist[i] = 0;
  __syncthreads();

  const int item = blockIdx.x * kTileTokens + threadIdx.x;
  uint64_t cks = 0;
  int flags = 0;
  if (item < items) {
    int tok, ids[KMAX];
    bool ok[KMAX];
    int64_t pos[KMAX];
    flags = load_item<KMAX, RM>(idx, item, s, k, e, tok, ids, ok, pos);
    const int nr = RM ? 1 : k;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < nr) {
        cks += static_cast<uint64_t>(static_cast<int64_t>(ids[j]) + 1) * static_cast<uint64_t>(pos[j] + 1);
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
  // expert-major table: row x holds expert x's count in every tile (row length ntp)
  for (int i = threadIdx.x; i < e; i += kTileTokens)
    tile_counts[static_cast<size_t>(i) * ntp + blockIdx.x] = hist[i];
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

// Tile counts of more than this many tiles are scanned by their own launch (measured at
// 512 and 1024 tiles: reading the whole table in every place workgroup costs more than the
// extra launch).
constexpr int kScanTiles = 256;

// Exclusive prefix over the tiles of expert x's row of the tile table, in place, and the
// expert's total into counts[x]. Thread i owns a contiguous run of tiles; the runs' sums
// are scanned across the workgroup (integer sums: exact in any order).
__global__ __launch_bounds__(kTileTokens) void layout_scan_kernel(int32_t* __restrict__ tile_counts,
                                                                  int ntiles, int ntp,
                                                                  int32_t* __restrict__ counts) {
  __shared__ int32_t wave_tot[kTileTokens / kWave];
  constexpr int kBatch = 8;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  int32_t* row = tile_counts + static_cast<size_t>(blockIdx.x) * ntp;
  const int per = (ntiles + kTileTokens - 1) / kTileTokens;
  const int b0 = static_cast<int>(threadIdx.x) * per;
  const int b1 = b0 + per < ntiles ? b0 + per : ntiles;
  int32_t sum = 0;
  for (int q = b0; q < b1; q += kBatch) {  // batches of independent loads
    int32_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = q + u < b1 ? row[q + u] : 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) sum += v[u];
  }
  int32_t incl = sum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  int32_t run = incl - sum, total = 0;
  for (int w = 0; w < kTileTokens / kWave; ++w) {
    if (w < wv) run += wave_tot[w];
    total += wave_tot[w];
  }
  for (int q = b0; q < b1; q += kBatch) {
    int32_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = q + u < b1 ? row[q + u] : 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (q + u < b1) row[q + u] = run;
      run += v[u];
    }
  }
  if (threadIdx.x == 0) counts[blockIdx.x] = total;
}

template <int KMAX, bool RM>
__global__ __launch_bounds__(kTileTokens) void layout_place_kernel(
    const int32_t* __restrict__ idx, int s, int e, int k, int items, int capacity, int pad,
    int32_t rows, int ntiles, int ntp, bool prefixed, const int32_t* __restrict__ tile_counts,
    const uint64_t* __restrict__ tile_checksum, const int32_t* __restrict__ tile_flags,
    int32_t* __restrict__ counts, int32_t* __restrict__ kept_out, int32_t* __restrict__ offsets_out,
    uint64_t* __restrict__ checksum, int32_t* __restrict__ flags, int32_t* __restrict__ dst,
    int32_t* __restrict__ src, int32_t* __restrict__ route_idx) {
  // LDS: the per-wave lane masks, then per expert tile base, total and segment offset
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
  const int my_tile = tile < ntiles ? tile : ntiles;  // workgroups past the tiles: padding only
  // A single tile has no count launch before it: every workgroup builds that tile's
  // histogram from the routes itself (workgroup 0 also its checksum and flags).
  const bool single = ntiles == 1;

  // this thread's routes, loaded first so that their latency overlaps the table reads
  const int item = (single ? 0 : tile) * kTileTokens + threadIdx.x;
  const int nr = RM ? 1 : k;
  int tok = 0, ids[KMAX];
  bool ok[KMAX];
  int64_t pos[KMAX];
  int item_flags = 0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ids[j] = -1;
    ok[j] = false;
    pos[j] = 0;
  }
  if ((tile < ntiles || single) && item < items)
    item_flags = load_item<KMAX, RM>(idx, item, s, k, e, tok, ids, ok, pos);
  // workgroup 0 publishes the checksum and flags: its first share of the tiles' values is
  // loaded now, beside the routes
  uint64_t tile_cks = 0;
  int tile_flg = 0;
  if (tile == 0 && !single && static_cast<int>(threadIdx.x) < ntiles) {
    tile_cks = tile_checksum[threadIdx.x];
    tile_flg = tile_flags[threadIdx.x];
  }
  if (tile < ntiles)  // cleared here, read after the barriers below
    for (int i = threadIdx.x; i < kWaves * e; i += kTileTokens) lane_masks[i] = 0ull;

  // per expert: sum over earlier tiles and over all tiles. Row x of the expert-major
  // tile table is read with 16-byte loads; with e <= 128 several threads share a row
  // (P parts of consecutive tiles) and their partial sums meet in LDS.
  __shared__ int32_t part_before[kTileTokens], part_all[kTileTokens];
  if (single) {
    // no earlier tile; the counts are the histogram of this tile's valid routes (LDS
    // integer adds, whose totals do not depend on their order)
    for (int x = threadIdx.x; x < e; x += kTileTokens) {
      base_s[x] = 0;
      total_s[x] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (ok[j]) atomicAdd(&total_s[ids[j]], 1);
    __syncthreads();
    for (int x = threadIdx.x; x < e; x += kTileTokens)
      off_s[x] = capacity > 0 ? capacity : (total_s[x] + pad - 1) / pad * pad;  // segment sizes
  } else if (prefixed) {
    // the scan launch left each tile's exclusive prefix in the table and the totals in
    // counts (workgroups past the tiles, padding only, take the totals as their base)
    for (int x = threadIdx.x; x < e; x += kTileTokens) {
      const int32_t tot = counts[x];
      base_s[x] = my_tile < ntiles ? tile_counts[static_cast<size_t>(x) * ntp + my_tile] : tot;
      total_s[x] = tot;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < e; x += kTileTokens)
      off_s[x] = capacity > 0 ? capacity : (total_s[x] + pad - 1) / pad * pad;  // segment sizes
  } else {
    const int P = e <= kTileTokens / 2 ? kTileTokens / e : 1;  // threads per expert
    const int nq = ntp / 4;                                      // int4 groups per row
    const int qlen = (nq + P - 1) / P;
    for (int slot = threadIdx.x; slot < (P > 1 ? P * e : e); slot += kTileTokens) {
      const int x = P > 1 ? slot % e : slot;
      const int part = P > 1 ? slot / e : 0;
      const int4* row = reinterpret_cast<const int4*>(tile_counts + static_cast<size_t>(x) * ntp);
      int32_t before = 0, all = 0;
      const int q1 = (part + 1) * qlen < nq ? (part + 1) * qlen : nq;
      // batches of independent loads (one dependent load per chunk costs a round trip each)
      constexpr int kBatch = 8;
      for (int q0 = part * qlen; q0 < q1; q0 += kBatch) {
        int4 cb[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) cb[u] = q0 + u < q1 ? row[q0 + u] : make_int4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int b = 4 * (q0 + u);
          const int32_t c0 = b < ntiles ? cb[u].x : 0, c1 = b + 1 < ntiles ? cb[u].y : 0;
          const int32_t c2 = b + 2 < ntiles ? cb[u].z : 0, c3 = b + 3 < ntiles ? cb[u].w : 0;
          before += (b < my_tile ? c0 : 0) + (b + 1 < my_tile ? c1 : 0) + (b + 2 < my_tile ? c2 : 0) +
                    (b + 3 < my_tile ? c3 : 0);
          all += c0 + c1 + c2 + c3;
        }
      }
      if (P > 1) {
        part_before[slot] = before;
        part_all[slot] = all;
      } else {
        base_s[x] = before;
        total_s[x] = all;
      }
    }
    if (P > 1) {
      __syncthreads();
      for (int x = threadIdx.x; x < e; x += kTileTokens) {
        int32_t before = 0, all = 0;
        for (int part = 0; part < P; ++part) {
          before += part_before[part * e + x];
          all += part_all[part * e + x];
        }
        base_s[x] = before;
        total_s[x] = all;
      }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < e; x += kTileTokens)
      off_s[x] = capacity > 0 ? capacity : (total_s[x] + pad - 1) / pad * pad;  // segment sizes
  }
  __syncthreads();
  const int32_t seg_total = block_exclusive_scan(off_s, e, wave_tot);
  if (threadIdx.x == 0) off_s[e] = seg_total;
  __syncthreads();

  if (tile == 0) {  // publish the layout's per-expert arrays, checksum and flags
    for (int x = threadIdx.x; x < e; x += kTileTokens) {
      const int32_t c = total_s[x];
      if (!prefixed) counts[x] = c;  // else the scan launch wrote them (other workgroups read them)
      kept_out[x] = capacity > 0 ? (c < capacity ? c : capacity) : c;
      offsets_out[x] = off_s[x];
    }
    if (threadIdx.x == 0) offsets_out[e] = off_s[e];
    uint64_t cks = 0;
    int f = 0;
    if (single) {  // this workgroup's own routes are the only tile's
      if (item < items) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (j < nr) cks += static_cast<uint64_t>(static_cast<int64_t>(ids[j]) + 1) * static_cast<uint64_t>(pos[j] + 1);
      }
      f = item_flags;
    } else {
      cks = tile_cks;
      f = tile_flg;
      for (int b = threadIdx.x + kTileTokens; b < ntiles; b += kTileTokens) {
        cks += tile_checksum[b];
        f |= tile_flags[b];
      }
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
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (ok[j]) atomicOr(&lane_masks[wv * e + ids[j]], 1ull << lane);
    __syncthreads();

    if (item < items) {
      const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < nr) {
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
          dst[pos[j]] = d;
          route_idx[pos[j]] = ids[j];
          if (d >= 0) src[d] = tok;
        }
      }
    }
  }

  // rows no route fills: the tail of each expert segment (capacity or pad rows), and
  // the rows past the last segment. Workgroup g takes segments x = g, g + grid, ...
  // (segment e is the tail), its threads striding over the segment's rows.
  for (int x = blockIdx.x; x <= e; x += gridDim.x) {
    int32_t r0, r1;
    if (x < e) {
      const int32_t c = total_s[x];
      r0 = off_s[x] + (capacity > 0 ? (c < capacity ? c : capacity) : c);
      r1 = capacity > 0 ? off_s[x] + capacity : off_s[x + 1];
    } else {
      r0 = off_s[e];
      r1 = rows;
    }
    for (int32_t r = r0 + threadIdx.x; r < r1; r += kTileTokens) src[r] = -1;
  }
}

template <int KMAX, bool RM>
static hipError_t launch_layout_k(const int32_t* idx, const LayoutView& L, hipStream_t stream) {
  const int ntiles = L.ntiles;
  const int items = RM ? L.s * L.k : L.s;
  if (ntiles > 1) {  // one tile: the place kernel counts it itself
    layout_count_kernel<KMAX, RM><<<ntiles, kTileTokens, L.e * sizeof(int32_t), stream>>>(
        idx, L.s, L.e, L.k, items, tile_row_length(ntiles), L.tile_counts, L.tile_checksum,
        L.tile_flags);
  }
  const bool prefixed = ntiles > kScanTiles;
  if (prefixed)
    layout_scan_kernel<<<L.e, kTileTokens, 0, stream>>>(L.tile_counts, ntiles, tile_row_length(ntiles),
                                                        L.counts);
  int grid = ntiles < 1 ? 1 : ntiles;
  if ((L.capacity > 0 || L.pad_multiple > 1) && grid < L.e + 1)
    grid = L.e + 1 < 1024 ? L.e + 1 : 1024;  // one workgroup per padded segment
  const size_t lds = static_cast<size_t>(kTileTokens / kWave) * L.e * sizeof(unsigned long long) +
                     (3 * static_cast<size_t>(L.e) + 1) * sizeof(int32_t);
  layout_place_kernel<KMAX, RM><<<grid, kTileTokens, lds, stream>>>(
      idx, L.s, L.e, L.k, items, L.capacity, L.pad_multiple, static_cast<int32_t>(L.rows), ntiles,
      tile_row_length(ntiles), prefixed, L.tile_counts, L.tile_checksum, L.tile_flags, L.counts, L.kept, L.offsets, L.checksum,
      L.flags, L.dst, L.src, L.route_idx);
  return hipGetLastError();
}

hipError_t launch_layout(const int32_t* idx, const LayoutView& L, hipStream_t stream) {
  if (L.route_major) return launch_layout_k<1, true>(idx, L, stream);
  switch (route_bound(L.k)) {
    case 1: return launch_layout_k<1, false>(idx, L, stream);
    case 2: return launch_layout_k<2, false>(idx, L, stream);
    case 4: return launch_layout_k<4, false>(idx, L, stream);
    case 8: return launch_layout_k<8, false>(idx, L, stream);
    default: return launch_layout_k<16, false>(idx, L, stream);
  }
}

}  // namespace moe
