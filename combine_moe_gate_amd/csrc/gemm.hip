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
// Tiling: a workgroup of 2 x NW waves computes a BM x BN tile of one expert's rows x
// output features; each wave owns WM x WN as (WM/32) x (WN/32) MFMA tiles of 32 x 32
// (v_mfma_f32_32x32x16 bf16/f16, float32 accumulators). Both operands are K-contiguous
// in memory (token rows; weight rows), so each is staged in LDS as [rows][BK elements]
// by direct-to-LDS loads into an XOR-swizzled layout (conflict-free 16-byte fragment
// reads). With 64-element K steps every staged row segment is one whole 128-byte line:
// each CU has a bounded number of L2 requests in flight, so whole-line requests double
// the bytes that bound admits. The token rows are staged SA K steps deep and the weights
// SB (SA >= SB): the loads of step kt + SA - 1 (kt + SB - 1) are issued while step kt is
// multiplied. Lane l of an MFMA reads row
// l%32, K elements 8*(l/32)..+7 of each operand (one ds_read_b128). The weights are the
// MFMA's first operand, so lane l holds token row l%32 and output features 8*(v/4) +
// 4*(l/32) + v%4 for v = 0..15: four consecutive features, written to the LDS output
// tile 8 bytes at a time (whole-row stores from there measured 1-3% faster than stores
// straight from the accumulators, results bit-identical).
//
// The input-row gradient, grad_A[r] = grad_out[r] @ W[x], is the same product with K = n
// and N = m and the weights read as [K][N] (BKN): that operand is staged K row by K row,
// each row's 256-column segment (512 bytes) filling half of a direct-to-LDS load, with
// 16-byte chunk positions XOR-swizzled by 4 (row % 4), and its MFMA fragments are read with
// gfx950's transposing LDS read ds_read_b64_tr_b16 (two per fragment, four K rows each).
// Within each 16-lane group that read hands lane i column i % 4 of the 4-element pieces
// the lanes i / 4 + 4 t (t = 0..3) point at; with lane j pointing at K row k0 + j / 4,
// columns c0 + 4 (j % 4) .. + 3, lane i receives K rows k0 .. k0 + 3 of column c0 + i. The
// 32 lanes served together touch 4 K rows x 4 chunks, which the swizzle spreads over 16
// distinct chunk positions of the 256-byte bank row.
//
// Schedule: the expert weights dominate the traffic (e * n * m elements, far above the
// L2), so tiles are ordered to read each weight tile few times. The tiles of all experts
// are numbered expert by expert; inside an expert, in bands of kBandRows row-blocks,
// column-block by column-block, row-block fastest. Workgroups are dealt round-robin over
// the 8 XCDs, so workgroup b takes tile (b mod 8) * T8 + b / 8 (T8 = ceil(tiles / 8)):
// each XCD walks one contiguous stretch of that order, and the workgroups resident on
// it at once share each weight tile across the band's row-blocks and each row-block's
// rows across neighbouring column-blocks through that XCD's L2. The 32 tiles an XCD runs
// together then span 8 row-blocks x 4 column-blocks: with 8-row bands the K-step slices
// they share are fewest (bands of 16 span 16 x 2 and read a third more per step; a
// dense 65536 x 3072 x 4096 product runs 10% faster with 8).
#include "gemm_common.h"
#include "internal.h"
#include "moe_device.h"

namespace moe {

constexpr int kBandRows = 8;  // row-blocks per band of the tile order
// Byte pitch of a row of the output tile staged in LDS (256 features of 2 bytes plus 16:
// successive rows start 4 banks apart).
constexpr int kOutPitch = 256 * 2 + 16;

// Waves are arranged 2 along the rows x NW along the columns of the tile; a K step is BK
// elements (BK / 8 chunks of 16 bytes per staged row); SA K steps of the token rows (A) and
// SB of the weights (B) are staged at once (SA >= SB).
template <int WM, int WN, int NW, int BK, int SA, int SB>
struct GemmShape {
  static constexpr int WAVES = 2 * NW, THREADS = WAVES * kWave;
  static constexpr int BM = 2 * WM, BN = NW * WN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int KS = BK / 16;                  // k16 MFMA steps per K step
  static constexpr int ROW_BYTES = BK * 2, CH = BK / 8;
  static constexpr int ROWS_PER_LOAD = 64 * 16 / ROW_BYTES;  // one direct-to-LDS load
  static constexpr int ROWS_PER_BANK_ROW = 256 / ROW_BYTES;  // rows per 256-byte bank row
  static constexpr int A_LOADS = BM / ROWS_PER_LOAD / WAVES;  // per wave per stage
  static constexpr int B_LOADS = BN / ROWS_PER_LOAD / WAVES;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int A_STAGE = BM * ROW_BYTES, B_STAGE = BN * ROW_BYTES;
  static constexpr int STAGED_BYTES = SA * A_STAGE + SB * B_STAGE;
  static constexpr int LDS_BYTES = STAGED_BYTES > BM * kOutPitch ? STAGED_BYTES : BM * kOutPitch;
  // loads a wave issues between those of step j and the wait that publishes step j (the
  // next step's, for the operands staged three deep)
  static constexpr int AHEAD = (SA >= 3 ? A_LOADS : 0) + (SB >= 3 ? B_LOADS : 0);
  static_assert(A_LOADS * ROWS_PER_LOAD * WAVES == BM && B_LOADS * ROWS_PER_LOAD * WAVES == BN,
                "stage split");
  static_assert(KS % 2 == 0, "fragment buffers alternate within a K step");
  static_assert(BN * 2 + 16 <= kOutPitch, "output tile rows fit the staging pitch");
  static_assert(SA >= SB && SB >= 2 && SA <= 3, "the token rows are staged at least as deep");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS of one workgroup");
  // XOR swizzle: slot p of staged row R holds chunk p ^ swz(R). The 16 lanes that one
  // 16-byte LDS read serves together read rows r .. r + 15 of one chunk; with this
  // swizzle they land in 16 different 16-byte groups of the 256-byte bank row.
  __device__ static constexpr int swz(int r) { return (r / ROWS_PER_BANK_ROW) % CH; }
};


// Stage one K step of rows into LDS with direct-to-LDS loads: instruction q of wave w
// fills the ROWS_PER_LOAD staged rows from (w * LOADS + q) * ROWS_PER_LOAD on, lane l
// writing row l / CH, slot l % CH, and so loading chunk (l % CH) ^ swz(row) of its row
// (c[q]). A chunk past the row end (the K tail) loads the row's first chunk instead, and
// its slot is cleared once landed.
template <int LOADS, int CH>
__device__ __forceinline__ void stage_rows(const chunk_t* const (&row)[LOADS], const int (&c)[LOADS],
                                           int kt, int kchunks, char* lds_rows) {
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int kq = kt * CH + c[q];
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(row[q] + (kq < kchunks ? kq : 0)),
                                     (lds_void_t*)(lds_rows + q * 64 * 16), 16, 0, 0);
  }
}

// Stage one K step of an operand stored [K][N] (each K row contiguous along N) with
// direct-to-LDS loads: instruction q of wave w fills the two staged K rows
// (w * LOADS + q) * 2 + {0, 1}, 512 bytes each; lane l writes row l / 32, slot l % 32, and
// so loads chunk (l % 32) ^ (4 (row % 4)) of that row's N segment (colp[q]). K rows past
// the end repeat the last one: the matching chunks of the other operand are cleared.
template <int LOADS>
__device__ __forceinline__ void stage_rows_kn(const chunk_t* const (&colp)[LOADS], const int (&krow)[LOADS],
                                              int kt, int K, int n_chunks, char* lds_rows) {
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int kk = kt * 64 + krow[q];
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(colp[q] + static_cast<size_t>(kk < K ? kk : K - 1) * n_chunks),
                                     (lds_void_t*)(lds_rows + q * 64 * 16), 16, 0, 0);
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// gfx950's transposing LDS read: within each 16-lane group, lane i receives column i % 4 of
// the 4-element pieces at the addresses of lanes i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12.
__device__ __forceinline__ uint2 read_tr16(const char* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

template <int LOADS, int CH>
__device__ __forceinline__ void clear_slots(const int (&c)[LOADS], int kt, int kchunks,
                                            char* lds_rows, int lane) {
  const chunk_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < LOADS; ++q)
    if (kt * CH + c[q] >= kchunks) *reinterpret_cast<chunk_t*>(lds_rows + q * 64 * 16 + lane * 16) = z;
}


// One workgroup per CU (its LDS stages take most of the CU's 160 KiB), NW / 2 waves per
// SIMD: the register file is these waves', so the schedule may keep two fragment sets live.
template <int DT, bool GATHER, bool SCALE, bool BKN, int WM, int WN, int NW, int BK, int SA, int SB>
__global__ __launch_bounds__(2 * NW * kWave)
__attribute__((amdgpu_waves_per_eu(NW / 2, NW / 2))) void expert_gemm_kernel(
    const chunk_t* __restrict__ a, const chunk_t* __restrict__ wts,
    const float* __restrict__ route_w, const int32_t* __restrict__ dst,
    const int32_t* __restrict__ src, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ offsets, int e, int k, int m, int n, int col_blocks,
    int band_rows, uint16_t* __restrict__ out) {
  using S = GemmShape<WM, WN, NW, BK, SA, SB>;
  static_assert(!BKN || (S::BN == 256 && BK == 64 && S::B_LOADS * 2 * S::WAVES == BK),
                "a [K][N] operand stages 64 K rows of 512 bytes, two per load instruction");
  // [SA][BM rows][ROW_BYTES] token rows, then [SB][BN rows][ROW_BYTES] weights; the output
  // tile reuses it at the end. No static LDS: the stages may take all 160 KiB.
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = wave_in_block();

  // every wave finds the workgroup's tile itself (the same for all)
  const TileCoord tc = find_tile<S::BM>(blockIdx.x, e, kept, col_blocks, band_rows);
  const int x = tc.expert;
  if (x < 0) return;  // no tile: uniform per workgroup
  const int row0 = offsets[x] + tc.rb * S::BM;
  const int rem = kept[x] - tc.rb * S::BM;
  const int nrows = rem < S::BM ? rem : S::BM;
  const int col0 = tc.cb * S::BN;
  const int wm = wv / NW, wn = wv % NW;  // this wave's part of the tile

  // the route weight of each output row this lane stores (weights after the experts)
  float row_sc[S::FM];
#pragma unroll
  for (int i = 0; i < S::FM; ++i) {
    row_sc[i] = 1.0f;
    if constexpr (SCALE) {
      const int row = wm * WM + i * 32 + (lane & 31);
      if (row < nrows) {
        const int r = row0 + row;
        const int t = src[r];
        for (int j = 0; j < k; ++j)
          if (dst[static_cast<size_t>(t) * k + j] == r) row_sc[i] = route_w[static_cast<size_t>(t) * k + j];
      }
    }
  }

  const int kchunks = m / 8;  // 16-byte chunks per operand row
  const int nk = (m + BK - 1) / BK;
  const chunk_t* wx = wts + static_cast<size_t>(x) * n * kchunks;

  // per load instruction: the staged row this lane fills, that row's start (columns past
  // n repeat column n - 1: they reach only output columns that are never stored), and
  // the chunk of it this lane stages
  const chunk_t* a_rows[S::A_LOADS];
  const chunk_t* b_rows[S::B_LOADS];
  int a_chunk[S::A_LOADS], b_chunk[S::B_LOADS];
#pragma unroll
  for (int q = 0; q < S::A_LOADS; ++q) {
    // rows past the segment repeat its first row: their products land only in output
    // rows that are never stored
    const int r = (wv * S::A_LOADS + q) * S::ROWS_PER_LOAD + lane / S::CH;
    const int rr = row0 + (r < nrows ? r : 0);
    a_rows[q] = a + static_cast<size_t>(GATHER ? src[rr] : rr) * kchunks;
    a_chunk[q] = (lane % S::CH) ^ S::swz(r);
  }
#pragma unroll
  for (int q = 0; q < S::B_LOADS; ++q) {
    if constexpr (BKN) {
      // weights stored [K][N]: this lane's column chunk of its staged K row (chunks past
      // N repeat the last one: they reach only output columns that are never stored), and
      // the K row itself
      const int kr = (wv * S::B_LOADS + q) * 2 + lane / 32;
      const int c = col0 / 8 + ((lane % 32) ^ (4 * (kr % 4)));
      b_rows[q] = wx + (c < n / 8 ? c : n / 8 - 1);
      b_chunk[q] = kr;
    } else {
      const int r = (wv * S::B_LOADS + q) * S::ROWS_PER_LOAD + lane / S::CH;
      const int j = col0 + r;
      b_rows[q] = wx + static_cast<size_t>(j < n ? j : n - 1) * kchunks;
      b_chunk[q] = (lane % S::CH) ^ S::swz(r);
    }
  }
  auto a_base = [&](int kt) { return lds + (kt % SA) * S::A_STAGE; };
  auto b_base = [&](int kt) { return lds + SA * S::A_STAGE + (kt % SB) * S::B_STAGE; };
  auto issue_a = [&](int kt) {
    stage_rows<S::A_LOADS, S::CH>(a_rows, a_chunk, kt, kchunks, a_base(kt) + wv * S::A_LOADS * 1024);
  };
  auto issue_b = [&](int kt) {
    char* st = b_base(kt) + wv * S::B_LOADS * 1024;
    if constexpr (BKN) stage_rows_kn<S::B_LOADS>(b_rows, b_chunk, kt, m, n / 8, st);
    else stage_rows<S::B_LOADS, S::CH>(b_rows, b_chunk, kt, kchunks, st);
  };
  // make step kt visible to the workgroup: this wave's loads for it have landed (only the
  // loads issued after them, those of step kt + 1 staged three deep, may remain), the
  // K-tail slots are cleared, then every wave meets at the barrier
  auto publish = [&](int kt) {
    if (S::AHEAD > 0 && kt + 1 < nk) __builtin_amdgcn_s_waitcnt(wait_vm(S::AHEAD));
    else __builtin_amdgcn_s_waitcnt(wait_vm(0));
    if ((kt + 1) * BK > m) {
      clear_slots<S::A_LOADS, S::CH>(a_chunk, kt, kchunks, a_base(kt) + wv * S::A_LOADS * 1024, lane);
      if constexpr (!BKN)
        clear_slots<S::B_LOADS, S::CH>(b_chunk, kt, kchunks, b_base(kt) + wv * S::B_LOADS * 1024, lane);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
    stage_barrier();
  };

  f32x16_t acc[S::FM][S::FN];
#pragma unroll
  for (int i = 0; i < S::FM; ++i)
#pragma unroll
    for (int jj = 0; jj < S::FN; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.0f;

  // fragment addresses: row (lane % 32) of each 32-row MFMA tile, chunk 2 ks + lane / 32,
  // found at slot chunk ^ swz(row) = chunk ^ swz(lane % 32) (tiles start at multiples of 32)
  const int a_frag = (wm * WM + (lane & 31)) * S::ROW_BYTES;
  const int b_frag = (wn * WN + (lane & 31)) * S::ROW_BYTES;
  const int fswz = S::swz(lane & 31);
  // [K][N] weights: each fragment is two transposing reads. Lane j of 16-lane group g
  // points at K row 8 (g / 2) + j / 4 of the k16 step (and 4 rows further for the second
  // read), N element 16 (g % 2) + 4 (j % 4) of the 32-column MFMA tile, at swizzled chunk
  // position chunk ^ 4 (row % 4); it receives 4 consecutive K rows of column lane % 32.
  const int tr_row = 8 * ((lane >> 4) >> 1) + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int tr_swz = 4 * ((lane & 15) >> 2);
  chunk_t fa[2][S::FM], fb[2][S::FN];
  auto read_frags = [&](int kt, int ks, int fbuf) {
    const char* sa = a_base(kt);
    const char* sb = b_base(kt);
    const int slot = ((2 * ks + (lane >> 5)) ^ fswz) * 16;
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
      fa[fbuf][i] = *reinterpret_cast<const chunk_t*>(sa + a_frag + i * 32 * S::ROW_BYTES + slot);
#pragma unroll
    for (int jj = 0; jj < S::FN; ++jj) {
      if constexpr (BKN) {
        const int byte = (wn * WN + jj * 32 + tr_col) * 2;
        const char* p = sb + (ks * 16 + tr_row) * 512 + (((byte >> 4) ^ tr_swz) << 4) + (byte & 15);
        const uint2 lo = read_tr16(p), hi = read_tr16(p + 4 * 512);
        fb[fbuf][jj] = chunk_t{lo.x, lo.y, hi.x, hi.y};
      } else {
        fb[fbuf][jj] = *reinterpret_cast<const chunk_t*>(sb + b_frag + jj * 32 * S::ROW_BYTES + slot);
      }
    }
  };
  // The weights are the MFMA's first operand, so each accumulator holds a 32-feature x
  // 32-row block transposed: lane l has row l % 32 and features 8 (v / 4) + 4 (l / 32) +
  // v % 4, four consecutive features per group of four values.
  auto mfmas = [&](int fbuf) {
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
      for (int jj = 0; jj < S::FN; ++jj)
        acc[i][jj] = mfma_32x32x16<DT>(fb[fbuf][jj], fa[fbuf][i], acc[i][jj]);
  };

  // prologue: the first SB - 1 weight steps and SA - 1 token-row steps in flight (weights
  // first at each step), step 0 published, its first fragments read
  for (int p = 0; p < SA - 1 && p < nk; ++p) {
    if (p < SB - 1) issue_b(p);
    issue_a(p);
  }
  publish(0);
  read_frags(0, 0, 0);

  // Per K step kt: issue the weights of step kt + SB - 1, then the token rows of step
  // kt + SA - 1 (each into the buffer step kt - 1 used, which every wave finished reading
  // before the last barrier). Each k16 step's fragments are read under the MFMAs of the
  // one before; before the last k16 step's MFMAs, step kt + 1 is published (the barrier
  // also tells every wave that step kt's buffers have been read out) and its first
  // fragments are read. The scheduling fences keep each batch of reads ahead of the MFMAs
  // that hide it.
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + SB - 1 < nk) issue_b(kt + SB - 1);
    if (kt + SA - 1 < nk) issue_a(kt + SA - 1);
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);  // this k16 step's fragments have landed
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < S::KS) {
        read_frags(kt, ks + 1, (ks + 1) & 1);
      } else if (kt + 1 < nk) {
        publish(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(kt + 1, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas(ks & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: optional route weight (weights after the experts), one narrowing. The
  // tile goes through LDS (free once every wave has left the main loop): each lane writes
  // its four-feature runs 8 bytes at a time, then the workgroup stores whole rows of the
  // tile, 32 lanes per 512-byte row, with 16-byte stores (straight from the accumulators,
  // an 8-byte store touches 32 rows and a 2-byte one 2: measured slower). n is a multiple
  // of 8, so a run or a 16-byte chunk never crosses it.
  __syncthreads();
  char* ot = lds;  // [BM][kOutPitch bytes]
#pragma unroll
  for (int i = 0; i < S::FM; ++i) {
    const int row = wm * WM + i * 32 + (lane & 31);
    const float sc = row_sc[i];
#pragma unroll
    for (int jj = 0; jj < S::FN; ++jj) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * WN + jj * 32 + 8 * g + 4 * (lane >> 5);
        float f[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          f[u] = acc[i][jj][4 * g + u];
          if constexpr (SCALE) f[u] = __fmul_rn(sc, f[u]);
        }
        *reinterpret_cast<uint2*>(ot + row * kOutPitch + col * 2) =
            uint2{narrow2<DT>(f[0], f[1]), narrow2<DT>(f[2], f[3])};
      }
    }
  }
  __syncthreads();
  constexpr int kRowChunks = S::BN * 2 / 16;
#pragma unroll 4
  for (int c = tid; c < S::BM * kRowChunks; c += S::THREADS) {
    const int row = c / kRowChunks, ch = c % kRowChunks;
    const int col = col0 + ch * 8;
    if (row < nrows && col < n)
      *reinterpret_cast<chunk_t*>(out + static_cast<size_t>(row0 + row) * n + col) =
          *reinterpret_cast<const chunk_t*>(ot + row * kOutPitch + ch * 16);
  }
}

// Tile shape chosen per launch (eight waves, 64-element K steps either way): 256 x 256
// tiles with both operands two steps deep when experts average at least 512 rows (the
// fewest operand bytes per MFMA), else 128 x 256 tiles three deep (less padding in short
// segments; the smaller stages leave LDS for a deeper pipeline). Staging the 256-row
// tiles' token rows three deep (all 160 KiB of LDS) measured 2-4% slower in interleaved
// runs on the Zipf, 32k-token and dropless workloads, forward and input-row gradient.
constexpr int kTallWM = 128, kTallWN = 64, kTallNW = 4, kTallBK = 64, kTallSA = 2, kTallSB = 2;
constexpr int kShortWM = 64, kShortWN = 64, kShortNW = 4, kShortBK = 64, kShortSA = 3, kShortSB = 3;

static bool use_tall(const LayoutView& L) {
  return L.capacity > 0 ? L.capacity >= 512 : static_cast<int64_t>(L.s) * L.k >= 512LL * L.e;
}

// An upper bound on the row-blocks in use, known on the host without reading the layout.
static int64_t row_block_bound(const LayoutView& L, int BM) {
  if (L.capacity > 0) return static_cast<int64_t>(L.e) * ((L.capacity + BM - 1) / BM);
  return (static_cast<int64_t>(L.s) * L.k + BM - 1) / BM + L.e;
}

static int64_t tile_grid(const LayoutView& L, int BM, int BN, int n) {
  if (L.s == 0) return 0;
  const int64_t col_blocks = (n + BN - 1) / BN;
  const int64_t tiles = row_block_bound(L, BM) * col_blocks;
  return (tiles + kXcds - 1) / kXcds * kXcds;
}

int64_t expert_gemm_grid(const LayoutView& L, int n) {
  return use_tall(L) ? tile_grid(L, 2 * kTallWM, kTallNW * kTallWN, n)
                     : tile_grid(L, 2 * kShortWM, kShortNW * kShortWN, n);
}

int64_t expert_gemm_kn_grid(const LayoutView& L, int N) {
  return tile_grid(L, 2 * kTallWM, kTallNW * kTallWN, N);
}

template <int DT, bool GATHER, bool SCALE, bool BKN, int WM, int WN, int NW, int BK, int SA, int SB>
static hipError_t gemm_launch(const LayoutView& L, const void* a, const void* w,
                              const float* route_w, int m, int n, void* out, hipStream_t stream) {
  using S = GemmShape<WM, WN, NW, BK, SA, SB>;
  auto kern = expert_gemm_kernel<DT, GATHER, SCALE, BKN, WM, WN, NW, BK, SA, SB>;
  // dynamic LDS above the 64 KiB default needs the per-kernel limit raised (idempotent)
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS_BYTES);
  if (err != hipSuccess) return err;
  const int64_t grid = tile_grid(L, S::BM, S::BN, n);
  if (grid == 0) return hipSuccess;
  const int col_blocks = (n + S::BN - 1) / S::BN;
  kern<<<static_cast<unsigned>(grid), S::THREADS, S::LDS_BYTES, stream>>>(
      static_cast<const chunk_t*>(a), static_cast<const chunk_t*>(w), route_w, L.dst, L.src, L.kept,
      L.offsets, L.e, L.k, m, n, col_blocks, kBandRows, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

template <int DT, bool GATHER, bool SCALE, bool BKN = false>
static hipError_t gemm_shape(const LayoutView& L, const void* a, const void* w,
                             const float* route_w, int m, int n, void* out, hipStream_t stream) {
  if (use_tall(L))
    return gemm_launch<DT, GATHER, SCALE, BKN, kTallWM, kTallWN, kTallNW, kTallBK, kTallSA, kTallSB>(
        L, a, w, route_w, m, n, out, stream);
  return gemm_launch<DT, GATHER, SCALE, BKN, kShortWM, kShortWN, kShortNW, kShortBK, kShortSA, kShortSB>(
      L, a, w, route_w, m, n, out, stream);
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

hipError_t launch_expert_gemm_kn(const LayoutView& L, const void* a, const void* w, int K, int N,
                                 int dtype, void* out, hipStream_t stream) {
  if (L.s > 0) {
    const hipError_t err =
        dtype == kBF16
            ? gemm_launch<kBF16, false, false, true, kTallWM, kTallWN, kTallNW, kTallBK, kTallSA, kTallSB>(
                  L, a, w, nullptr, K, N, out, stream)
            : gemm_launch<kF16, false, false, true, kTallWM, kTallWN, kTallNW, kTallBK, kTallSA, kTallSB>(
                  L, a, w, nullptr, K, N, out, stream);
    if (err != hipSuccess) return err;
  }
  return launch_zero_unfilled_rows(L, out, static_cast<int64_t>(N) * 2 / 16, stream);
}

}  // namespace moe
