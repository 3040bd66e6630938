// Pieces shared by the grouped expert GEMM kernels (forward and weight gradient) on
// gfx950: MFMA wrappers, element narrowing, a wave scan, and the LDS wait/barrier helpers.
#pragma once

#include "moe_device.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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

// Two values narrowed to a packed pair of the element type (a in the low half).
template <int DT>
__device__ __forceinline__ uint32_t narrow2(float a, float b) {
  if constexpr (DT == kBF16) return f32x2_to_bf16x2_rne(a, b);
  else return f32_to_f16_rne(a) | (f32_to_f16_rne(b) << 16);
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

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8): wait for LDS operations only; wait until at most n vector-memory loads remain.
constexpr int kWaitLdsOnly = 0xC07F;
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Barrier without a memory fence: the waits that make LDS contents visible are explicit
// (each wave's own direct-to-LDS loads and LDS writes have completed before it arrives),
// and the vector loads still in flight for later stages must not be waited for here.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

struct TileCoord {
  int expert, rb, cb;  // expert; row-block within its segment; column-block
};

// This workgroup's tile (expert = -1: none). Wave 0 only; uniform across the wave.
template <int BM>
__device__ __forceinline__ TileCoord find_tile(int b, int e, const int32_t* __restrict__ kept,
                                               int col_blocks, int band_rows) {
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
      const int band = u / (band_rows * col_blocks);
      const int left = R - band * band_rows;
      const int rows_in_band = left < band_rows ? left : band_rows;
      const int v = u - band * band_rows * col_blocks;
      tc.expert = c0 + owner;
      tc.cb = v / rows_in_band;
      tc.rb = band * band_rows + v % rows_in_band;
      return tc;
    }
    before += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return tc;
}


}  // namespace moe
