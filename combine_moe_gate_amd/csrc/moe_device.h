// Device helpers shared by the gfx950 kernels of the MoE gate / dispatch / combine path:
// 16-byte row chunks, element conversions, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kBlock = 256;         // threads per workgroup of the gate kernels
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kTileTokens = 256;    // tokens per layout tile (one workgroup)

enum Dtype : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

// One 16-byte row chunk (a native vector, so loads/stores are single dwordx4 ops).
typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));

// Elements of each type in one 16-byte chunk.
template <int DT> struct ChunkElems { static constexpr int value = 8; };
template <> struct ChunkElems<kF32> { static constexpr int value = 4; };

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave index inside the workgroup, made provably uniform so that per-wave metadata
// goes through scalar registers.
__device__ __forceinline__ int wave_in_block() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ---------------------------------------------------------------------------------
// element conversions (widening is exact; narrowing rounds to nearest even)

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two float32 values to a packed pair of bfloat16, round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950 (low half = a, high half = b).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// The empty asm pins `a` as a materialised float32 register value. Without it the
// backend folds "float32 product, then narrow to f16" into one mixed-precision
// multiply that rounds only once, which is not the two-step rounding defined here.
__device__ __forceinline__ uint32_t f32_to_f16_rne(float a) {
  asm volatile("" : "+v"(a));
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(a));
}

// Unpack one 16-byte chunk into float32 values.
template <int DT>
__device__ __forceinline__ void unpack(const chunk_t& v, float (&f)[ChunkElems<DT>::value]) {
  if constexpr (DT == kF32) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  } else if constexpr (DT == kBF16) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  } else {
    f[0] = f16_bits_to_f32(v.x & 0xffffu); f[1] = f16_bits_to_f32(v.x >> 16);
    f[2] = f16_bits_to_f32(v.y & 0xffffu); f[3] = f16_bits_to_f32(v.y >> 16);
    f[4] = f16_bits_to_f32(v.z & 0xffffu); f[5] = f16_bits_to_f32(v.z >> 16);
    f[6] = f16_bits_to_f32(v.w & 0xffffu); f[7] = f16_bits_to_f32(v.w >> 16);
  }
}

// Pack float32 values into one 16-byte chunk of the element type.
template <int DT>
__device__ __forceinline__ chunk_t pack(const float (&f)[ChunkElems<DT>::value]) {
  chunk_t v;
  if constexpr (DT == kF32) {
    v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
    v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
  } else if constexpr (DT == kBF16) {
    v.x = f32x2_to_bf16x2_rne(f[0], f[1]);
    v.y = f32x2_to_bf16x2_rne(f[2], f[3]);
    v.z = f32x2_to_bf16x2_rne(f[4], f[5]);
    v.w = f32x2_to_bf16x2_rne(f[6], f[7]);
  } else {
    v.x = f32_to_f16_rne(f[0]) | (f32_to_f16_rne(f[1]) << 16);
    v.y = f32_to_f16_rne(f[2]) | (f32_to_f16_rne(f[3]) << 16);
    v.z = f32_to_f16_rne(f[4]) | (f32_to_f16_rne(f[5]) << 16);
    v.w = f32_to_f16_rne(f[6]) | (f32_to_f16_rne(f[7]) << 16);
  }
  return v;
}

// ---------------------------------------------------------------------------------
// wave64 reductions (butterfly over lane xor masks; every lane gets the result)

// 64-bit value of the lane that a DPP control names (all lanes must be active).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_move64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL,
                                             0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)),
                                             CTRL, 0xf, 0xf, false);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Wave-wide reductions, returned uniformly to every lane. Inside each row of 16 lanes:
// combine with the neighbour (quad_perm 1,0,3,2), the other pair (quad_perm 2,3,0,1),
// the mirrored half-row and the mirrored row, after which every lane of a row holds
// the row's result; the four rows are then combined from readlane values in the
// fixed order (r0 op r1) op (r2 op r3). All lanes must be active. No LDS traffic.
template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  static_assert(sizeof(T) == 8, "64-bit values");
  auto bits = [](T x) { return __builtin_bit_cast(uint64_t, x); };
  auto val = [](uint64_t u) { return __builtin_bit_cast(T, u); };
  v = op(v, val(dpp_move64<0xb1>(bits(v))));   // quad_perm [1,0,3,2]
  v = op(v, val(dpp_move64<0x4e>(bits(v))));   // quad_perm [2,3,0,1]
  v = op(v, val(dpp_move64<0x141>(bits(v))));  // row_half_mirror
  v = op(v, val(dpp_move64<0x140>(bits(v))));  // row_mirror
  const T a = val(readlane64(bits(v), 0)), b = val(readlane64(bits(v), 16));
  const T c = val(readlane64(bits(v), 32)), d = val(readlane64(bits(v), 48));
  return op(op(a, b), op(c, d));
}

__device__ __forceinline__ double wave_sum(double v) {
  return wave_reduce(v, [](double a, double b) { return a + b; });
}

__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
  return wave_reduce(v, [](uint64_t a, uint64_t b) { return a + b; });
}

__device__ __forceinline__ int wave_or(int v) {
  const uint64_t r = wave_reduce(static_cast<uint64_t>(static_cast<uint32_t>(v)),
                                 [](uint64_t a, uint64_t b) { return a | b; });
  return static_cast<int>(r);
}

// 32-bit maximum over the 64 lanes, returned uniformly: the same DPP pattern, where
// each step is a single v_max_u32 with a DPP source.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto step = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xb1, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4e, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xf, 0xf, false)));
  const uint32_t a = __builtin_amdgcn_readlane(static_cast<int>(v), 0);
  const uint32_t b = __builtin_amdgcn_readlane(static_cast<int>(v), 16);
  const uint32_t c = __builtin_amdgcn_readlane(static_cast<int>(v), 32);
  const uint32_t d = __builtin_amdgcn_readlane(static_cast<int>(v), 48);
  return step(step(a, b), step(c, d));
}

// 32-bit minimum over the 64 lanes, returned uniformly (the same steps as the maximum).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  auto step = [](uint32_t x, uint32_t y) { return x < y ? x : y; };
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xb1, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4e, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xf, 0xf, false)));
  const uint32_t a = __builtin_amdgcn_readlane(static_cast<int>(v), 0);
  const uint32_t b = __builtin_amdgcn_readlane(static_cast<int>(v), 16);
  const uint32_t c = __builtin_amdgcn_readlane(static_cast<int>(v), 32);
  const uint32_t d = __builtin_amdgcn_readlane(static_cast<int>(v), 48);
  return step(step(a, b), step(c, d));
}

// Sum over one DPP row (16 lanes), the result in every lane of the row: the four in-row
// steps of the wave reductions above, without the cross-row readlanes. All lanes must be
// active.
__device__ __forceinline__ double row_sum_f64(double v) {
  auto bits = [](double x) { return __builtin_bit_cast(uint64_t, x); };
  auto val = [](uint64_t u) { return __builtin_bit_cast(double, u); };
  v = v + val(dpp_move64<0xb1>(bits(v)));
  v = v + val(dpp_move64<0x4e>(bits(v)));
  v = v + val(dpp_move64<0x141>(bits(v)));
  v = v + val(dpp_move64<0x140>(bits(v)));
  return v;
}

// Maximum over the 64 lanes, returned uniformly.
__device__ __forceinline__ uint64_t wave_max(uint64_t v) {
  return wave_reduce(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  return __builtin_bit_cast(double, readlane64(u, lane));
}

}  // namespace moe
