// Top-k gate and its backward on gfx950.
//
// The gate: one wave64 per token. The e logits of a row sit in registers, ceil(e/64) per lane,
// as 32-bit order-preserving images of the float32 values (element i at lane i mod 64,
// slot i / 64). Each of the k rounds takes the wave-wide maximum of the untaken keys
// (DPP max steps plus four readlanes), then finds the lowest expert id holding it, so
// ties go to the lower id, and the owner marks it taken. With up to 8 slots that is one
// ballot per slot until one hits (ids of slot v are all below those of slot v+1); with 16
// (e > 512), whose ballot loop the compiler leaves rolled, a wave-wide minimum of each
// lane's lowest id holding the maximum (2.8x faster there, slower below). The experts
// come out in descending order.
// The weights are a softmax over the k selected logits, formed in float64 (equal to
// the full softmax renormalised over the selection: the full denominator cancels), for
// the workgroup's four tokens at once in one wave, one 16-lane row per token --
// DeepSpeed PR "MoE dispatch: fix silent Tutel + TP corruption, speed up native and
// Tutel paths", part 1: the gate hands on per-route expert ids and gate values, not a
// dense mask. (A 16-lane-row form with four tokens per wave, as the backward below uses,
// measured slower here: its k selection rounds are long dependent chains within a wave,
// while the wave-per-token grid fits on the chip at once.)
//
// The backward: one DPP row of 16 lanes per token for e <= 256 (a wave per token beyond).
#include "internal.h"
#include "moe_device.h"

namespace moe {

// Order-preserving map of a float32 to uint32 (-0.0 folded onto +0.0 first).
__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

template <int VPL>
__global__ __launch_bounds__(kBlock) void gate_topk_kernel(const float* __restrict__ logits,
                                                           int s, int e, int k,
                                                           int32_t* __restrict__ idx_out,
                                                           float* __restrict__ w_out) {
  // The softmax over each token's k selections runs once per workgroup, in wave 0: row q
  // (16 lanes) of that wave takes token q of the workgroup, lane r its route r (k <= 16).
  // Done in every wave instead, it would cost each token a whole wave's float64 work.
  static_assert(kWavesPerBlock * 16 == kWave, "one 16-lane row per token of the workgroup");
  __shared__ float sel_logit[kWavesPerBlock][16];
  const int lane = lane_id();
  const int wv = wave_in_block();
  const int t0 = blockIdx.x * kWavesPerBlock;
  const int t = t0 + wv;
  if (t < s) {  // uniform per wave; every wave still meets the barrier below
    const float* row = logits + static_cast<size_t>(t) * e;
    uint32_t key[VPL];
    bool taken[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int i = lane + v * kWave;
      taken[v] = i >= e;  // lanes past e never compete
      key[v] = taken[v] ? 0u : ordered_key(row[i]);
    }

    int my_idx = 0;  // lane r keeps the r-th selection
    uint32_t my_key = 0;
    for (int r = 0; r < k; ++r) {
      uint32_t best = 0;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const uint32_t kv = taken[v] ? 0u : key[v];
        best = kv > best ? kv : best;
      }
      best = wave_max_u32(best);
      int sel = 0;
      if constexpr (VPL <= 8) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          const uint64_t hit = __ballot(!taken[v] && key[v] == best);
          if (hit != 0ull) {  // uniform: the lowest id with the maximum is in slot v
            const int owner = static_cast<int>(__builtin_ctzll(hit));
            sel = owner + v * kWave;
            if (lane == owner) taken[v] = true;
            break;
          }
        }
      } else {  // 16 slots: each lane's lowest id holding the maximum, then their minimum
        uint32_t mine = 0xffffffffu;
#pragma unroll
        for (int v = VPL - 1; v >= 0; --v)
          if (!taken[v] && key[v] == best) mine = static_cast<uint32_t>(lane + v * kWave);
        sel = static_cast<int>(wave_min_u32(mine));
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (sel == lane + v * kWave) taken[v] = true;
      }
      if (lane == r) {
        my_idx = sel;
        my_key = best;
      }
    }
    if (lane < k) {
      idx_out[static_cast<size_t>(t) * k + lane] = my_idx;
      sel_logit[wv][lane] = key_to_float(my_key);
    }
  }
  __syncthreads();
  if (wv != 0) return;

  // w_r = exp(l_r - l_0) / sum_q exp(l_q - l_0) in float64, l_0 the largest selection
  const int q = lane >> 4, r = lane & 15;
  const bool active = t0 + q < s && r < k;
  const double ex = active ? exp(static_cast<double>(sel_logit[q][r]) - static_cast<double>(sel_logit[q][0]))
                           : 0.0;
  const double denom = row_sum_f64(ex);  // all lanes active here
  if (active) w_out[static_cast<size_t>(t0 + q) * k + r] = static_cast<float>(ex / denom);
}

// Gate backward: grad_logits[idx_j] = w_j (grad_w_j - sum_q w_q grad_w_q), float64,
// zero elsewhere. One wave per token; lanes j < k hold route j.
template <int VPL>
__global__ __launch_bounds__(kBlock) void gate_topk_backward_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, const float* __restrict__ gw,
    int s, int e, int k, float* __restrict__ gl) {
  const int lane = lane_id();
  const int t = blockIdx.x * kWavesPerBlock + wave_in_block();
  if (t >= s) return;
  const bool active = lane < k;
  const size_t o = static_cast<size_t>(t) * k + lane;
  const int my_idx = active ? idx[o] : -1;
  const double wj = active ? static_cast<double>(w[o]) : 0.0;
  const double gj = active ? static_cast<double>(gw[o]) : 0.0;
  const double dot = wave_sum(wj * gj);
  const double contrib = active ? wj * (gj - dot) : 0.0;

  int sel[16];
  double val[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    sel[j] = -1;
    val[j] = 0.0;
    if (j < k) {  // k is uniform: these are scalar reads of lane j
      sel[j] = __builtin_amdgcn_readlane(my_idx, j);
      val[j] = readlane_f64(contrib, j);
    }
  }
  float* out = gl + static_cast<size_t>(t) * e;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int i = lane + v * kWave;
    if (i < e) {
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < k && sel[j] == i) acc += val[j];
      out[i] = static_cast<float>(acc);
    }
  }
}

// The gate backward with one DPP row per token (four tokens per wave), for e <= 256: the
// row's lanes j < k hold route j; every lane gets all k (id, contribution) pairs from
// its row and writes its experts' entries (r, r + 16, ...: 64 contiguous bytes per row
// and store), summing repeated ids in route order.
template <int VPR>
__global__ __launch_bounds__(kBlock) void gate_topk_row_backward_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, const float* __restrict__ gw,
    int s, int e, int k, float* __restrict__ gl) {
  const int lane = lane_id();
  const int r = lane & 15;
  const int base = lane & ~15;
  const int t = (blockIdx.x * kWavesPerBlock + wave_in_block()) * 4 + (lane >> 4);
  const bool live = t < s;
  const bool active = live && r < k;
  const size_t o = static_cast<size_t>(live ? t : 0) * k + r;
  const int my_idx = active ? idx[o] : -1;
  const double wj = active ? static_cast<double>(w[o]) : 0.0;
  const double gj = active ? static_cast<double>(gw[o]) : 0.0;
  const double dot = row_sum_f64(wj * gj);
  const double contrib = active ? wj * (gj - dot) : 0.0;
  const uint64_t cbits = __builtin_bit_cast(uint64_t, contrib);
  const int c_lo = static_cast<int>(static_cast<uint32_t>(cbits));
  const int c_hi = static_cast<int>(static_cast<uint32_t>(cbits >> 32));

  double acc[VPR];
#pragma unroll
  for (int v = 0; v < VPR; ++v) acc[v] = 0.0;
  for (int j = 0; j < k; ++j) {  // k is uniform
    const int sel = __shfl(my_idx, base + j);
    const uint64_t lo = static_cast<uint32_t>(__shfl(c_lo, base + j));
    const uint64_t hi = static_cast<uint32_t>(__shfl(c_hi, base + j));
    const double val = __builtin_bit_cast(double, (hi << 32) | lo);
#pragma unroll
    for (int v = 0; v < VPR; ++v)
      if (sel == r + 16 * v) acc[v] += val;
  }
  if (live) {
    float* out = gl + static_cast<size_t>(t) * e;
#pragma unroll
    for (int v = 0; v < VPR; ++v) {
      const int i = r + 16 * v;
      if (i < e) out[i] = static_cast<float>(acc[v]);
    }
  }
}

// Weights renormalised over each token's kept routes (dst >= 0): w' = w / S with S the
// float64 sum of the kept weights in route order; 0 for dropped routes, and for every
// route when nothing is kept. One thread per token.
__global__ __launch_bounds__(kBlock) void renormalize_kept_kernel(const int32_t* __restrict__ dst,
                                                                  const float* __restrict__ w,
                                                                  int s, int k,
                                                                  float* __restrict__ w_out) {
  const int t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= s) return;
  const size_t o = static_cast<size_t>(t) * k;
  double S = 0.0;
  for (int j = 0; j < k; ++j)
    if (dst[o + j] >= 0) S += static_cast<double>(w[o + j]);
  for (int j = 0; j < k; ++j) {
    const bool keep = dst[o + j] >= 0 && S != 0.0;
    w_out[o + j] = keep ? static_cast<float>(static_cast<double>(w[o + j]) / S) : 0.0f;
  }
}

// Its backward: with u_j = w_j / S over kept routes, grad_w_i = (g_i - sum_q u_q g_q) / S
// for kept i and 0 otherwise, in float64 (sums in route order).
__global__ __launch_bounds__(kBlock) void renormalize_kept_backward_kernel(
    const int32_t* __restrict__ dst, const float* __restrict__ w, const float* __restrict__ g,
    int s, int k, float* __restrict__ gw) {
  const int t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= s) return;
  const size_t o = static_cast<size_t>(t) * k;
  double S = 0.0;
  for (int j = 0; j < k; ++j)
    if (dst[o + j] >= 0) S += static_cast<double>(w[o + j]);
  double dot = 0.0;
  if (S != 0.0)
    for (int j = 0; j < k; ++j)
      if (dst[o + j] >= 0) dot += (static_cast<double>(w[o + j]) / S) * static_cast<double>(g[o + j]);
  for (int j = 0; j < k; ++j) {
    const bool keep = dst[o + j] >= 0 && S != 0.0;
    gw[o + j] = keep ? static_cast<float>((static_cast<double>(g[o + j]) - dot) / S) : 0.0f;
  }
}

hipError_t launch_renormalize_kept(const LayoutView& L, const float* w, float* w_out,
                                   hipStream_t stream) {
  if (L.s == 0) return hipSuccess;
  renormalize_kept_kernel<<<(L.s + kBlock - 1) / kBlock, kBlock, 0, stream>>>(L.dst, w, L.s, L.k, w_out);
  return hipGetLastError();
}

hipError_t launch_renormalize_kept_backward(const LayoutView& L, const float* w,
                                            const float* grad_out, float* grad_w,
                                            hipStream_t stream) {
  if (L.s == 0) return hipSuccess;
  renormalize_kept_backward_kernel<<<(L.s + kBlock - 1) / kBlock, kBlock, 0, stream>>>(
      L.dst, w, grad_out, L.s, L.k, grad_w);
  return hipGetLastError();
}

static int values_per_lane(int e) {
  const int v = (e + kWave - 1) / kWave;
  return v <= 1 ? 1 : v <= 2 ? 2 : v <= 4 ? 4 : v <= 8 ? 8 : 16;
}

// Values per lane of the 16-lane row backward kernel (e <= 256).
static int values_per_row_lane(int e) {
  const int v = (e + 15) / 16;
  return v <= 1 ? 1 : v <= 2 ? 2 : v <= 4 ? 4 : v <= 8 ? 8 : 16;
}

hipError_t launch_gate_topk(const float* logits, int s, int e, int k, int32_t* idx, float* w,
                            hipStream_t stream) {
  if (s == 0) return hipSuccess;
  const dim3 grid((s + kWavesPerBlock - 1) / kWavesPerBlock), block(kBlock);
  switch (values_per_lane(e)) {
    case 1: gate_topk_kernel<1><<<grid, block, 0, stream>>>(logits, s, e, k, idx, w); break;
    case 2: gate_topk_kernel<2><<<grid, block, 0, stream>>>(logits, s, e, k, idx, w); break;
    case 4: gate_topk_kernel<4><<<grid, block, 0, stream>>>(logits, s, e, k, idx, w); break;
    case 8: gate_topk_kernel<8><<<grid, block, 0, stream>>>(logits, s, e, k, idx, w); break;
    default: gate_topk_kernel<16><<<grid, block, 0, stream>>>(logits, s, e, k, idx, w); break;
  }
  return hipGetLastError();
}

hipError_t launch_gate_topk_backward(const int32_t* idx, const float* w, const float* gw, int s,
                                     int e, int k, float* gl, hipStream_t stream) {
  if (s == 0) return hipSuccess;
  if (e <= 256) {
    const dim3 grid((s + 4 * kWavesPerBlock - 1) / (4 * kWavesPerBlock)), block(kBlock);
    switch (values_per_row_lane(e)) {
      case 1: gate_topk_row_backward_kernel<1><<<grid, block, 0, stream>>>(idx, w, gw, s, e, k, gl); break;
      case 2: gate_topk_row_backward_kernel<2><<<grid, block, 0, stream>>>(idx, w, gw, s, e, k, gl); break;
      case 4: gate_topk_row_backward_kernel<4><<<grid, block, 0, stream>>>(idx, w, gw, s, e, k, gl); break;
      case 8: gate_topk_row_backward_kernel<8><<<grid, block, 0, stream>>>(idx, w, gw, s, e, k, gl); break;
      default: gate_topk_row_backward_kernel<16><<<grid, block, 0, stream>>>(idx, w, gw, s, e, k, gl); break;
    }
    return hipGetLastError();
  }
  const dim3 grid((s + kWavesPerBlock - 1) / kWavesPerBlock), block(kBlock);
  switch (values_per_lane(e)) {
    case 8: gate_topk_backward_kernel<8><<<grid, block, 0, stream>>>(idx, w, gw, s, e, k, gl); break;
    default: gate_topk_backward_kernel<16><<<grid, block, 0, stream>>>(idx, w, gw, s, e, k, gl); break;
  }
  return hipGetLastError();
}

}  // namespace moe
