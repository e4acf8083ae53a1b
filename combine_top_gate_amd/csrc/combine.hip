// Combine: out[t][:] = sum_j topk_w[t][j] * y[dst_row[t][j]][:] (+ y[R + t][:] of the
// shared expert), fp32 accumulation in slot order, written in token order -- the
// expert windows are read where they are and nothing is restored in between
// ("Relay Buffer Independent Communication over Pooled HBM for Efficient MoE
// Inference on Ascend", abstract: direct reading from expert windows).
// Each thread owns one 16-byte piece of a token row: 8 bf16 or 4 fp32 values.
#include "kernels.h"

namespace {

template <bool F32>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  constexpr int V = F32 ? 4 : 8;
  const int tok = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * V;
  if (c >= a.H) return;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  auto add_row = [&](int r, float w) {
    if constexpr (F32) {
      const float4 y = *reinterpret_cast<const float4*>(static_cast<const float*>(a.y) + (int64_t)r * a.H + c);
      acc[0] = fmaf(w, y.x, acc[0]);
      acc[1] = fmaf(w, y.y, acc[1]);
      acc[2] = fmaf(w, y.z, acc[2]);
      acc[3] = fmaf(w, y.w, acc[3]);
    } else {
      const uint4 y = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.y) + (int64_t)r * a.H + c);
      const uint32_t u[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(w, bf16_to_f32(u[q] & 0xFFFFu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(w, bf16_to_f32(u[q] >> 16), acc[2 * q + 1]);
      }
    }
  };
  for (int j = 0; j < a.k; ++j) {
    const int r = a.dst_row[(int64_t)tok * a.k + j];
    if (r >= 0) add_row(r, a.topk_w[(int64_t)tok * a.k + j]);
  }
  if (a.has_shared) add_row(a.R + tok, 1.0f);
  if constexpr (F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (int64_t)tok * a.H + c) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
    uint4 o;
    o.x = bf16_bits(acc[0]) | (bf16_bits(acc[1]) << 16);
    o.y = bf16_bits(acc[2]) | (bf16_bits(acc[3]) << 16);
    o.z = bf16_bits(acc[4]) | (bf16_bits(acc[5]) << 16);
    o.w = bf16_bits(acc[6]) | (bf16_bits(acc[7]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (int64_t)tok * a.H + c) = o;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const int V = a.out_f32 ? 4 : 8;
  const dim3 grid(a.T, (a.H + 256 * V - 1) / (256 * V));
  if (a.out_f32)
    hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
