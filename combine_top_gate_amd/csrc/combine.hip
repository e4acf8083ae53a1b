// Combine: out[t][:] = sum_j topk_w[t][j] * y[dst_row[t][j]][:] (+ y[R + t][:] of the
// shared expert), fp32 accumulation in slot order, written in token order -- the
// expert windows are read where they are and nothing is restored in between
// ("Relay Buffer Independent Communication over Pooled HBM for Efficient MoE
// Inference on Ascend", abstract: direct reading from expert windows).
// Each thread owns one 16-byte piece of a token row: 8 bf16 or 4 fp32 values.  k <= 16.
// The output is the row in y's dtype, or FP8 codes with 1x128 scales for the next layer.
#include "kernels.h"

namespace {

// KM >= k row slots are loaded (a slot past k, or with no row, loads row 0 and is not
// added), so the loads carry no condition and are all in flight together; then the rows
// are added in slot order, the shared expert's (weight 1) last.
//
// Q8: the output is requantised for the next layer's FP8 input instead of rounded to
// the output dtype: per token row and 128-element block, s = fl32(amax / 448) (1 when
// amax = 0) and code = e4m3(clamp(fl32(v / s), +-448)), nearest even -- the rule of the
// h requantisation.  A block is 128 / V consecutive threads (aligned, all active since
// H is a multiple of 128), so its amax is a butterfly over those lanes.
// NTL: the y rows are read with nontemporal loads (streamed past the caches), for y larger
// than the 256 MB last-level cache, where the rows would not be read again anyway.  Measured
// alone on MI355X: 4096-token prefill (528 MB of y) 106.4 -> 93.1 us; the decode shapes,
// whose y stays cached, were 0.2 us slower with them (128-token 3.02 -> 3.24 us).
typedef unsigned int comb_u4 __attribute__((ext_vector_type(4)));
template <bool NTL>
__device__ __forceinline__ uint4 load_row16(const uint8_t* p) {
  if constexpr (NTL) {
    const comb_u4 v = __builtin_nontemporal_load((const __attribute__((address_space(1))) comb_u4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

template <bool F32, int KM, bool SH, bool Q8, bool NTL>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  constexpr int V = F32 ? 4 : 8;
  const int tok = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * V;
  if (c >= a.H) return;
  const uint8_t* ybase = static_cast<const uint8_t*>(a.y) + (int64_t)c * (F32 ? 4 : 2);
  const int64_t ystride = (int64_t)a.H * (F32 ? 4 : 2);
  // the token's row map and weights are the same for the whole workgroup (scalar loads);
  // the row map is read as KM consecutive entries (its buffer has MOE_MAX_TOPK entries of
  // padding past the last token), the weights only up to k
  const int32_t* rmap = a.dst_row + (int64_t)tok * a.k;
  const float* wmap = a.topk_w + (int64_t)tok * a.k;
  int rows[KM];
  float wts[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    rows[j] = j < a.k ? rmap[j] : -1;
    wts[j] = wmap[min(j, a.k - 1)];
  }
  uint4 yv[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) yv[j] = load_row16<NTL>(ybase + max(rows[j], 0) * ystride);
  uint4 ysh;
  if constexpr (SH) ysh = load_row16<NTL>(ybase + (int64_t)(a.R + tok) * ystride);
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  auto add = [&](const uint4& y, float w) {
    if constexpr (F32) {
      acc[0] = fmaf(w, __uint_as_float(y.x), acc[0]);
      acc[1] = fmaf(w, __uint_as_float(y.y), acc[1]);
      acc[2] = fmaf(w, __uint_as_float(y.z), acc[2]);
      acc[3] = fmaf(w, __uint_as_float(y.w), acc[3]);
    } else {
      const uint32_t u[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(w, bf16_to_f32(u[q] & 0xFFFFu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(w, bf16_to_f32(u[q] >> 16), acc[2 * q + 1]);
      }
    }
  };
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (rows[j] >= 0) add(yv[j], wts[j]);  // uniform
  if constexpr (SH) add(ysh, 1.0f);
  if constexpr (Q8) {
    constexpr int L = 128 / V;  // lanes per block
    float m = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) m = fmaxf(m, fabsf(acc[v]));
#pragma unroll
    for (int o = 1; o < L; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float sc = m > 0.f ? m / 448.0f : 1.0f;
    float q[V];
#pragma unroll
    for (int v = 0; v < V; ++v) q[v] = fminf(fmaxf(acc[v] / sc, -448.0f), 448.0f);
    uint8_t* orow = static_cast<uint8_t*>(a.out) + (int64_t)tok * a.H + c;
    if constexpr (F32) {
      *reinterpret_cast<uint32_t*>(orow) = pack4_e4m3(q[0], q[1], q[2], q[3]);
    } else {
      *reinterpret_cast<uint2*>(orow) = make_uint2(pack4_e4m3(q[0], q[1], q[2], q[3]), pack4_e4m3(q[4], q[5], q[6], q[7]));
    }
    if ((threadIdx.x & (L - 1)) == 0) a.out_scale[(int64_t)tok * (a.H >> 7) + (c >> 7)] = sc;
  } else if constexpr (F32) {
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

template <bool F32, bool SH, bool Q8, bool NTL>
void launch_km(const CombineArgs& a, dim3 grid, hipStream_t st) {
  if (a.k <= 2)
    hipLaunchKernelGGL((k_combine<F32, 2, SH, Q8, NTL>), grid, dim3(256), 0, st, a);
  else if (a.k <= 4)
    hipLaunchKernelGGL((k_combine<F32, 4, SH, Q8, NTL>), grid, dim3(256), 0, st, a);
  else if (a.k <= 8)
    hipLaunchKernelGGL((k_combine<F32, 8, SH, Q8, NTL>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_combine<F32, MOE_MAX_TOPK, SH, Q8, NTL>), grid, dim3(256), 0, st, a);
}

constexpr int64_t kLastLevelCacheBytes = 256ll << 20;

template <bool F32, bool Q8>
void launch_sh(const CombineArgs& a, dim3 grid, hipStream_t st) {
  const int64_t ybytes = (int64_t)(a.R + (a.has_shared ? a.T : 0)) * a.H * (F32 ? 4 : 2);
  if (ybytes > kLastLevelCacheBytes)
    a.has_shared ? launch_km<F32, true, Q8, true>(a, grid, st) : launch_km<F32, false, Q8, true>(a, grid, st);
  else
    a.has_shared ? launch_km<F32, true, Q8, false>(a, grid, st) : launch_km<F32, false, Q8, false>(a, grid, st);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const int V = a.y_f32 ? 4 : 8;
  const dim3 grid(a.T, (a.H + 256 * V - 1) / (256 * V));
  const bool q8 = a.out_scale != nullptr;
  if (a.y_f32)
    q8 ? launch_sh<true, true>(a, grid, st) : launch_sh<true, false>(a, grid, st);
  else
    q8 ? launch_sh<false, true>(a, grid, st) : launch_sh<false, false>(a, grid, st);
  return hipGetLastError();
}
