// Measurement and verification aids (not part of the layer).
//
// The FP8 MFMA rate this GPU sustains with no memory traffic, the
// denominator the prefill GEMMs are compared with besides the published peak.
//
// Every wave runs kChains independent chains of v_mfma_scale_f32_16x16x128_f8f6f4 (the
// instruction the GEMMs use) on operands held in registers; a launch of `blocks`
// workgroups of 256 threads does blocks * 4 * iters * kChains MFMAs of 2*16*16*128 flop.
// The accumulators are summed into sink[blockIdx.x % 4] so the work is not discarded.
#include "kernels.h"

namespace {

constexpr int kChains = 4;

__global__ __launch_bounds__(256) void k_mfma_fp8_probe(float* sink, int iters) {
  const int lane = threadIdx.x & 63;
  // e4m3 0x38 = 1.0 and 0x30 = 0.5: finite operands, sums stay far from overflow
  const int a = 0x38383838, b = (lane & 1) ? 0x30303030 : 0x38383838;
  const v8i av = {a, a, a, a, a, a, a, a};
  const v8i bv = {b, b, b, b, b, b, b, b};
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[c], MFMA_FMT_FP8, MFMA_FMT_FP8, 0,
                                                                E8M0_ONE, 0, E8M0_ONE);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (lane == 0) atomicAdd(sink + (blockIdx.x & 3), s);
}

// One v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales: out[i][j] = the instruction's own
// sum over k of a[i][k] * b[j][k] for 16 rows a[i] (e4m3 or e2m1 codes, one per byte) and 16
// columns b[j] (e4m3) of 128 k.  Lane l holds row (and column) l % 16; with g = l / 16, an
// e4m3 operand holds k = 16 g + 0..15 in bytes 0..15 and k = 64 + 16 g + 0..15 in bytes
// 16..31, an e2m1 operand k = 32 g + 0..31 in nibbles 0..31 (low nibble first).  The
// result's lane l, register r is row 4 g + r, column l % 16.  Every lane stores its four
// results, so the instruction runs with all 64 lanes active (were only one lane's result
// used, the compiler could move the instruction and the operand assembly under that lane's
// branch).
template <bool FP4>
__global__ __launch_bounds__(64) void k_mfma_dot(const uint8_t* a, const uint8_t* b, float* out) {
  const int l = threadIdx.x, g = l >> 4, rc = l & 15;
  const uint8_t* ar = a + rc * 128;
  const uint8_t* br = b + rc * 128;
  v8i av, bv;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k0 = i < 4 ? 16 * g + 4 * i : 64 + 16 * g + 4 * (i - 4);
    bv[i] = (int)br[k0] | ((int)br[k0 + 1] << 8) | ((int)br[k0 + 2] << 16) | ((int)br[k0 + 3] << 24);
    if constexpr (FP4) {
      int w = 0;
      if (i < 4) {
#pragma unroll
        for (int n = 0; n < 8; ++n) w |= ((int)ar[32 * g + 8 * i + n] & 15) << (4 * n);
      }
      av[i] = w;
    } else {
      av[i] = (int)ar[k0] | ((int)ar[k0 + 1] << 8) | ((int)ar[k0 + 2] << 16) | ((int)ar[k0 + 3] << 24);
    }
  }
  const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
      av, bv, v4f{0.f, 0.f, 0.f, 0.f}, FP4 ? MFMA_FMT_FP4 : MFMA_FMT_FP8, MFMA_FMT_FP8, 0, E8M0_ONE, 0, E8M0_ONE);
#pragma unroll
  for (int q = 0; q < 4; ++q) out[(4 * g + q) * 16 + rc] = r[q];
}

}  // namespace

hipError_t launch_mfma_dot(bool a_fp4, const uint8_t* a, const uint8_t* b, float* out, hipStream_t st) {
  if (a_fp4)
    hipLaunchKernelGGL(k_mfma_dot<true>, dim3(1), dim3(64), 0, st, a, b, out);
  else
    hipLaunchKernelGGL(k_mfma_dot<false>, dim3(1), dim3(64), 0, st, a, b, out);
  return hipGetLastError();
}

hipError_t launch_mfma_fp8_probe(float* sink, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(k_mfma_fp8_probe, dim3(blocks), dim3(256), 0, st, sink, iters);
  return hipGetLastError();
}

int mfma_fp8_probe_chains() { return kChains; }
