// Measurement aid: the FP8 MFMA rate this GPU sustains with no memory traffic, the
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

}  // namespace

hipError_t launch_mfma_fp8_probe(float* sink, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(k_mfma_fp8_probe, dim3(blocks), dim3(256), 0, st, sink, iters);
  return hipGetLastError();
}

int mfma_fp8_probe_chains() { return kChains; }
