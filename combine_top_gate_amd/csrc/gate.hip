// Gating ahead of dispatch: router logits and the top-k softmax gate.
//
// Each token is sent to the experts its gating result names and collected again
// afterwards ("GC-MoE: Decoupling MoE Communication and Computation with CUDA Green
// Contexts", section "Why Expert Parallelism Is Inefficient in MoE Decoding"); the gate
// is the sparsely-gated MoE layer's ("Relay Buffer Independent Communication over
// Pooled HBM for Efficient MoE Inference on Ascend", "Builds on"): keep the k largest
// logits (ties to the lower expert id, slot 0 the largest) and take a softmax over the
// kept ones.
//
// k_router: logits[t][e] = sum_h x[t][h] * wr[e][h], bf16 inputs, fp32 accumulation,
// on v_mfma_f32_16x16x32_bf16 (measured on gfx950: lane l, element i of the A operand is
// row l % 16 at k = 8 (l / 16) + i, the same for B's columns; result lane l, register i
// is row 4 (l / 16) + i, column l % 16).  A workgroup owns 16 experts x 16 tokens; its 4
// waves split H and add their partial tiles through LDS.  Experts sit in the A slot and
// tokens in the B slot, so each lane's operands are 16 contiguous bytes of a row.
//
// k_topk: one wave per token; E <= 256 logits, 4 per lane; k rounds of a wave argmax
// ordered by (logit descending, expert id ascending), then the softmax in fp32.
#include <math.h>

#include "kernels.h"

namespace {

typedef short v8s __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ u32x4 gload16(const uint16_t* p) { return *(const GLOBAL u32x4*)p; }
__device__ __forceinline__ v8s as_v8s(u32x4 v) {
  v8s r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (short)(v[i] & 0xFFFFu);
    r[2 * i + 1] = (short)(v[i] >> 16);
  }
  return r;
}

__global__ __launch_bounds__(256) void k_router(RouterArgs a) {
  __shared__ float s_part[4][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int r16 = lane & 15, g4 = lane >> 4;
  // rows past the end repeat the last one (their results are not stored)
  const int e = min(e0 + r16, a.E - 1), t = min(t0 + r16, a.T - 1);
  const uint16_t* wrow = a.wr + (int64_t)e * a.H + 8 * g4;
  const uint16_t* xrow = a.x + (int64_t)t * a.H + 8 * g4;
  const int steps = a.H / 32;  // 32-deep K steps, split over the 4 waves
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  int s = wave;
  for (; s + 12 < steps; s += 16) {  // four steps in flight per wave
    u32x4 wa[4], xb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wa[u] = gload16(wrow + (int64_t)(s + 4 * u) * 32);
      xb[u] = gload16(xrow + (int64_t)(s + 4 * u) * 32);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8s(wa[u]), as_v8s(xb[u]), acc, 0, 0, 0);
  }
  for (; s < steps; s += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8s(gload16(wrow + (int64_t)s * 32)),
                                                   as_v8s(gload16(xrow + (int64_t)s * 32)), acc, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) s_part[wave][lane][i] = acc[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the four waves' partial sums, added in wave order
      const float v = ((s_part[0][lane][i] + s_part[1][lane][i]) + s_part[2][lane][i]) + s_part[3][lane][i];
      const int er = e0 + 4 * g4 + i, tc = t0 + r16;  // result row = expert, column = token
      if (er < a.E && tc < a.T) a.logits[(int64_t)tc * a.E + er] = v;
    }
  }
}

__global__ __launch_bounds__(256) void k_topk(TopkArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;  // whole waves
  const float* z = a.logits + (int64_t)t * a.E;
  float v[4];
  bool taken[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < a.E ? z[e] : -INFINITY;
    taken[j] = e >= a.E;
  }
  float zsel = 0.f, zmax = 0.f, sum = 0.f;
  int myid = -1;
  float myz = 0.f;
  for (int r = 0; r < a.k; ++r) {
    // this lane's best untaken (largest logit, then lowest id: j ascending is id ascending)
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (!taken[j] && (v[j] > bv || bi == 0x7FFFFFFF)) {
        bv = v[j];
        bi = lane + 64 * j;
      }
    // wave argmax by (value desc, id asc)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == bi) taken[j] = true;
    zsel = bv;
    if (r == 0) zmax = bv;
    const float ex = expf(zsel - zmax);
    sum += ex;
    if (lane == r) {
      myid = bi;
      myz = zsel;
    }
  }
  if (lane < a.k) {
    a.ids[(int64_t)t * a.k + lane] = myid;
    a.w[(int64_t)t * a.k + lane] = expf(myz - zmax) / sum;
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_router, dim3((a.E + 15) / 16, (a.T + 15) / 16), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_topk, dim3((a.T + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}
