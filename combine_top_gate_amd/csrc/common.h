// Shared device-side definitions of the HIP kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ctg_moe.h"

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// MFMA operand formats of v_mfma_scale_f32_16x16x128_f8f6f4
#define MFMA_FMT_FP8 0
#define MFMA_FMT_FP4 4
#define E8M0_ONE 127

// Per-source input pointers, passed by value in the kernel arguments.
struct SrcPtrs {
  const uint8_t* x[MOE_MAX_SRC];
  const float* xs[MOE_MAX_SRC];
};

// Sizes of the current batch.
struct BatchDims {
  int S, T_s, k, E;   // sources, tokens per source, slots, routed experts
  int H, I, Ish;      // hidden, routed intermediate, shared intermediate (0 = none)
  int R;              // S*T_s*k window rows
  int T;              // S*T_s tokens
  int hstride;        // bytes (FP8) or floats (F32) per row of the h window = max(I, Ish)
};

// Workgroup index -> position in a flat work list, so that consecutive list entries
// land on one XCD: the hardware hands workgroup b to XCD b % 8, and entries of one
// expert share that expert's activation rows in the XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  if ((total & 7) != 0) return b;
  return (b & 7) * (total >> 3) + (b >> 3);
}

// Row m of expert group g: routed experts concatenate, over sources in order, that
// source's bucket [s*T_s*k + off[s][g], + cnt[s][g]) of the rank-major window.
// Returns the window row, or -1 if m is past the expert's rows.
__device__ __forceinline__ int routed_row(const int32_t* cnt, const int32_t* off, int S, int E,
                                          int seg, int g, int m) {
  int base = 0;
  for (int s = 0; s < S; ++s) {
    int c = cnt[s * E + g];
    if (m < base + c) return s * seg + off[s * E + g] + (m - base);
    base += c;
  }
  return -1;
}

// fp32 -> 4 packed OCP e4m3 codes (round to nearest even; caller clamps to +-448).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32).
typedef float cvt_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 cvt_b2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((cvt_f2){lo, hi}, cvt_b2));
}
__device__ __forceinline__ uint32_t bf16_bits(float f) { return pack2_bf16(f, 0.f) & 0xFFFFu; }

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// SiLU with the hardware reciprocal (v_rcp_f32, 1 ulp) in place of an IEEE division.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// A value of a 1x128 block divided by the block's fp32 scale, clamped to the e4m3 range:
// inv_sc = __builtin_amdgcn_rcpf(scale), computed once per block (v_rcp_f32, 1 ulp).
__device__ __forceinline__ float e4m3_scaled(float v, float inv_sc) { return fminf(fmaxf(v * inv_sc, -448.0f), 448.0f); }

// Waits until this wave's vector memory operations, its stores included, have completed
// (s_waitcnt vmcnt(0): vmcnt 0, expcnt and lgkmcnt not waited for).  A workgroup barrier
// does not wait for other waves' stores, so before one wave releases the workgroup's
// stores at agent scope every wave calls this ahead of the barrier.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Makes the workgroup's global stores so far visible at agent scope with a single write-back
// of the XCD's L2 (issued by wave 0) instead of one per wave.  Every thread calls it; it
// ends with a barrier, so any thread may then publish with a relaxed agent-scope atomic.
__device__ __forceinline__ void release_workgroup_stores() {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x < 64) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
}
