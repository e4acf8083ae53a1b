// Grouped GEMMs of the fp32 layer (no quantisation): h = silu(x W13g^T) * (x W13u^T)
// kept fp32, then y = h W2^T in fp32.  A plain FMA kernel: this layer is small, and it
// is here for the fp32 configuration's parity, not for speed.  Same work list as the
// low-precision kernels (routed experts, then the shared expert, group E), with a group's
// rows also spread over kRowSets workgroups (grid.y), since a small layer has few
// groups.  Each thread owns one output column of a row and walks its weight row and the
// token row in 16-byte pieces into four partial sums (one per lane of the piece), added
// pairwise at the end, so its loads are not serialised behind one chain of FMAs.
#include "kernels.h"

namespace {

constexpr int kCols = 64;     // output columns per workgroup; 4 token rows at a time
constexpr int kRowSets = 8;  // workgroups per column block, each taking every 8th group of 4 rows

__device__ __forceinline__ void group_of(const BatchDims& d, int nb_r, int nb_s, int& g, int& nb) {
  const int L = blockIdx.x;
  if (L < d.E * nb_r) {
    g = L / nb_r;
    nb = L - g * nb_r;
  } else {
    g = d.E;
    nb = L - d.E * nb_r;
  }
  (void)nb_s;
}

__device__ __forceinline__ int rows_of(const GemmArgs& p, int g) {
  if (g == p.d.E) return p.d.T;
  int M = 0;
  for (int s = 0; s < p.d.S; ++s) M += p.cnt[s * p.d.E + g];
  return M;
}

// sum over c < K of a[c] * b[c] (K a multiple of 4, rows 16-byte aligned), as four
// partial sums over the lanes of 16-byte pieces, added pairwise.
__device__ __forceinline__ float dot4(const float* a, const float* b, int K) {
  const float4* a4 = reinterpret_cast<const float4*>(a);
  const float4* b4 = reinterpret_cast<const float4*>(b);
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 8
  for (int c = 0; c < (K >> 2); ++c) {
    const float4 x = a4[c], y = b4[c];
    s0 = fmaf(x.x, y.x, s0);
    s1 = fmaf(x.y, y.y, s1);
    s2 = fmaf(x.z, y.z, s2);
    s3 = fmaf(x.w, y.w, s3);
  }
  return (s0 + s1) + (s2 + s3);
}

// this thread's first row and row step: rows of 4 per workgroup, kRowSets workgroups
__device__ __forceinline__ int first_row() { return blockIdx.y * (256 / kCols) + threadIdx.x / kCols; }
constexpr int kRowStep = kRowSets * (256 / kCols);

__global__ __launch_bounds__(256) void k_gemm1_f32(GemmArgs p) {
  const BatchDims& d = p.d;
  int g, nb;
  group_of(d, d.I / kCols, d.Ish / kCols, g, nb);
  const bool shared = g == d.E;
  const int inter = shared ? d.Ish : d.I;
  const int M = rows_of(p, g);
  const int n = nb * kCols + (threadIdx.x & (kCols - 1));
  const float* W = reinterpret_cast<const float*>(shared ? p.w_sh : p.w + (int64_t)g * p.w_stride);
  const float* wg = W + (int64_t)n * d.H;
  const float* wu = W + (int64_t)(inter + n) * d.H;
  const int seg = d.T_s * d.k;
  float* h = reinterpret_cast<float*>(p.h);
  for (int m = first_row(); m < M; m += kRowStep) {
    const float* x;
    int orow;
    if (shared) {
      const int s = m / d.T_s, t = m - s * d.T_s;
      x = reinterpret_cast<const float*>(p.src.x[s]) + (int64_t)t * d.H;
      orow = d.R + m;
    } else {
      orow = routed_row(p.cnt, p.off, d.S, d.E, seg, g, m);
      x = reinterpret_cast<const float*>(p.a) + (int64_t)orow * d.H;
    }
    const float ag = dot4(x, wg, d.H), au = dot4(x, wu, d.H);
    h[(int64_t)orow * d.hstride + n] = silu(ag) * au;
  }
}

__global__ __launch_bounds__(256) void k_gemm2_f32(GemmArgs p) {
  const BatchDims& d = p.d;
  int g, nb;
  group_of(d, d.H / kCols, d.Ish ? d.H / kCols : 0, g, nb);
  const bool shared = g == d.E;
  const int K = shared ? d.Ish : d.I;
  const int M = rows_of(p, g);
  const int n = nb * kCols + (threadIdx.x & (kCols - 1));
  const float* W = reinterpret_cast<const float*>(shared ? p.w_sh : p.w + (int64_t)g * p.w_stride);
  const float* wr = W + (int64_t)n * K;
  const int seg = d.T_s * d.k;
  const float* hbuf = reinterpret_cast<const float*>(p.a);
  for (int m = first_row(); m < M; m += kRowStep) {
    const int r = shared ? d.R + m : routed_row(p.cnt, p.off, d.S, d.E, seg, g, m);
    const float* h = hbuf + (int64_t)r * d.hstride;
    p.yf[(int64_t)r * d.H + n] = dot4(h, wr, K);
  }
}

}  // namespace

hipError_t launch_gemm1_f32(const GemmArgs& a, hipStream_t st) {
  const dim3 grid(a.d.E * (a.d.I / kCols) + a.d.Ish / kCols, kRowSets);
  hipLaunchKernelGGL(k_gemm1_f32, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm2_f32(const GemmArgs& a, hipStream_t st) {
  const dim3 grid(a.d.E * (a.d.H / kCols) + (a.d.Ish ? a.d.H / kCols : 0), kRowSets);
  hipLaunchKernelGGL(k_gemm2_f32, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
