// Dispatch: per-source expert histogram + prefix sum + stable in-bucket rank, then
// a scatter of each token row into its k rank-major window rows.
//
// Layout (the rank-major push of "One-Sided Expert-Parallel All-to-All for
// Mixture-of-Experts Inference over NVLink", abstract; counts and offsets as the
// only control state, "Relay Buffer Independent Communication over Pooled HBM for
// Efficient MoE Inference on Ascend", abstract): source s owns window rows
// [s*T_s*k, (s+1)*T_s*k); its valid (token, slot) pairs, i = t*k + j, are placed
// at s*T_s*k + off[s][e] + (rank of i among source s's pairs for e), where off is
// the exclusive prefix of source s's own counts.  No source reads another's ids.
#include "kernels.h"

namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / 64;

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// One workgroup per source.  Pass 1 counts pairs per expert in LDS, a wave scan
// turns the counts into offsets, pass 2 walks the pairs in order, 256 at a time:
// inside a wave the rank among equal ids comes from ballots over the id bits, and
// earlier waves' counts (in LDS) are added, so the order is i-ascending in every
// bucket without atomics deciding it.
__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a) {
  __shared__ int s_hist[MOE_MAX_EXPERTS];
  __shared__ int s_run[MOE_MAX_EXPERTS];
  __shared__ int s_wcnt[kRouteWaves][MOE_MAX_EXPERTS];
  __shared__ int s_part[kRouteWaves];

  const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.T_s * a.k, E = a.E;
  const int base = s * n;
  const int32_t* ids = a.ids + base;

  for (int e = tid; e < MOE_MAX_EXPERTS; e += kRouteThreads) {
    s_hist[e] = 0;
    for (int w = 0; w < kRouteWaves; ++w) s_wcnt[w][e] = 0;
  }
  __syncthreads();

  bool bad = false;
  for (int i = tid; i < n; i += kRouteThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E)
      atomicAdd(&s_hist[e], 1);
    else if (e != -1)
      bad = true;
  }
  if (bad) atomicOr(a.err, MOE_DEVERR_BAD_ID);
  __syncthreads();

  // exclusive scan of the histogram (E <= 256 = one entry per thread)
  const int v = tid < E ? s_hist[tid] : 0;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_part[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_part[w];
  int total = 0;
  for (int w = 0; w < kRouteWaves; ++w) total += s_part[w];
  if (tid < E) {
    const int excl = before + incl - v;
    a.cnt[s * E + tid] = v;
    a.off[s * E + tid] = excl;
    s_run[tid] = excl;
  }
  __syncthreads();

  const uint64_t lt = lanemask_lt(lane);
  for (int c0 = 0; c0 < n; c0 += kRouteThreads) {
    const int i = c0 + tid;
    const int e = i < n ? ids[i] : -1;
    const bool valid = e >= 0 && e < E;
    // lanes of this wave holding the same expert id (ids < 256: 8 bits)
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    const int rank = __popcll(same & lt);
    if (valid && rank == 0) s_wcnt[wave][e] = __popcll(same);
    __syncthreads();
    if (i < n) {
      if (valid) {
        int pos = s_run[e] + rank;
        for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
        const int r = base + pos;
        a.dst_row[base + i] = r;
        a.row_src[r] = base + i;
      } else {
        a.dst_row[base + i] = -1;
      }
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
      for (int w = 0; w < kRouteWaves; ++w) {
        add += s_wcnt[w][tid];
        s_wcnt[w][tid] = 0;
      }
      s_run[tid] += add;
    }
    __syncthreads();
  }
  // rows past this source's valid pairs stay unused
  for (int r = total + tid; r < n; r += kRouteThreads) a.row_src[base + r] = -1;
}

// One workgroup per token: the row is read once as 16-byte vectors and written to
// each of its (up to k) window rows; its 1x128 scales follow the same way.
__global__ __launch_bounds__(256) void k_scatter(ScatterArgs a) {
  __shared__ int s_dst[MOE_MAX_TOPK];
  const int tok = blockIdx.x;
  const int s = tok / a.T_s, t = tok - s * a.T_s;
  if (threadIdx.x < a.k) s_dst[threadIdx.x] = a.dst_row[(int64_t)tok * a.k + threadIdx.x];
  __syncthreads();
  const uint4* src = reinterpret_cast<const uint4*>(a.src.x[s] + (int64_t)t * a.row_bytes);
  const int nv = a.row_bytes >> 4;
  for (int v = threadIdx.x; v < nv; v += 256) {
    const uint4 val = src[v];
    for (int j = 0; j < a.k; ++j) {
      const int r = s_dst[j];
      if (r >= 0) reinterpret_cast<uint4*>(a.win + (int64_t)r * a.row_bytes)[v] = val;
    }
  }
  if (a.nsc) {
    const float* ss = a.src.xs[s] + (int64_t)t * a.nsc;
    for (int c = threadIdx.x; c < a.nsc; c += 256) {
      const float sv = ss[c];
      for (int j = 0; j < a.k; ++j) {
        const int r = s_dst[j];
        if (r >= 0) a.wsc[(int64_t)r * a.nsc + c] = sv;
      }
    }
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_route, dim3(a.S), dim3(kRouteThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_scatter, dim3(a.S * a.T_s), dim3(256), 0, st, a);
  return hipGetLastError();
}
