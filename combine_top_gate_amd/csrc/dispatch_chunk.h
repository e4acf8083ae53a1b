// Dispatch of one chunk of one source's tokens: per-source expert histogram +
// prefix sum + stable in-bucket rank, and the scatter of each of the chunk's token
// rows into its k rank-major window rows.  The dispatch kernel runs one chunk per
// workgroup; the fused SENTINEL launch runs the chunks in its lowest-numbered
// workgroups, ahead of the GEMM1 work items.
//
// Layout (the rank-major push of "One-Sided Expert-Parallel All-to-All for
// Mixture-of-Experts Inference over NVLink", abstract; counts and offsets as the
// only control state, "Relay Buffer Independent Communication over Pooled HBM for
// Efficient MoE Inference on Ascend", abstract): source s owns window rows
// [s*T_s*k, (s+1)*T_s*k); its valid (token, slot) pairs, i = t*k + j, are placed
// at s*T_s*k + off[s][e] + (rank of i among source s's pairs for e), where off is
// the exclusive prefix of source s's own counts.  No source reads another's ids.
//
// Chunk p owns tokens [p*tpb, (p+1)*tpb) of source s.  Every chunk builds s's
// histogram itself (the ids are a few KB, read from L2), so no workgroup waits for
// another: the ranks of its own pairs follow from the histogram of the pairs
// before the chunk plus in-chunk ballots.  Chunk 0 writes s's counts and offsets.
//
// Publication for the SENTINEL schedule ("GC-MoE: Overlapping Expert-Parallel
// Token Dispatch with FP8/FP4 Grouped GEMM via CUDA Green Contexts", three-node
// graph and token-ring handshake; epoch-tagged instead of cleared between calls):
// once chunk 0 of source s has written s's counts and offsets (all a GEMM needs to
// find its rows), it release-stores rflag[s] = epoch; every chunk then counts its
// arrival on arrive[s], and the last one to arrive (all of s's window rows
// written) resets that counter and release-stores dflag[s] = epoch.  The row maps
// (dst_row, row_src) are read only by kernels launched after the dispatch.
#pragma once
#include "kernels.h"

constexpr int kDispatchThreads = 256;  // the calling workgroup's size
// 16 bytes as a clang vector: an array of them stays in registers
typedef unsigned int dispatch_vec4 __attribute__((ext_vector_type(4)));
constexpr int kDispatchWaves = kDispatchThreads / 64;

struct DispatchSmem {
  int hist[MOE_MAX_EXPERTS];
  int run[MOE_MAX_EXPERTS];  // pairs of e before the chunk, then running position
  int wcnt[kDispatchWaves][MOE_MAX_EXPERTS];
  int part[kDispatchWaves];
  int dst[kMaxDispatchPairs];
};

__device__ __forceinline__ uint64_t dispatch_lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Copies `work` 16-byte vectors (the token rows from t0 on, nv vectors each) to the window
// rows in s_dst.  A thread issues U loads before its first store, with no branch between
// them (indices past the last vector read that vector again and store nothing), so a wave
// keeps U loads in flight instead of one.  U = 2 where the chunk is at most two vectors
// per thread (four would only add repeated reads: 7.1 against 6.5 us warm at 128 FP8
// tokens), else 4.  Measured on MI355X against one load per thread, dispatch alone, us
// warm / cold: 128 FP8 tokens 6.2 / 10.7 against 6.5 / 11.6; 256 bf16 tokens 8.3 / 13.1
// against 9.1 / 16.5; the 4096-token prefill 51 / 73 against 60 / 73.
template <int U>
struct DispatchCopyRegs {
  dispatch_vec4 val[U];
  int tt[U], vv[U];
};

// The U loads of the round that starts at vector w0 (work > 0).
template <int U>
__device__ __forceinline__ void dispatch_copy_load(const DispatchArgs& a, int s, int t0, int nv, int work, int w0,
                                                   DispatchCopyRegs<U>& r) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int w = min(w0 + u * kDispatchThreads, work - 1);
    r.tt[u] = w / nv;
    r.vv[u] = w - r.tt[u] * nv;
    r.val[u] = reinterpret_cast<const dispatch_vec4*>(a.src.x[s] + (int64_t)(t0 + r.tt[u]) * a.row_bytes)[r.vv[u]];
  }
}

template <int U>
__device__ __forceinline__ void dispatch_copy_store(const DispatchArgs& a, int work, int w0,
                                                    const DispatchCopyRegs<U>& r, const int* s_dst) {
  for (int j = 0; j < a.k; ++j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = s_dst[r.tt[u] * a.k + j];
      if (w0 + u * kDispatchThreads < work && row >= 0)
        reinterpret_cast<dispatch_vec4*>(a.win + (int64_t)row * a.row_bytes)[r.vv[u]] = r.val[u];
    }
  }
}

// Workgroup-uniform: chunk p (tokens [p*tpb, (p+1)*tpb)) of source s, of `chunks`, with
// U loads per thread per copy round.
template <int U>
__device__ __forceinline__ void dispatch_chunk_u(const DispatchArgs& a, int s, int p, int chunks, DispatchSmem& sm) {
  int* s_hist = sm.hist;
  int* s_run = sm.run;
  int (*s_wcnt)[MOE_MAX_EXPERTS] = sm.wcnt;
  int* s_part = sm.part;
  int* s_dst = sm.dst;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.T_s * a.k, E = a.E;
  const int t0 = p * a.tpb, t1 = min(a.T_s, t0 + a.tpb);
  const int i0 = t0 * a.k, i1 = t1 * a.k;
  const int base = s * n;
  const int32_t* ids = a.ids + base;
  // the copy's first round of loads goes out now: the source rows' addresses do not depend
  // on the routing below, so their latency overlaps it
  const int nv = a.row_bytes >> 4;
  const int work = (t1 - t0) * nv;
  DispatchCopyRegs<U> first;
  if (work > 0) dispatch_copy_load<U>(a, s, t0, nv, work, tid, first);

  for (int e = tid; e < MOE_MAX_EXPERTS; e += kDispatchThreads) {
    s_hist[e] = 0;
    s_run[e] = 0;
    for (int w = 0; w < kDispatchWaves; ++w) s_wcnt[w][e] = 0;
  }
  __syncthreads();

  bool bad = false;
  for (int i = tid; i < n; i += kDispatchThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E) {
      atomicAdd(&s_hist[e], 1);
      if (i < i0) atomicAdd(&s_run[e], 1);
    } else if (e != -1) {
      bad = true;
    }
  }
  if (bad && p == 0) atomicOr(a.err, MOE_DEVERR_BAD_ID);
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
  int before = 0, total = 0;
  for (int w = 0; w < kDispatchWaves; ++w) {
    if (w < wave) before += s_part[w];
    total += s_part[w];
  }
  if (tid < E) {
    const int excl = before + incl - v;
    if (p == 0) {
      a.cnt[s * E + tid] = v;
      a.off[s * E + tid] = excl;
    }
    s_run[tid] += excl;
  }
  __syncthreads();

  // ranks of this chunk's pairs, kDispatchThreads at a time: inside a wave the rank among
  // equal ids comes from ballots over the 8 id bits, earlier waves' counts are added
  const uint64_t lt = dispatch_lanemask_lt(lane);
  for (int c0 = i0; c0 < i1; c0 += kDispatchThreads) {
    const int i = c0 + tid;
    const int e = i < i1 ? ids[i] : -1;
    const bool valid = e >= 0 && e < E;
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
    if (i < i1) {
      int r = -1;
      if (valid) {
        int pos = s_run[e] + rank;
        for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
        r = base + pos;
        a.row_src[r] = base + i;
      }
      a.dst_row[base + i] = r;
      s_dst[i - i0] = r;
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
      for (int w = 0; w < kDispatchWaves; ++w) {
        add += s_wcnt[w][tid];
        s_wcnt[w][tid] = 0;
      }
      s_run[tid] += add;
    }
    __syncthreads();
  }
  // rows past this source's valid pairs stay unused
  if (p == chunks - 1)
    for (int r = total + tid; r < n; r += kDispatchThreads) a.row_src[base + r] = -1;
  if (a.rflag && p == 0) {
    wait_vmem();  // every wave's count and offset stores are done before thread 0 releases them
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.rflag + s, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (a.delay_ticks) {
    // test aid: hold the window rows back, so GEMM1 workgroups that have seen the counts
    // must wait for the rows (bounded: the host caps the delay far below the wait limit)
    // (each pass sleeps 512 clocks, over 20 ticks: the pass count ends the loop too)
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + a.delay_ticks;
    for (uint32_t it = 0; it < a.delay_ticks && __builtin_amdgcn_s_memrealtime() < t_end; ++it)
      __builtin_amdgcn_s_sleep(8);
  }

  // copy: each token row is read once as 16-byte vectors and written to its k rows
  if (tid < work) dispatch_copy_store<U>(a, work, tid, first, s_dst);
  for (int w0 = tid + U * kDispatchThreads; w0 < work; w0 += U * kDispatchThreads) {
    DispatchCopyRegs<U> r;
    dispatch_copy_load<U>(a, s, t0, nv, work, w0, r);
    dispatch_copy_store<U>(a, work, w0, r, s_dst);
  }
  if (a.nsc) {
    const int swork = (t1 - t0) * a.nsc;
    for (int w = tid; w < swork; w += kDispatchThreads) {
      const int tt = w / a.nsc, c = w - tt * a.nsc;
      const float sv = a.src.xs[s][(int64_t)(t0 + tt) * a.nsc + c];
      for (int j = 0; j < a.k; ++j) {
        const int r = s_dst[tt * a.k + j];
        if (r >= 0) a.wsc[(int64_t)r * a.nsc + c] = sv;
      }
    }
  }
  if (a.dflag) {
    wait_vmem();  // every wave's window rows are stored before thread 0 releases them
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(a.arrive + s, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == (uint32_t)chunks - 1) {
        // every workgroup of s has arrived: nobody touches the counter again this call
        __hip_atomic_store(a.arrive + s, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.dflag + s, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

__device__ __forceinline__ void dispatch_chunk(const DispatchArgs& a, int s, int p, int chunks, DispatchSmem& sm) {
  const int t0 = p * a.tpb, t1 = min(a.T_s, t0 + a.tpb);
  if ((t1 - t0) * (a.row_bytes >> 4) > 2 * kDispatchThreads)
    dispatch_chunk_u<4>(a, s, p, chunks, sm);
  else
    dispatch_chunk_u<2>(a, s, p, chunks, sm);
}
