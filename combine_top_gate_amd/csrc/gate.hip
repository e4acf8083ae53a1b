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
// is row 4 (l / 16) + i, column l % 16).  A workgroup owns 16 experts x 16 TT tokens;
// its waves split the H / 32 MFMA steps round-robin and issue a whole batch of steps'
// loads before the first MFMA, so a wave waits on memory once per batch, not per step.
// The partial tiles are added through LDS in wave order (a fixed order: the result does
// not depend on timing).  Experts sit in the A slot and tokens in the B slot, so each
// lane's operands are 16 contiguous bytes of a row.
//
// k_router_split (the fused gate's first launch): the same tiles, with the K steps also
// split into ks contiguous slices over workgroups, so that a small batch still spreads
// over every CU; each workgroup writes its slice's partial tile to a workspace.
//
// k_router_lds (many tokens, H a multiple of 128): a workgroup owns 64 tokens x 64
// experts and a K slice.  128-deep K chunks of both operands are staged in LDS, each row
// padded to 272 bytes, double-buffered; the loads (16 contiguous bytes per thread and
// piece, whole 256-byte rows per 16 threads) run two chunks ahead in two register sets,
// and a chunk is written to the free buffer after the current one's MFMAs, one barrier
// per chunk.  Four waves of 32 tokens x 32 experts (2 x 2 MFMA tiles each); each wave
// chains its whole K slice in one accumulator.  The fragment
// loads of the other two kernels, 16 bytes from each of 16 rows per instruction and every
// row re-read by each expert block, bound them at a few percent of the MFMA rate once the
// batch has thousands of tokens.
//
// k_topk: one wave (and workgroup) per token, E <= 256 logits, 4 per lane (added up from the ks partial
// sums in slice order first, when there are several).  The k-th largest logit is
// found exactly by a radix select over order-preserving 32-bit keys (one ballot per
// lane register and bit); the k selected logits (ties at the threshold to the lower
// expert ids) go to LDS, where each is ranked by (logit descending, id ascending) and
// the softmax over them is taken in fp32.
#include <math.h>

#include <algorithm>

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

// TT token tiles per workgroup, W waves splitting K, NB steps in flight per wave.
template <int TT, int W, int NB>
__global__ __launch_bounds__(64 * W) void k_router(RouterArgs a) {
  __shared__ v4f s_part[W][TT][64];
  // the wave index is made a scalar so the step loop and its bounds test stay uniform
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int eb = blockIdx.x, tb = blockIdx.y;
  if (TT > 1) {
    // Workgroups reach the 8 XCDs round-robin by linear id.  Renumber them so that XCD x
    // takes one contiguous run of token tiles with every expert block: a token tile is
    // then fetched into one XCD's L2 once and read there by all expert blocks.
    const int n = gridDim.x * gridDim.y, b = blockIdx.x + gridDim.x * blockIdx.y;
    const int xcd = b & 7, per = n >> 3, extra = n & 7;
    const int L = xcd * per + min(xcd, extra) + (b >> 3);
    eb = L % gridDim.x;
    tb = L / gridDim.x;
  }
  const int e0 = eb * 16, t0 = tb * 16 * TT;
  const int r16 = lane & 15, g4 = lane >> 4;
  // rows past the end repeat the last one (their results are not stored)
  const uint16_t* wrow = a.wr + (int64_t)min(e0 + r16, a.E - 1) * a.H + 8 * g4;
  const uint16_t* xrow[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) xrow[u] = a.x + (int64_t)min(t0 + 16 * u + r16, a.T - 1) * a.H + 8 * g4;
  const int steps = a.H / 32;
  v4f acc[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
  int s0 = wave;
  for (; s0 + (NB - 1) * W < steps; s0 += W * NB) {  // whole batches: every load before any MFMA
    u32x4 wa[NB], xb[NB][TT];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t off = (int64_t)(s0 + i * W) * 32;
      wa[i] = gload16(wrow + off);
#pragma unroll
      for (int u = 0; u < TT; ++u) xb[i][u] = gload16(xrow[u] + off);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the whole batch of loads ahead of the MFMAs
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int u = 0; u < TT; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8s(wa[i]), as_v8s(xb[i][u]), acc[u], 0, 0, 0);
  }
  for (; s0 < steps; s0 += W) {  // the rest, a step at a time
    const int64_t off = (int64_t)s0 * 32;
    const u32x4 wa = gload16(wrow + off);
#pragma unroll
    for (int u = 0; u < TT; ++u)
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8s(wa), as_v8s(gload16(xrow[u] + off)), acc[u], 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < TT; ++u) s_part[wave][u][lane] = acc[u];
  __syncthreads();
  for (int idx = threadIdx.x; idx < TT * 64 * 4; idx += 64 * W) {
    const int u = idx >> 8, l = (idx >> 2) & 63, i = idx & 3;
    float v = s_part[0][u][l][i];
#pragma unroll
    for (int w = 1; w < W; ++w) v += s_part[w][u][l][i];
    const int er = e0 + 4 * (l >> 4) + i, tc = t0 + 16 * u + (l & 15);  // row = expert, column = token
    if (er < a.E && tc < a.T) a.logits[(int64_t)tc * a.E + er] = v;
  }
}

template <int TT, int NB>
__global__ __launch_bounds__(256) void k_router_split(RouterSplitArgs a) {
  constexpr int W = 4;
  __shared__ v4f s_part[W][TT][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16 * TT, slice = blockIdx.z;
  const int r16 = lane & 15, g4 = lane >> 4;
  const uint16_t* wrow = a.wr + (int64_t)min(e0 + r16, a.E - 1) * a.H + 8 * g4;
  const uint16_t* xrow[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) xrow[u] = a.x + (int64_t)min(t0 + 16 * u + r16, a.T - 1) * a.H + 8 * g4;
  const int steps = a.H / 32;
  const int s_begin = (int)((int64_t)steps * slice / a.ks), s_end = (int)((int64_t)steps * (slice + 1) / a.ks);
  v4f acc[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
  int s0 = s_begin + wave;
  for (; s0 + (NB - 1) * W < s_end; s0 += W * NB) {
    u32x4 wa[NB], xb[NB][TT];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t off = (int64_t)(s0 + i * W) * 32;
      wa[i] = gload16(wrow + off);
#pragma unroll
      for (int u = 0; u < TT; ++u) xb[i][u] = gload16(xrow[u] + off);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int u = 0; u < TT; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8s(wa[i]), as_v8s(xb[i][u]), acc[u], 0, 0, 0);
  }
  for (; s0 < s_end; s0 += W) {
    const int64_t off = (int64_t)s0 * 32;
    const u32x4 wa = gload16(wrow + off);
#pragma unroll
    for (int u = 0; u < TT; ++u)
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8s(wa), as_v8s(gload16(xrow[u] + off)), acc[u], 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < TT; ++u) s_part[wave][u][lane] = acc[u];
  __syncthreads();
  float* out = a.partial + (int64_t)slice * a.T * a.E;
  for (int idx = threadIdx.x; idx < TT * 64 * 4; idx += 64 * W) {
    const int u = idx >> 8, l = (idx >> 2) & 63, i = idx & 3;
    const float v = ((s_part[0][u][l][i] + s_part[1][u][l][i]) + s_part[2][u][l][i]) + s_part[3][u][l][i];
    const int er = e0 + 4 * (l >> 4) + i, tc = t0 + 16 * u + (l & 15);
    if (er < a.E && tc < a.T) out[(int64_t)tc * a.E + er] = v;
  }
}

// Order-preserving key: for non-NaN floats, a < b  <=>  key(a) < key(b), and +0 and -0
// (equal as floats) share one key.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f == 0.f ? 0.f : f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

// One token per 64-thread workgroup: the tokens spread over as many CUs as there are
// tokens (measured on MI355X against four per workgroup: 17.2 against 18.2 us per gate
// call at 128 tokens, 10.5 against 11.1 at 8).  NS is a power of two >= ks.
template <int NS>
__global__ __launch_bounds__(64) void k_topk(TopkArgs a) {
  __shared__ uint32_t s_key[MOE_MAX_TOPK];
  __shared__ int s_id[MOE_MAX_TOPK];
  __shared__ float s_val[MOE_MAX_TOPK];
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  const float* z = a.logits + (int64_t)t * a.E;
  const int64_t slice_stride = (int64_t)a.T * a.E;
  float v[4];
  uint32_t key[4];
  // every partial sum's load is issued before the first addition, with no branch between
  // them: slices past ks - 1 read slice ks - 1 again and columns past E read column E - 1,
  // and both are dropped (a load under a per-slice branch made the compiler wait for each
  // one before issuing the next).  The sums are then taken in slice order.
  float part[4][NS];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = min(lane + 64 * j, a.E - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) part[j][s] = z[min(s, a.ks - 1) * slice_stride + e];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    float zz = part[j][0];
#pragma unroll
    for (int s = 1; s < NS; ++s)
      if (s < a.ks) zz += part[j][s];
    if (e < a.E && a.logits_out) a.logits_out[(int64_t)t * a.E + e] = zz;
    v[j] = e < a.E ? zz : 0.f;
    key[j] = e < a.E ? order_key(zz) : 0u;  // below every real logit's key (k <= E)
  }
  // thr = the largest key with at least k keys >= it, i.e. the k-th largest key
  uint32_t thr = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = thr | (1u << b);
    int n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) n += wave_count(key[j] >= c);
    if (n >= a.k) thr = c;
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) gt += wave_count(key[j] > thr);
  // keys equal to thr fill the remaining k - gt places in expert-id order (j, then lane)
  int eq_left = a.k - gt, slot = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t meq = __ballot(key[j] == thr);
    const int before_eq = __popcll(meq & below);
    const bool sel = key[j] > thr || (key[j] == thr && before_eq < eq_left);
    const uint64_t msel = __ballot(sel);
    if (sel) {
      const int p = slot + __popcll(msel & below);
      s_key[p] = key[j];
      s_id[p] = lane + 64 * j;
      s_val[p] = v[j];
    }
    slot += __popcll(msel);
    eq_left -= min(eq_left, __popcll(meq));
  }
  __syncthreads();
  if (lane < a.k) {
    const uint32_t mk = s_key[lane];
    const int mid = s_id[lane];
    const float mv = s_val[lane];
    int rank = 0;
    float zmax = -INFINITY;
    for (int p = 0; p < a.k; ++p) {
      const uint32_t ok = s_key[p];
      rank += ok > mk || (ok == mk && s_id[p] < mid);
      zmax = fmaxf(zmax, s_val[p]);
    }
    float sum = 0.f;
    for (int p = 0; p < a.k; ++p) sum += expf(s_val[p] - zmax);
    a.ids[(int64_t)t * a.k + rank] = mid;
    a.w[(int64_t)t * a.k + rank] = expf(mv - zmax) / sum;
  }
}

constexpr int kRlRows = 64;                 // tokens, and experts, per workgroup
constexpr int kRlK = 128;                   // K elements per staged chunk
constexpr int kRlStride = kRlK * 2 + 16;    // bytes per staged row
constexpr int kRlPieces = kRlRows * kRlK * 2 / 16 / 256;  // 16-byte pieces per thread and operand
struct RlSmem {
  uint8_t x[2][kRlRows * kRlStride];
  uint8_t w[2][kRlRows * kRlStride];
};

// partial[slice][t][e] over K chunks [nch * slice / ks, nch * (slice + 1) / ks) (nch = H / 128).
__global__ __launch_bounds__(256) void k_router_lds(RouterSplitArgs a) {
  __shared__ __align__(16) RlSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  // XCD x takes a contiguous run of workgroups, expert blocks fastest, so that a token
  // block's rows are fetched into one XCD's L2 for all its expert blocks
  const int gx = gridDim.x, gy = gridDim.y;
  const int n = gx * gy * gridDim.z, b = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int xcd = b & 7, per = n >> 3, extra = n & 7;
  const int L = xcd * per + min(xcd, extra) + (b >> 3);
  const int eb = L % gx, rest = L / gx;
  const int e0 = eb * kRlRows, t0 = (rest % gy) * kRlRows, slice = rest / gy;
  const int nch = a.H / kRlK;
  const int c_begin = (int)((int64_t)nch * slice / a.ks), c_end = (int)((int64_t)nch * (slice + 1) / a.ks);
  // this thread's pieces: piece q = tid + 256 i is 16 bytes at column 16 (q % 16) of row q / 16
  const uint16_t* xs[kRlPieces];
  const uint16_t* ws[kRlPieces];
  int so[kRlPieces];
#pragma unroll
  for (int i = 0; i < kRlPieces; ++i) {
    const int q = tid + 256 * i, row = q >> 4, col = q & 15;
    xs[i] = a.x + (int64_t)min(t0 + row, a.T - 1) * a.H + 8 * col;
    ws[i] = a.wr + (int64_t)min(e0 + row, a.E - 1) * a.H + 8 * col;
    so[i] = row * kRlStride + 16 * col;
  }
  // two register sets of staged pieces: chunk j of the slice (j >= 1) travels in set j & 1
  u32x4 xv[2][kRlPieces], wv[2][kRlPieces];
  auto load = [&](int set, int j) {
    const int64_t off = (int64_t)(c_begin + j) * kRlK;
#pragma unroll
    for (int i = 0; i < kRlPieces; ++i) {
      xv[set][i] = gload16(xs[i] + off);
      wv[set][i] = gload16(ws[i] + off);
    }
  };
  auto store = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < kRlPieces; ++i) {
      *reinterpret_cast<u32x4*>(sm.x[buf] + so[i]) = xv[set][i];
      *reinterpret_cast<u32x4*>(sm.w[buf] + so[i]) = wv[set][i];
    }
  };
  const int wm = wave >> 1, wn = wave & 1;  // token half, expert half
  v4f acc[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[j][u] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
    const uint8_t* xb = sm.x[buf] + (wm * 32 + r16) * kRlStride + 16 * g4;
    const uint8_t* wb = sm.w[buf] + (wn * 32 + r16) * kRlStride + 16 * g4;
#pragma unroll
    for (int s = 0; s < kRlK / 32; ++s) {
      u32x4 fa[2], fb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) fa[j] = *reinterpret_cast<const u32x4*>(wb + j * 16 * kRlStride + 64 * s);
#pragma unroll
      for (int u = 0; u < 2; ++u) fb[u] = *reinterpret_cast<const u32x4*>(xb + u * 16 * kRlStride + 64 * s);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[j][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8s(fa[j]), as_v8s(fb[u]), acc[j][u], 0, 0, 0);
    }
  };
  const int nc = c_end - c_begin;
  if (nc >= 5) {
    // chunks two ahead: at step j, LDS buffer j & 1 holds chunk j, set (j + 1) & 1 chunk
    // j + 1 (stored after this step's MFMAs) and set j & 1 chunk j + 2 (in flight); the
    // freed set then takes chunk j + 3.  No condition around a load inside the loop: the
    // last four steps are peeled.
    load(0, 0);
    store(0, 0);
    __syncthreads();
    load(1, 1);
    load(0, 2);
    auto step = [&](int j, int set) {  // set = (j + 1) & 1
      compute(j & 1);
      __builtin_amdgcn_sched_barrier(0);
      store(set, (j + 1) & 1);
      __syncthreads();
    };
    int j = 0;
    for (; j + 4 < nc; j += 2) {
      step(j, 1);
      load(1, j + 3);
      __builtin_amdgcn_sched_barrier(0);  // the loads right after the barrier
      step(j + 1, 0);
      load(0, j + 4);
      __builtin_amdgcn_sched_barrier(0);
    }
    // j is even; the steps j .. nc - 1 remain (1 to 4 of them), chunk j + 3 still to load
    // when it exists
    const int r = nc - j;
    if (r == 4) {
      step(j, 1);
      load(1, j + 3);
      step(j + 1, 0);
      step(j + 2, 1);
      compute((j + 3) & 1);
    } else if (r == 3) {
      step(j, 1);
      step(j + 1, 0);
      compute((j + 2) & 1);
    } else if (r == 2) {
      step(j, 1);
      compute((j + 1) & 1);
    } else {
      compute(j & 1);
    }
  } else if (nc > 0) {
    // a few chunks: one ahead
    load(0, 0);
    store(0, 0);
    __syncthreads();
    for (int j = 0; j < nc; ++j) {
      if (j + 1 < nc) load(1, j + 1);
      compute(j & 1);
      if (j + 1 < nc) {
        store(1, (j + 1) & 1);
        __syncthreads();
      }
    }
  }
  float* out = a.partial + (int64_t)slice * a.T * a.E;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int er = e0 + wn * 32 + 16 * j + 4 * g4 + i, tc = t0 + wm * 32 + 16 * u + r16;
        if (er < a.E && tc < a.T) out[(int64_t)tc * a.E + er] = acc[j][u][i];
      }
}

}  // namespace

// The LDS-tiled router from this many tokens on (H a multiple of 128).
constexpr int kRouterLdsMinT = 256;
static bool router_lds(int T, int H) { return T >= kRouterLdsMinT && H % kRlK == 0; }
static int rl_tiles(int T, int E) { return ((E + kRlRows - 1) / kRlRows) * ((T + kRlRows - 1) / kRlRows); }

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
  if (router_lds(a.T, a.H)) {
    const RouterSplitArgs r{a.x, a.wr, a.logits, a.T, a.H, a.E, 1};
    hipLaunchKernelGGL(k_router_lds, dim3((a.E + kRlRows - 1) / kRlRows, (a.T + kRlRows - 1) / kRlRows, 1), dim3(256),
                       0, st, r);
    return hipGetLastError();
  }
  // Enough workgroups to cover the CUs with 16-token tiles when T is small; wider token
  // tiles cut the L2 re-reads of the router weights once there are tokens to spare.
  const int eb = (a.E + 15) / 16;
  if ((int64_t)eb * ((a.T + 63) / 64) >= 256)
    hipLaunchKernelGGL((k_router<4, 8, 6>), dim3(eb, (a.T + 63) / 64), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((k_router<1, 16, 7>), dim3(eb, (a.T + 15) / 16), dim3(1024), 0, st, a);
  return hipGetLastError();
}

int gate_split(int T, int H, int E) {
  if (router_lds(T, H)) {
    // about 256 workgroups, within the no-allocation scratch (ks x T x E fp32 partial
    // sums, 4 MiB: ks x T <= 4096 at 256 experts)
    const int want = (256 + rl_tiles(T, E) - 1) / rl_tiles(T, E);
    return std::max(1, std::min({want, 4096 / T, kGateMaxSplit, H / kRlK}));
  }
  // Token tiles of up to 128 tokens; split K until about 256 workgroups are in flight, with
  // at least 8 K steps (two per wave) in every slice.  Measured on MI355X (H 7168, 256
  // experts, gate call in us), against every fixed split of 1-16: the rule's choice is the
  // fastest or within 0.1 us of it from 1 to 4096 tokens (e.g. 8.6 at 8 tokens, 11.1 at
  // 64, 13.6 at 128, 39.3 at 1024); aiming at 384-1024 workgroups instead (up to 28
  // slices) was slower at every size (15.8 us at 128 tokens, 9.6 at 8).
  const int tiles = ((E + 15) / 16) * ((T + 127) / 128);
  const int ks = (256 + tiles - 1) / tiles;
  return std::max(1, std::min({ks, kGateMaxSplit, H / 256}));
}

hipError_t launch_router_split(const RouterSplitArgs& a, hipStream_t st) {
  if (router_lds(a.T, a.H)) {
    hipLaunchKernelGGL(k_router_lds, dim3((a.E + kRlRows - 1) / kRlRows, (a.T + kRlRows - 1) / kRlRows, a.ks),
                       dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const int eb = (a.E + 15) / 16;
  if (a.T > 64)
    hipLaunchKernelGGL((k_router_split<8, 3>), dim3(eb, (a.T + 127) / 128, a.ks), dim3(256), 0, st, a);
  else if (a.T > 32)
    hipLaunchKernelGGL((k_router_split<4, 5>), dim3(eb, 1, a.ks), dim3(256), 0, st, a);
  else if (a.T > 16)
    hipLaunchKernelGGL((k_router_split<2, 8>), dim3(eb, 1, a.ks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_router_split<1, 8>), dim3(eb, 1, a.ks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  static_assert(kGateMaxSplit == 16, "k_topk is instantiated for up to 16 slices");
  if (a.ks <= 1)
    hipLaunchKernelGGL(k_topk<1>, dim3(a.T), dim3(64), 0, st, a);
  else if (a.ks <= 2)
    hipLaunchKernelGGL(k_topk<2>, dim3(a.T), dim3(64), 0, st, a);
  else if (a.ks <= 4)
    hipLaunchKernelGGL(k_topk<4>, dim3(a.T), dim3(64), 0, st, a);
  else if (a.ks <= 8)
    hipLaunchKernelGGL(k_topk<8>, dim3(a.T), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(k_topk<16>, dim3(a.T), dim3(64), 0, st, a);
  return hipGetLastError();
}
