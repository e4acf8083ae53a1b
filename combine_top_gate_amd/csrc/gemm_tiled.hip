// Grouped GEMMs for large expert row counts (prefill): FP8 e4m3 x FP8 with 128x128
// weight scales and 1x128 token scales, tiled through LDS on gfx950 MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4.  Same arithmetic as the decode kernels
// (gemm_lowp.hip): GEMM1 + SwiGLU + 1x128 e4m3 requantisation, then GEMM2 to bf16
// ("GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4 Grouped GEMM via
// CUDA Green Contexts", full text), over windows read in place.
//
// With hundreds to thousands of rows per expert the layer is bound by MFMA, not by the
// weight stream, so both operands are reused from LDS: a workgroup computes a tile of
// 128 token rows x 256 weight rows; per 128-deep K slab it stages the token slab
// (16 KB) and the weight slab (32 KB) in LDS (double buffered, loads for slab k+1 in
// flight while slab k is multiplied), and each of its 8 waves multiplies 64 tokens x
// 64 weight rows (16 MFMAs per slab), promoting every MFMA result with
// (weight scale x token scale).  GEMM1's 256 weight rows are 128 gate + the matching
// 128 up rows, so SwiGLU and the per-128-column requantisation stay in the epilogue.
//
// Experts' loads are uneven (skewed routing), so work is a flat list of
// (expert, 128-row token tile, column block) items built on the device from the row
// counts (k_plan) and handed out by an atomic counter to a persistent grid: a
// workgroup that finishes early takes the next item, whichever expert it belongs to.
#include "kernels.h"
#include "pack_layout.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define GLOBAL __attribute__((address_space(1)))

constexpr int BM = 128;            // token rows per tile
constexpr int BN = 256;            // weight rows per tile
constexpr int kThreads = 512;      // 8 waves: 2 (token halves) x 4 (weight quarters)
constexpr int kStride = 144;       // LDS bytes per staged 128-byte row (+16 against bank conflicts)
constexpr int kAPieces = BM * 8;   // 16-byte pieces of a token slab
constexpr int kWPieces = BN * 8;   // 16-byte pieces of a weight slab
constexpr int kALd = kAPieces / kThreads;  // 2
constexpr int kWLd = kWPieces / kThreads;  // 4

__device__ __forceinline__ u32x4 gload16(const uint8_t* p) { return *(const GLOBAL u32x4*)p; }
__device__ __forceinline__ float gloadf(const float* p) { return *(const GLOBAL float*)p; }

struct Tiles {
  uint8_t a[2][BM * kStride];
  uint8_t w[2][BN * kStride];
  float sx[2][BM];          // token scales of the staged slab
  float sw[2][2];           // weight scales of the staged slab (two 128-row blocks)
  float amax[4][BM];        // GEMM1: per weight quarter, per token row
  int pre[MOE_MAX_SRC + 1]; // expert row segments (see gemm_lowp.hip SegTable)
  int row0[MOE_MAX_SRC];
  int item;
};

// k_plan: per group g, tiles[g] = ceil(rows/BM); item prefix for GEMM1 and GEMM2.
// plan layout: [0] total GEMM1 items, [1] total GEMM2 items, [2 + g] GEMM1 item start
// of group g, [2 + 260 + g] GEMM2 item start, [2 + 520 + g] rows of g; [522 + 260] the
// two work counters (zeroed here for the launches that follow).
constexpr int kPlanG1 = 2, kPlanG2 = 2 + 260, kPlanRows = 2 + 520, kPlanCtr = 2 + 780;

__global__ __launch_bounds__(256) void k_plan(TiledArgs t) {
  const BatchDims& d = t.g1.d;
  __shared__ int s_rows[MOE_MAX_EXPERTS + 1];
  const int nG = d.E + (d.Ish ? 1 : 0);
  for (int g = threadIdx.x; g < nG; g += blockDim.x) {
    int M = 0;
    if (g < d.E)
      for (int s = 0; s < d.S; ++s) M += t.g1.cnt[s * d.E + g];
    else
      M = d.T;
    s_rows[g] = M;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a1 = 0, a2 = 0;
    for (int g = 0; g < nG; ++g) {
      const int tiles = (s_rows[g] + BM - 1) / BM;
      t.plan[kPlanG1 + g] = a1;
      t.plan[kPlanG2 + g] = a2;
      t.plan[kPlanRows + g] = s_rows[g];
      a1 += tiles * (g < d.E ? t.nb1_r : t.nb1_s);
      a2 += tiles * t.nb2;
    }
    t.plan[kPlanG1 + nG] = a1;
    t.plan[kPlanG2 + nG] = a2;
    t.plan[0] = a1;
    t.plan[1] = a2;
    t.plan[kPlanCtr] = 0;
    t.plan[kPlanCtr + 1] = 0;
  }
}

__device__ __forceinline__ void segments(const GemmArgs& p, int g, Tiles& T) {
  const BatchDims& d = p.d;
  if (threadIdx.x < 64 && g < d.E) {
    const int s = threadIdx.x;
    const int c = s < d.S ? p.cnt[s * d.E + g] : 0;
    const int o = s < d.S ? p.off[s * d.E + g] : 0;
    int inc = c;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
      const int y = __shfl_up(inc, k, 64);
      if (s >= k) inc += y;
    }
    if (s < d.S) {
      T.pre[s] = inc - c;
      T.row0[s] = s * d.T_s * d.k + o;
    }
  }
}

__device__ __forceinline__ int seg_row(const Tiles& T, int S, int m) {
  int s = 0;
  while (s + 1 < S && m >= T.pre[s + 1]) ++s;
  return T.row0[s] + (m - T.pre[s]);
}

// One item: token tile [m0, m0 + BM) of group g (M rows), weight block nb.
template <bool GEMM1>
__device__ void tile_item(const GemmArgs& p, int g, int M, int m0, int nb, Tiles& T, bool t_packed) {
  const BatchDims& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;  // token half, weight quarter
  const bool shared = g == d.E;
  const int inter = shared ? d.Ish : d.I;
  const int K = GEMM1 ? d.H : inter;
  const int KB = K >> 7;
  const int seg = d.T_s * d.k;
  (void)seg;

  // ---- where this thread's slab pieces come from
  const uint8_t* asrc[kALd];
  const float* tscp = nullptr;
  int adst[kALd];
#pragma unroll
  for (int i = 0; i < kALd; ++i) {
    const int q = tid + kThreads * i;
    const int r = q >> 3;               // tile row
    const int m = min(m0 + r, M - 1);   // rows past the end repeat the last one (not stored)
    const uint8_t* rowp;
    if (GEMM1 && shared) {
      const int s = m / d.T_s, tt = m - s * d.T_s;
      rowp = p.src.x[s] + (int64_t)tt * d.H;
    } else {
      const int wr = shared ? d.R + m : seg_row(T, d.S, m);
      rowp = p.a + (int64_t)wr * (GEMM1 ? d.H : d.hstride);
    }
    asrc[i] = rowp + (q & 7) * 16;
    adst[i] = r * kStride + (q & 7) * 16;
  }
  if (tid < BM) {
    const int m = min(m0 + tid, M - 1);
    if (GEMM1 && shared) {
      const int s = m / d.T_s, tt = m - s * d.T_s;
      tscp = p.src.xs[s] + (int64_t)tt * (d.H >> 7);
    } else {
      const int wr = shared ? d.R + m : seg_row(T, d.S, m);
      tscp = p.as + (int64_t)wr * ((GEMM1 ? d.H : d.hstride) >> 7);
    }
  }
  const uint8_t* W = shared ? p.w_sh : p.w + (int64_t)g * p.w_stride;
  const float* WS = static_cast<const float*>(shared ? p.ws_sh : p.ws) + (shared ? 0 : (int64_t)g * p.ws_stride);
  // weight slab pieces: row-major rows, or the same bytes in the packed streaming order
  // (pack_layout.h), where slab kb of a row block is one 8 KB run per wave
  const uint8_t* wsrc[kWLd];
  int wdst[kWLd];
  const int64_t wstep = t_packed ? 8192 : 128;
#pragma unroll
  for (int i = 0; i < kWLd; ++i) {
    const int q = tid + kThreads * i;
    const int r = q >> 3;  // 0..255
    if (t_packed) {
      int wv, mt, rr;
      if (GEMM1) {
        const int ro = r & 127;
        wv = ro >> 5;
        mt = (r >= 128 ? 2 : 0) + ((ro >> 4) & 1);
        rr = ro & 15;
      } else {
        const int rc = min(r, d.H - 1 - nb * BN);
        wv = rc >> 6;
        mt = (rc >> 4) & 3;
        rr = rc & 15;
      }
      const int h = (q & 7) >> 2, gq = q & 3;
      wsrc[i] = W + pack_w_offset(MOE_FP8_E4M3, K, nb, wv, 0) + (mt * 2 + h) * 1024 + (gq * 16 + rr) * 16;
    } else {
      int wrow;
      if (GEMM1)
        wrow = (r < 128 ? 0 : inter) + nb * 128 + (r & 127);
      else
        wrow = min(nb * BN + r, d.H - 1);
      wsrc[i] = W + (int64_t)wrow * K + (q & 7) * 16;
    }
    wdst[i] = r * kStride + (q & 7) * 16;
  }
  // weight scale rows of the tile's two 128-row blocks
  const float* ws0 = WS + (int64_t)(GEMM1 ? nb : min(2 * nb, (d.H >> 7) - 1)) * KB;
  const float* ws1 = WS + (int64_t)(GEMM1 ? (inter >> 7) + nb : min(2 * nb + 1, (d.H >> 7) - 1)) * KB;

  u32x4 ra[kALd], rw[kWLd];
  float rsx = 0.f, rsw = 0.f;
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < kALd; ++i) ra[i] = gload16(asrc[i] + (int64_t)kb * 128);
#pragma unroll
    for (int i = 0; i < kWLd; ++i) rw[i] = gload16(wsrc[i] + (int64_t)kb * wstep);
    if (tid < BM) rsx = gloadf(tscp + kb);
    if (tid >= BM && tid < BM + 2) rsw = gloadf((tid == BM ? ws0 : ws1) + kb);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kALd; ++i) *reinterpret_cast<u32x4*>(&T.a[buf][adst[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < kWLd; ++i) *reinterpret_cast<u32x4*>(&T.w[buf][wdst[i]]) = rw[i];
    if (tid < BM) T.sx[buf][tid] = rsx;
    if (tid >= BM && tid < BM + 2) T.sw[buf][tid - BM] = rsw;
  };

  // this wave: token tiles wm*64 + 16*tt (tt = 0..3); weight tiles (GEMM1) gate rows
  // wn*32 + 16*j and up rows 128 + wn*32 + 16*j (j = 0, 1); (GEMM2) rows wn*64 + 16*j
  int wrows[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wrows[j] = GEMM1 ? ((j >> 1) * 128 + wn * 32 + 16 * (j & 1)) : (wn * 64 + 16 * j);
  const int wsel = GEMM1 ? -1 : (wn >> 1);  // GEMM2: this wave's 64 rows lie in block wn/2

  v4f acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[j][tt] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < KB) gload(kb + 1);
    v8i wv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* ap = &T.w[buf][(wrows[j] + r16) * kStride + 16 * g4];
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(ap);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(ap + 64);
      wv[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
    float swj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) swj[j] = T.sw[buf][GEMM1 ? (j >> 1) : wsel];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int trow = wm * 64 + 16 * tt + r16;
      const uint8_t* bp = &T.a[buf][trow * kStride + 16 * g4];
      const u32x4 y0 = *reinterpret_cast<const u32x4*>(bp);
      const u32x4 y1 = *reinterpret_cast<const u32x4*>(bp + 64);
      const v8i bv = {(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
      const float sx = T.sx[buf][trow];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wv[j], bv, v4f{0.f, 0.f, 0.f, 0.f}, MFMA_FMT_FP8, MFMA_FMT_FP8, 0, E8M0_ONE, 0, E8M0_ONE);
        const float sc = swj[j] * sx;
        acc[j][tt][0] = fmaf(r[0], sc, acc[j][tt][0]);
        acc[j][tt][1] = fmaf(r[1], sc, acc[j][tt][1]);
        acc[j][tt][2] = fmaf(r[2], sc, acc[j][tt][2]);
        acc[j][tt][3] = fmaf(r[3], sc, acc[j][tt][3]);
      }
    }
    if (kb + 1 < KB) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue; lane holds weight rows wrows[j] + 4*g4 + i of token wm*64 + 16*tt + r16
  if constexpr (GEMM1) {
    float hv[2][4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = silu(acc[j][tt][i]) * acc[2 + j][tt][i];
          hv[j][tt][i] = v;
          mx = fmaxf(mx, fabsf(v));
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (g4 == 0) T.amax[wn][wm * 64 + 16 * tt + r16] = mx;
    }
    __syncthreads();
    const int hsc_stride = d.hstride >> 7;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tr = wm * 64 + 16 * tt + r16;
      const int m = m0 + tr;
      if (m >= M) continue;
      const int orow = shared ? d.R + m : seg_row(T, d.S, m);
      const float amax = fmaxf(fmaxf(T.amax[0][tr], T.amax[1][tr]), fmaxf(T.amax[2][tr], T.amax[3][tr]));
      const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(hv[j][tt][i] / sc, -448.0f), 448.0f);
        *reinterpret_cast<uint32_t*>(p.h + (int64_t)orow * d.hstride + nb * 128 + wn * 32 + 16 * j + 4 * g4) =
            pack4_e4m3(q[0], q[1], q[2], q[3]);
      }
      if (wn == 0 && g4 == 0) p.hs[(int64_t)orow * hsc_stride + nb] = sc;
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int m = m0 + wm * 64 + 16 * tt + r16;
      if (m >= M) continue;
      const int orow = shared ? d.R + m : seg_row(T, d.S, m);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = nb * BN + wrows[j] + 4 * g4;
        if (n >= d.H) continue;
        const uint32_t lo = bf16_bits(acc[j][tt][0]) | (bf16_bits(acc[j][tt][1]) << 16);
        const uint32_t hi = bf16_bits(acc[j][tt][2]) | (bf16_bits(acc[j][tt][3]) << 16);
        *reinterpret_cast<uint2*>(p.y + (int64_t)orow * d.H + n) = make_uint2(lo, hi);
      }
    }
  }
}

// Persistent grid: items of one GEMM, handed out by an atomic counter.
template <bool GEMM1>
__global__ __launch_bounds__(kThreads, 1) void k_tiled(TiledArgs t) {
  __shared__ Tiles T;
  const GemmArgs& p = GEMM1 ? t.g1 : t.g2;
  const BatchDims& d = p.d;
  const int nG = d.E + (d.Ish ? 1 : 0);
  const int* start = t.plan + (GEMM1 ? kPlanG1 : kPlanG2);
  const int total = t.plan[GEMM1 ? 0 : 1];
  int* ctr = t.plan + kPlanCtr + (GEMM1 ? 0 : 1);
  for (;;) {
    if (threadIdx.x == 0) T.item = atomicAdd(ctr, 1);
    __syncthreads();
    const int i = T.item;
    if (i >= total) break;  // uniform
    int g = 0;
    while (g + 1 < nG && i >= start[g + 1]) ++g;
    const int nbg = GEMM1 ? (g < d.E ? t.nb1_r : t.nb1_s) : t.nb2;
    const int j = i - start[g];
    const int tm = j / nbg, nb = j - tm * nbg;
    const int M = t.plan[kPlanRows + g];
    segments(p, g, T);
    __syncthreads();
    tile_item<GEMM1>(p, g, M, tm * BM, nb, T, t.packed != 0);
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_tiled(const TiledArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tiled<true>, dim3(grid), dim3(kThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_tiled<false>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

int tiled_plan_words() { return kPlanCtr + 2; }
