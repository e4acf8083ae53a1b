// Grouped GEMMs for large expert row counts (prefill): FP8 e4m3 x FP8 with 128x128
// weight scales and 1x128 token scales, tiled through LDS on gfx950 MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4.  Same arithmetic as the decode kernels
// (gemm_lowp.hip): GEMM1 + SwiGLU + 1x128 e4m3 requantisation, then GEMM2 to bf16
// ("GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4 Grouped GEMM via
// CUDA Green Contexts", full text), over windows read in place.
//
// With hundreds to thousands of rows per expert the layer is bound by MFMA, not by the
// weight stream, so both operands are reused from LDS: a workgroup computes a tile of
// 256 token rows x 256 weight rows; per 128-deep K slab it stages the token slab
// (32 KB), the weight slab (32 KB) and their scales in LDS, and each of its 8 waves
// multiplies 128 tokens x 64 weight rows (32 MFMAs per slab), promoting every MFMA
// result with (weight scale x token scale).  The slabs go from memory straight into
// a ring of two LDS stages (global_load_lds), the next slab in flight while one is
// multiplied, with no staging registers; one barrier per slab.  GEMM1's 256 weight
// rows are 128 gate + the matching 128 up rows, so SwiGLU and the per-128-column
// requantisation stay in the epilogue.
//
// Work items are (expert, 256-row token tile, column block), grouped into super-tiles
// of 4 token tiles x 8 column blocks of one expert, built on the device from the row
// counts (k_plan).  An XCD's 32 CUs work on one super-tile at a time, so its token
// tiles and weight blocks are read once into that XCD's L2 and reused 8 and 4 times.  Each XCD has
// its own queue of super-tiles (every 8th one), served by an atomic counter to a
// persistent grid; when its queue is empty, a workgroup takes items from the next
// XCD's queue, so skewed expert loads still balance across the GPU.
#include "kernels.h"
#include "pack_layout.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define GLOBAL __attribute__((address_space(1)))

constexpr int BM = 256;            // token rows per tile
constexpr int BN = 256;            // weight rows per tile
constexpr int kThreads = 512;      // 8 waves: 2 (token halves) x 4 (weight quarters)
constexpr int kTT = BM / 32;       // 16-row token tiles per wave (each wave: BM/2 tokens x 64 weights)
constexpr int kStride = 128;       // LDS bytes per staged 128-byte row (16-byte chunks swizzled)
constexpr int kAPieces = BM * 8;   // 16-byte pieces of a token slab
constexpr int kWPieces = BN * 8;   // 16-byte pieces of a weight slab
constexpr int kALd = kAPieces / kThreads;  // 16-byte token pieces per thread per slab
constexpr int kWLd = kWPieces / kThreads;  // 16-byte weight pieces per thread per slab
constexpr int kSxWaves = BM / 64;          // waves that load the token scales
constexpr int kLoadsPerSlab = kALd + kWLd + 1;
static_assert(kSxWaves < kThreads / 64, "a wave is left for the weight scales");

__device__ __forceinline__ u32x4 gload16(const uint8_t* p) { return *(const GLOBAL u32x4*)p; }
__device__ __forceinline__ float gloadf(const float* p) { return *(const GLOBAL float*)p; }

// Staged rows keep their eight 16-byte chunks in swizzled order: chunk c of row r sits at
// chunk c ^ ((r >> 1) & 7).  A B-operand read (16 consecutive rows, one chunk) then
// touches 16 distinct groups of 4 banks, and a store of two rows (16 lanes) fills the
// two halves of the 64 banks: both conflict-free.
__device__ __forceinline__ int swz(int r, int c) { return r * kStride + ((c ^ ((r >> 1) & 7)) << 4); }

#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ uint32_t lds_off(const void* p) { return (uint32_t)(uintptr_t)(const LDS_AS uint8_t*)p; }

// Memory -> LDS without registers: lane l of the wave writes its 16 (4) bytes at
// dst + 16 l (4 l), dst wave-uniform; counted by vmcnt like any load.  Issued from
// assembly: the compiler cannot tell which LDS stage such a load fills, and if it knew
// of them it would wait for every one in flight (later stages included) before any
// LDS read.  It does not need to know: the data is read only after wait7_barrier() /
// wait0_barrier(), whose memory clobbers also keep every LDS access on its side.
// No register is written, so nothing of the load is left to land in a register.  M0
// (the LDS base, read when the load issues) is saved and restored around it, with the
// wait state an LDS-DMA needs after an M0 write.
__device__ __forceinline__ void dma16(const void* src, const void* dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_off(dst));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}
__device__ __forceinline__ void dma4(const void* src, const void* dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_off(dst));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}
// Wait until at most N of this wave's memory loads are in flight, then the workgroup
// barrier, in one block: __syncthreads() would also wait for every pending
// memory-to-LDS load, and a bare barrier intrinsic would let the compiler move memory
// operations across it.  The memory clobber keeps both orders.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}



constexpr int kStages = 2;  // LDS ring depth: loads run kStages - 1 slabs ahead

// Where an expert's rows live: source s's bucket holds rows pre[s] .. pre[s+1]-1 of the
// expert window, starting at window row row0[s] (see gemm_lowp.hip SegTable).
struct Segs {
  int pre[MOE_MAX_SRC + 1];
  int row0[MOE_MAX_SRC];
};

struct __align__(16) Tiles {
  uint8_t a[kStages][BM * kStride];
  uint8_t w[kStages][BN * kStride];
  float sx[kStages][BM];    // token scales of the staged slab
  float sw[kStages][64];    // weight scales of the staged slab (two 128-row blocks) in [0..1]
  float sdummy[64];         // where the idle lanes' scale loads go
  float amax[4][BM];        // GEMM1: per weight quarter, per token row
  Segs seg[2];              // expert row segments of the current and the next item
  int item;
};

constexpr int kSTM = 4, kSTN = 8;  // super-tile: token tiles x column blocks
constexpr int kSlots = kSTM * kSTN;
constexpr int kXcds = 8;

// k_plan: per group g, tiles = ceil(rows/BM) token tiles, and its super-tiles for GEMM1
// and GEMM2.  plan layout: [0] GEMM1 super-tiles, [1] GEMM2 super-tiles, [2 + g]
// first GEMM1 super-tile of group g, [2 + 260 + g] first GEMM2 super-tile, [2 + 520 +
// g] rows of g; from [2 + 780] the 8 GEMM1 and 8 GEMM2 queue counters (zeroed here for
// the launches that follow).
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
      const int stm = (s_rows[g] + BM * kSTM - 1) / (BM * kSTM);
      t.plan[kPlanG1 + g] = a1;
      t.plan[kPlanG2 + g] = a2;
      t.plan[kPlanRows + g] = s_rows[g];
      a1 += stm * (((g < d.E ? t.nb1_r : t.nb1_s) + kSTN - 1) / kSTN);
      a2 += stm * ((t.nb2 + kSTN - 1) / kSTN);
    }
    t.plan[kPlanG1 + nG] = a1;
    t.plan[kPlanG2 + nG] = a2;
    t.plan[0] = a1;
    t.plan[1] = a2;
  }
  if (threadIdx.x < 2 * kXcds) t.plan[kPlanCtr + threadIdx.x] = 0;
}

__device__ __forceinline__ void segments(const GemmArgs& p, int g, Segs& T) {
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

__device__ __forceinline__ int seg_row(const Segs& T, int S, int m) {
  int s = 0;
  while (s + 1 < S && m >= T.pre[s + 1]) ++s;
  return T.row0[s] + (m - T.pre[s]);
}

typedef float v16f __attribute__((ext_vector_type(16)));

// One item: token tile [m0, m0 + BM) of group g (M rows), weight block nb.  M32: the K
// loop on v_mfma_scale_f32_32x32x64_f8f6f4 instead of 16x16x128 (see below).
// This thread's DMA sources for one work item (token tile [m0, m0 + BM) of group g with M
// rows, weight block nb).  Instruction i of wave w fills the 1 KB at 16 * ((w * n + i) * 64
// + lane) of a stage buffer: chunk p = (w * n + i) * 64 + lane is physical chunk p % 8 of
// row p / 8, which holds that row's logical chunk (p % 8) ^ ((row >> 1) & 7) (the swizzle
// of swz()).
struct TileSrc {
  const uint8_t* a[kALd];
  const uint8_t* w[kWLd];
  const float* s;
  int64_t wstep;
};

template <bool GEMM1>
__device__ __forceinline__ TileSrc make_src(const GemmArgs& p, int g, int M, int m0, int nb, const Segs& sg,
                                            bool t_packed) {
  const BatchDims& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool shared = g == d.E;
  const int inter = shared ? d.Ish : d.I;
  const int K = GEMM1 ? d.H : inter;
  const int KB = K >> 7;
  TileSrc src;
#pragma unroll
  for (int i = 0; i < kALd; ++i) {
    const int q = (wave * kALd + i) * 64 + lane;
    const int r = q >> 3;
    const int c = (q & 7) ^ ((r >> 1) & 7);
    const int m = min(m0 + r, M - 1);   // rows past the end repeat the last one (not stored)
    const uint8_t* rowp;
    if (GEMM1 && shared) {
      const int s = m / d.T_s, tt = m - s * d.T_s;
      rowp = p.src.x[s] + (int64_t)tt * d.H;
    } else {
      const int wr = shared ? d.R + m : seg_row(sg, d.S, m);
      rowp = p.a + (int64_t)wr * (GEMM1 ? d.H : d.hstride);
    }
    src.a[i] = rowp + c * 16;
  }
  const uint8_t* W = shared ? p.w_sh : p.w + (int64_t)g * p.w_stride;
  const float* WS = static_cast<const float*>(shared ? p.ws_sh : p.ws) + (shared ? 0 : (int64_t)g * p.ws_stride);
  // weight slab pieces.  Packed (pack_layout.h): slab kb of the tile is four 8 KB runs,
  // run v = the rows of tiled wave v (GEMM1: gate rows nb*128 + 32v + 0/16 and the
  // matching up rows; GEMM2: rows nb*256 + 64v + 16 mt), each already in MFMA operand
  // order [tile mt][half h][lane][16 B].  They are copied as they are, 1 KB per
  // instruction, and read back at (run, mt, h, lane).  Row-major: rows in the swizzled
  // layout of the tokens.  (Packed rows past a ragged end of H are the layout's
  // padding: read, never stored.)
  src.wstep = t_packed ? 8192 : 128;
#pragma unroll
  for (int i = 0; i < kWLd; ++i) {
    const int q = (wave * kWLd + i) * 64 + lane;
    const int r = q >> 3;  // 0..255
    const int c = (q & 7) ^ ((r >> 1) & 7);
    if (t_packed) {
      const int bi = wave * kWLd + i;  // 1 KB block bi of the slab: block bi % 8 of run bi / 8
      src.w[i] = W + pack_w_offset(MOE_FP8_E4M3, K, nb, bi >> 3, 0) + (bi & 7) * 1024 + lane * 16;
    } else {
      int wrow;
      if (GEMM1)
        wrow = (r < 128 ? 0 : inter) + nb * 128 + (r & 127);
      else
        wrow = min(nb * BN + r, d.H - 1);
      src.w[i] = W + (int64_t)wrow * K + c * 16;
    }
  }
  // scales, one 4-byte DMA per wave per slab (so every wave issues the same number of
  // loads per slab): waves w < kSxWaves the token scales of rows 64 w + lane, wave
  // kSxWaves in lanes 0-1 the weight scales of the tile's two 128-row blocks, the rest
  // into sdummy
  const float* ws0 = WS + (int64_t)(GEMM1 ? nb : min(2 * nb, (d.H >> 7) - 1)) * KB;
  const float* ws1 = WS + (int64_t)(GEMM1 ? (inter >> 7) + nb : min(2 * nb + 1, (d.H >> 7) - 1)) * KB;
  if (wave < kSxWaves) {
    const int m = min(m0 + 64 * wave + lane, M - 1);
    if (GEMM1 && shared) {
      const int s = m / d.T_s, tt = m - s * d.T_s;
      src.s = p.src.xs[s] + (int64_t)tt * (d.H >> 7);
    } else {
      const int wr = shared ? d.R + m : seg_row(sg, d.S, m);
      src.s = p.as + (int64_t)wr * ((GEMM1 ? d.H : d.hstride) >> 7);
    }
  } else {
    src.s = lane == 1 ? ws1 : ws0;
  }
  return src;
}

// The DMAs of K slab kb into ring stage st (every wave issues kLoadsPerSlab of them).
__device__ __forceinline__ void issue_slab(const TileSrc& src, int kb, int st, Tiles& T) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kALd; ++i) dma16(src.a[i] + (int64_t)kb * 128, &T.a[st][(wave * kALd + i) * 1024]);
#pragma unroll
  for (int i = 0; i < kWLd; ++i) dma16(src.w[i] + (int64_t)kb * src.wstep, &T.w[st][(wave * kWLd + i) * 1024]);
  float* sdst = wave < kSxWaves ? &T.sx[st][64 * wave] : (wave == kSxWaves ? &T.sw[st][0] : &T.sdummy[0]);
  dma4(src.s + kb, sdst);
}

template <bool GEMM1, bool M32>
__device__ void tile_item(const GemmArgs& p, int g, int M, int m0, int nb, Tiles& T, bool t_packed) {
  const BatchDims& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;  // token half, weight quarter
  const bool shared = g == d.E;
  const int inter = shared ? d.Ish : d.I;
  const int K = GEMM1 ? d.H : inter;
  const int KB = K >> 7;
  const TileSrc src = make_src<GEMM1>(p, g, M, m0, nb, T.seg[0], t_packed);
  auto issue = [&](int kb, int st) { issue_slab(src, kb, st, T); };

  const int wsel = GEMM1 ? -1 : (wn >> 1);  // GEMM2: this wave's 64 rows lie in block wn/2
  constexpr int D = kStages - 1;  // slabs in flight ahead of the one multiplied
  if constexpr (M32) {
    // 32x32x64 MFMAs.  This wave's 64 weight rows are 2 tiles of 32 (GEMM1: gate rows
    // wn*32 + r and up rows 128 + wn*32 + r; GEMM2: rows wn*64 + 32 j + r) and its 128
    // token rows 4 tiles of 32 (wm*128 + 32 tt + r).  Operand lane l holds row (column)
    // l % 32 and, of the slab's half h (64 k), k = 64 h + 32 (l / 32) + 0..31: the 16-byte
    // chunks 4 h + 2 (l / 32) and + 1 of its 128-byte row (the same k order on both
    // sides, so the contraction is right whatever order the instruction sums in).  Result
    // lane l, register i: weight row 8 (i / 4) + 4 (l / 32) + i % 4 of the tile, token
    // l % 32 (measured on gfx950).  Per tile and slab the two halves chain in the matrix
    // core and one promotion follows; the accumulator is still 128 registers per lane,
    // and the freed result registers let one tile's promotion overlap the next tile's MFMAs.
    const int r32 = lane & 31, g2 = lane >> 5;
    // fragment offsets: tiles lie 32 or 128 rows apart (the swizzle term (r >> 1) & 7
    // unchanged), so each (half, part) is one base plus immediates
    int aoff[2][2], woff[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        aoff[h][q] = swz(wm * (BM / 2) + r32, 4 * h + 2 * g2 + q);
        woff[h][q] = t_packed ? wn * 8192 + (r32 >> 4) * 2048 + h * 1024 + ((2 * g2 + q) * 16 + (r32 & 15)) * 16
                              : swz((GEMM1 ? wn * 32 : wn * 64) + r32, 4 * h + 2 * g2 + q);
      }
    const int wstep = t_packed ? 2 * 2048 : (GEMM1 ? 128 : 32) * kStride;  // weight tile j -> j + 1
    v16f acc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][tt][i] = 0.f;
    __syncthreads();  // the previous item's last reads of the ring are done
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (i < KB) issue(i, i);
    for (int kb = 0; kb < KB; ++kb) {
      const int st = kb % kStages;
      if (D > 1 && kb + D - 1 < KB)
        wait_barrier<(D > 1 ? D - 1 : 0) * kLoadsPerSlab>();
      else
        wait_barrier<0>();
      if (kb + D < KB) issue(kb + D, (kb + D) % kStages);
      const uint8_t* ws_ = T.w[st];
      const uint8_t* as_ = T.a[st];
      v8i wv[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w0 = *reinterpret_cast<const u32x4*>(ws_ + woff[h][0] + j * wstep);
          const u32x4 w1 = *reinterpret_cast<const u32x4*>(ws_ + woff[h][1] + j * wstep);
          wv[j][h] = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
        }
      const float swj[2] = {T.sw[st][0], T.sw[st][1]};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        v8i bv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 x0 = *reinterpret_cast<const u32x4*>(as_ + aoff[h][0] + tt * 32 * kStride);
          const u32x4 x1 = *reinterpret_cast<const u32x4*>(as_ + aoff[h][1] + tt * 32 * kStride);
          bv[h] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
        const float sx = T.sx[st][wm * (BM / 2) + 32 * tt + r32];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          v16f r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv[j][0], bv[0], v16f{}, MFMA_FMT_FP8, MFMA_FMT_FP8,
                                                                   0, E8M0_ONE, 0, E8M0_ONE);
          r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv[j][1], bv[1], r, MFMA_FMT_FP8, MFMA_FMT_FP8, 0,
                                                              E8M0_ONE, 0, E8M0_ONE);
          const float sc = swj[GEMM1 ? j : wsel] * sx;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[j][tt][i] = fmaf(r[i], sc, acc[j][tt][i]);
        }
      }
    }
    // ---- epilogue; lane holds weight rows 8 (i / 4) + 4 g2 + i % 4 of tile j, token
    // wm*128 + 32 tt + r32
    if constexpr (GEMM1) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = silu(acc[0][tt][i]) * acc[1][tt][i];
          acc[0][tt][i] = v;
          mx = fmaxf(mx, fabsf(v));
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (g2 == 0) T.amax[wn][wm * (BM / 2) + 32 * tt + r32] = mx;
      }
      __syncthreads();
      const int hsc_stride = d.hstride >> 7;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int tr = wm * (BM / 2) + 32 * tt + r32;
        const int m = m0 + tr;
        if (m >= M) continue;
        const int orow = shared ? d.R + m : seg_row(T.seg[0], d.S, m);
        const float amax = fmaxf(fmaxf(T.amax[0][tr], T.amax[1][tr]), fmaxf(T.amax[2][tr], T.amax[3][tr]));
        const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          float q[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(acc[0][tt][4 * i4 + i] / sc, -448.0f), 448.0f);
          *reinterpret_cast<uint32_t*>(p.h + (int64_t)orow * d.hstride + nb * 128 + wn * 32 + 8 * i4 + 4 * g2) =
              pack4_e4m3(q[0], q[1], q[2], q[3]);
        }
        if (wn == 0 && g2 == 0) p.hs[(int64_t)orow * hsc_stride + nb] = sc;
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int m = m0 + wm * (BM / 2) + 32 * tt + r32;
        if (m >= M) continue;
        const int orow = shared ? d.R + m : seg_row(T.seg[0], d.S, m);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int n = nb * BN + wn * 64 + 32 * j + 8 * i4 + 4 * g2;
            if (n >= d.H) continue;
            const uint32_t lo = bf16_bits(acc[j][tt][4 * i4]) | (bf16_bits(acc[j][tt][4 * i4 + 1]) << 16);
            const uint32_t hi = bf16_bits(acc[j][tt][4 * i4 + 2]) | (bf16_bits(acc[j][tt][4 * i4 + 3]) << 16);
            *reinterpret_cast<uint2*>(p.y + (int64_t)orow * d.H + n) = make_uint2(lo, hi);
          }
      }
    }
    return;
  } else {
  // this wave: token tiles wm*(BM/2) + 16*tt (tt < kTT); weight tiles (GEMM1) gate rows
  // wn*32 + 16*j and up rows 128 + wn*32 + 16*j (j = 0, 1); (GEMM2) rows wn*64 + 16*j
  int wrows[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wrows[j] = GEMM1 ? ((j >> 1) * 128 + wn * 32 + 16 * (j & 1)) : (wn * 64 + 16 * j);
  // byte offsets (within a stage) of this lane's fragments
  // Fragment offsets: tiles lie 16 or 128 rows apart, which leaves the swizzle term
  // (r >> 1) & 7 unchanged, so every fragment is a base (two registers per operand)
  // plus a constant the LDS instructions take as an immediate.
  const int w0 = t_packed ? wn * 8192 + lane * 16 : swz(wrows[0] + r16, g4);
  const int w1 = t_packed ? w0 + 1024 : swz(wrows[0] + r16, g4 + 4);
  const int a0 = swz(wm * (BM / 2) + r16, g4), a1 = swz(wm * (BM / 2) + r16, g4 + 4);
  auto wfrag_off = [&](int j, int h) {  // weight tile j, half h
    const int base = h ? w1 : w0;
    return t_packed ? base + 2 * j * 1024 : base + (wrows[j] - wrows[0]) * kStride;
  };

  v4f acc[4][kTT];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) acc[j][tt] = v4f{0.f, 0.f, 0.f, 0.f};

  __syncthreads();  // the previous item's last reads of the ring are done
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < KB) issue(i, i);
  for (int kb = 0; kb < KB; ++kb) {
    const int st = kb % kStages;
    // this wave's loads of slab kb have landed (those of the D - 1 later slabs may stay
    // in flight), then every wave's; stage (kb + D) % kStages was last read at kb - 1
    if (D > 1 && kb + D - 1 < KB)
      wait_barrier<(D > 1 ? D - 1 : 0) * kLoadsPerSlab>();
    else
      wait_barrier<0>();
    if (kb + D < KB) issue(kb + D, (kb + D) % kStages);
    const uint8_t* ws_ = T.w[st];
    const uint8_t* as_ = T.a[st];
    u32x4 wf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wf[i] = *reinterpret_cast<const u32x4*>(ws_ + wfrag_off(i >> 1, i & 1));
    const float swj[2] = {T.sw[st][0], T.sw[st][1]};
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(as_ + a0 + tt * 16 * kStride);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(as_ + a1 + tt * 16 * kStride);
      const v8i bv = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      const float sx = T.sx[st][wm * (BM / 2) + 16 * tt + r16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8i wv = {(int)wf[2 * j].x, (int)wf[2 * j].y, (int)wf[2 * j].z, (int)wf[2 * j].w,
                        (int)wf[2 * j + 1].x, (int)wf[2 * j + 1].y, (int)wf[2 * j + 1].z, (int)wf[2 * j + 1].w};
        const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wv, bv, v4f{0.f, 0.f, 0.f, 0.f}, MFMA_FMT_FP8, MFMA_FMT_FP8, 0, E8M0_ONE, 0, E8M0_ONE);
        const float sc = swj[GEMM1 ? (j >> 1) : wsel] * sx;
        acc[j][tt][0] = fmaf(r[0], sc, acc[j][tt][0]);
        acc[j][tt][1] = fmaf(r[1], sc, acc[j][tt][1]);
        acc[j][tt][2] = fmaf(r[2], sc, acc[j][tt][2]);
        acc[j][tt][3] = fmaf(r[3], sc, acc[j][tt][3]);
      }
    }
  }

  // ---- epilogue; lane holds weight rows wrows[j] + 4*g4 + i of token wm*(BM/2) + 16*tt + r16
  if constexpr (GEMM1) {
    // SwiGLU in place: acc[j] (gate, j = 0, 1) becomes h; acc[2 + j] (up) is then dead
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = silu(acc[j][tt][i]) * acc[2 + j][tt][i];
          acc[j][tt][i] = v;
          mx = fmaxf(mx, fabsf(v));
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (g4 == 0) T.amax[wn][wm * (BM / 2) + 16 * tt + r16] = mx;
    }
    __syncthreads();
    const int hsc_stride = d.hstride >> 7;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      const int tr = wm * (BM / 2) + 16 * tt + r16;
      const int m = m0 + tr;
      if (m >= M) continue;
      const int orow = shared ? d.R + m : seg_row(T.seg[0], d.S, m);
      const float amax = fmaxf(fmaxf(T.amax[0][tr], T.amax[1][tr]), fmaxf(T.amax[2][tr], T.amax[3][tr]));
      const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(acc[j][tt][i] / sc, -448.0f), 448.0f);
        *reinterpret_cast<uint32_t*>(p.h + (int64_t)orow * d.hstride + nb * 128 + wn * 32 + 16 * j + 4 * g4) =
            pack4_e4m3(q[0], q[1], q[2], q[3]);
      }
      if (wn == 0 && g4 == 0) p.hs[(int64_t)orow * hsc_stride + nb] = sc;
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      const int m = m0 + wm * (BM / 2) + 16 * tt + r16;
      if (m >= M) continue;
      const int orow = shared ? d.R + m : seg_row(T.seg[0], d.S, m);
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
}

// Persistent grid: the items of one GEMM from the per-XCD queues.  Queue x holds
// super-tiles x, x + 8, ...; its counter k names slot k % 32 of its (k / 32)-th one.
// Workgroup b runs on XCD b % 8 (the GPU's round-robin placement; any other placement
// only costs locality).  Slots past an expert's last token tile or column block are
// empty.  A workgroup leaves when every queue is exhausted.
template <bool GEMM1, bool M32>
__global__ __launch_bounds__(kThreads, 1) void k_tiled(TiledArgs t) {
  __shared__ Tiles T;
  const GemmArgs& p = GEMM1 ? t.g1 : t.g2;
  const BatchDims& d = p.d;
  const int nG = d.E + (d.Ish ? 1 : 0);
  const int* start = t.plan + (GEMM1 ? kPlanG1 : kPlanG2);
  const int n_sup = t.plan[GEMM1 ? 0 : 1];
  int* ctr = t.plan + kPlanCtr + (GEMM1 ? 0 : kXcds);
  int q = blockIdx.x % kXcds;
  for (int left = kXcds; left > 0;) {
    if (threadIdx.x == 0) T.item = atomicAdd(ctr + q, 1);
    __syncthreads();
    const int k = T.item;
    __syncthreads();  // T.item is rewritten by the next round
    const int sup = q + kXcds * (k / kSlots), slot = k % kSlots;
    if (sup >= n_sup) {  // this queue is exhausted (uniform): move on to the next
      q = (q + 1) % kXcds;
      --left;
      continue;
    }
    int g = 0;
    while (g + 1 < nG && sup >= start[g + 1]) ++g;
    const int nbg = GEMM1 ? (g < d.E ? t.nb1_r : t.nb1_s) : t.nb2;
    const int ncb = (nbg + kSTN - 1) / kSTN;  // column super-blocks of g
    const int j = sup - start[g];
    const int tm = (j / ncb) * kSTM + slot / kSTN, nb = (j % ncb) * kSTN + slot % kSTN;
    const int M = t.plan[kPlanRows + g];
    if (tm * BM >= M || nb >= nbg) continue;  // an empty slot (uniform)
    segments(p, g, T.seg[0]);
    __syncthreads();
    tile_item<GEMM1, M32>(p, g, M, tm * BM, nb, T, t.packed != 0);
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_tiled(const TiledArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.m32)
    hipLaunchKernelGGL((k_tiled<true, true>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_tiled<true, false>), dim3(grid), dim3(kThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.m32)
    hipLaunchKernelGGL((k_tiled<false, true>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_tiled<false, false>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

int tiled_plan_words() { return kPlanCtr + 2 * kXcds; }
