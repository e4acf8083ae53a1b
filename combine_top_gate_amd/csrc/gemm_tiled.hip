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
// per item height: TT 16-row token tiles per wave (kTT, or kTT / 2 for a half-height
// item of BM / 2 rows): token pieces per thread, waves loading token scales, DMAs per wave
template <int TT>
constexpr int kALdOf = TT * 32 * 8 / kThreads;
template <int TT>
constexpr int kSxWavesOf = TT * 32 / 64;
template <int TT>
constexpr int kLoadsOf = kALdOf<TT> + kWLd + 1;
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

// Memory -> LDS without registers: lane l of the wave writes its 16 (4) bytes at LDS
// address dst + 16 l (4 l), dst wave-uniform; counted by vmcnt like any load.  Issued from
// assembly: the compiler cannot tell which LDS stage such a load fills, and if it knew
// of them it would wait for every one in flight (later stages included) before any
// LDS read.  It does not need to know: the data is read only after wait7_barrier() /
// wait0_barrier(), whose memory clobbers also keep every LDS access on its side.
// No register is written, so nothing of the load is left to land in a register.  M0
// (the LDS base, read when the load issues) is saved and restored around it, with the
// wait state an LDS-DMA needs after an M0 write.
__device__ __forceinline__ void dma16(const void* src, uint32_t dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}
// The same from a wave-uniform base (scalar registers) plus this lane's 32-bit offset:
// lane l reads base + voff(l).  (No instruction offset: an LDS-DMA adds it to the LDS
// address as well.)
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t dst) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(m)
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
  Segs seg;                 // expert row segments of the item being set up
  int rows[2][BM];          // row table of the current and the next item (row_table)
  SrcPtrs src;              // GEMM1: the source buffers (the shared expert's rows), copied
                            // once, so that a row's buffer is an LDS read, not a load
  int pstart[MOE_MAX_EXPERTS + 2];  // this GEMM's plan: first super-tile of each group,
  int prows[MOE_MAX_EXPERTS + 1];   // and its rows (copied once from the plan buffer)
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
// then 1 KB where epilogue lanes without an output store (see kEpiStores)
constexpr int kPlanTrash = (kPlanCtr + 2 * kXcds + 15) / 16 * 16, kTrashWords = 256;

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

// The rows of token tile [m0, m0 + BM) of group g (M rows), one per tile row, built once
// per item by the workgroup (then an LDS read wherever a row is needed): the window row
// (GEMM2: the h row; the shared expert's are R + m), or for GEMM1's shared expert the
// token index m.  Rows past M repeat the last one (their loads are harmless, their
// results never stored).  Ends with a barrier.
template <bool GEMM1>
__device__ __forceinline__ void row_table(const GemmArgs& p, int g, int M, int m0, const Segs& sg, int* rows) {
  const BatchDims& d = p.d;
  for (int r = threadIdx.x; r < BM; r += kThreads) {
    const int m = min(m0 + r, M - 1);
    rows[r] = g == d.E ? (GEMM1 ? m : d.R + m) : seg_row(sg, d.S, m);
  }
  __syncthreads();
}

typedef float v16f __attribute__((ext_vector_type(16)));

// This thread's DMA sources for one work item (token tile [m0, m0 + BM) of group g with M
// rows, weight block nb).  Instruction i of wave w fills the 1 KB at 16 * ((w * n + i) * 64
// + lane) of a stage buffer: chunk p = (w * n + i) * 64 + lane is physical chunk p % 8 of
// row p / 8, which holds that row's logical chunk (p % 8) ^ ((row >> 1) & 7) (the swizzle
// of swz()).
// PK (packed weights): every DMA of a wave's weight pieces reads one run at consecutive
// 1 KB blocks, so one wave-uniform base (scalar registers) replaces per-lane pointers.
static_assert(8 % kWLd == 0, "a wave's weight pieces lie in one packed run");
template <bool PK>
struct TileSrc {
  const uint8_t* a[kALd];
  const uint8_t* w[PK ? 1 : kWLd];
  const float* s;
};

__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <bool GEMM1, bool PK, int TT = kTT>
__device__ __forceinline__ TileSrc<PK> make_src(const GemmArgs& p, int g, int nb, const int* rows, const Tiles& T) {
  constexpr int nA = kALdOf<TT>;
  const BatchDims& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool shared = g == d.E;
  const int inter = shared ? d.Ish : d.I;
  const int K = GEMM1 ? d.H : inter;
  const int KB = K >> 7;
  TileSrc<PK> src;
#pragma unroll
  for (int i = 0; i < nA; ++i) {
    const int q = (wave * nA + i) * 64 + lane;
    const int r = q >> 3;
    const int c = (q & 7) ^ ((r >> 1) & 7);
    const int wr = rows[r];
    const uint8_t* rowp;
    if (GEMM1 && shared) {
      const int s = wr / d.T_s, tt = wr - s * d.T_s;  // token index -> its source buffer
      rowp = T.src.x[s] + (int64_t)tt * d.H;
    } else {
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
  if constexpr (PK) {
    const int bi = wave * kWLd;  // 1 KB block bi of the slab: block bi % 8 of run bi / 8
    src.w[0] = uniform_ptr(W + pack_w_offset(MOE_FP8_E4M3, K, nb, bi >> 3, 0) + (bi & 7) * 1024);
  } else {
#pragma unroll
  for (int i = 0; i < kWLd; ++i) {
    const int q = (wave * kWLd + i) * 64 + lane;
    const int r = q >> 3;  // 0..255
    const int c = (q & 7) ^ ((r >> 1) & 7);
    {
      int wrow;
      if (GEMM1)
        wrow = (r < 128 ? 0 : inter) + nb * 128 + (r & 127);
      else
        wrow = min(nb * BN + r, d.H - 1);
      src.w[i] = W + (int64_t)wrow * K + c * 16;
    }
  }
  }
  // scales, one 4-byte DMA per wave per slab (so every wave issues the same number of
  // loads per slab): waves w < kSxWaves the token scales of rows 64 w + lane, wave
  // kSxWaves in lanes 0-1 the weight scales of the tile's two 128-row blocks, the rest
  // into sdummy
  const float* ws0 = WS + (int64_t)(GEMM1 ? nb : min(2 * nb, (d.H >> 7) - 1)) * KB;
  const float* ws1 = WS + (int64_t)(GEMM1 ? (inter >> 7) + nb : min(2 * nb + 1, (d.H >> 7) - 1)) * KB;
  if (wave < kSxWavesOf<TT>) {
    const int wr = rows[64 * wave + lane];
    if (GEMM1 && shared) {
      const int s = wr / d.T_s, tt = wr - s * d.T_s;
      src.s = T.src.xs[s] + (int64_t)tt * (d.H >> 7);
    } else {
      src.s = p.as + (int64_t)wr * ((GEMM1 ? d.H : d.hstride) >> 7);
    }
  } else {
    src.s = lane == 1 ? ws1 : ws0;
  }
  return src;
}

// The DMAs of K slab kb into ring stage st (every wave issues kLoadsOf<TT> of them).
template <bool PK, int TT = kTT>
__device__ __forceinline__ void issue_slab(const TileSrc<PK>& src, int kb, int st, Tiles& T) {
  constexpr int nA = kALdOf<TT>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // LDS addresses as plain offsets from the tile buffers' base (uniform, scalar registers)
  const uint32_t t0 = __builtin_amdgcn_readfirstlane(lds_off(&T));
#pragma unroll
  for (int i = 0; i < nA; ++i)
    dma16(src.a[i] + (int64_t)kb * 128, t0 + offsetof(Tiles, a) + st * (BM * kStride) + (wave * nA + i) * 1024);
  const uint32_t wdst = t0 + offsetof(Tiles, w) + st * (BN * kStride) + wave * kWLd * 1024;
  if constexpr (PK) {
    const uint8_t* wb = src.w[0] + (int64_t)kb * 8192;  // uniform
    static_assert(kWLd == 4, "four 1 KB weight pieces per wave and slab");
#pragma unroll
    for (int i = 0; i < kWLd; ++i) dma16s(wb, i * 1024 + lane * 16, wdst + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < kWLd; ++i) dma16(src.w[i] + (int64_t)kb * 128, wdst + i * 1024);
  }
  const uint32_t sdst = wave < kSxWavesOf<TT> ? t0 + offsetof(Tiles, sx) + (st * BM + 64 * wave) * 4
                        : wave == kSxWaves ? t0 + offsetof(Tiles, sw) + st * 64 * 4
                                           : t0 + offsetof(Tiles, sdummy);
  dma4(src.s + kb, sdst);
}

// One item on 32x32x64 MFMAs (option): token tile [m0, m0 + BM) of group g (M rows),
// weight block nb, segments in T.seg; loads, K loop and epilogue in sequence.
template <bool GEMM1, bool PK>
__device__ void tile_item_m32(const GemmArgs& p, int g, int M, int m0, int nb, Tiles& T) {
  constexpr bool t_packed = PK;
  const BatchDims& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;  // token half, weight quarter
  const bool shared = g == d.E;
  const int inter = shared ? d.Ish : d.I;
  const int K = GEMM1 ? d.H : inter;
  const int KB = K >> 7;
  row_table<GEMM1>(p, g, M, m0, T.seg, T.rows[0]);
  const TileSrc<PK> src = make_src<GEMM1, PK>(p, g, nb, T.rows[0], T);
  auto issue = [&](int kb, int st) { issue_slab<PK>(src, kb, st, T); };

  const int wsel = GEMM1 ? -1 : (wn >> 1);  // GEMM2: this wave's 64 rows lie in block wn/2
  constexpr int D = kStages - 1;  // slabs in flight ahead of the one multiplied
  {
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
        const int orow = GEMM1 && shared ? d.R + T.rows[0][m - m0] : T.rows[0][m - m0];
        const float amax = fmaxf(fmaxf(T.amax[0][tr], T.amax[1][tr]), fmaxf(T.amax[2][tr], T.amax[3][tr]));
        const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
        const float inv = __builtin_amdgcn_rcpf(sc);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          float q[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) q[i] = e4m3_scaled(acc[0][tt][4 * i4 + i], inv);
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
        const int orow = GEMM1 && shared ? d.R + T.rows[0][m - m0] : T.rows[0][m - m0];
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
  }
}


// ---- the default K loop (16x16x128), with work items pipelined.  When an item's K loop
// ends, the ring is idle: the next item's first two slabs are issued into it before this
// item's epilogue runs, so their latency overlaps the epilogue, and the epilogue's stores
// drain while the next K loop runs.  Vector-memory stores count in the same in-order
// counter (vmcnt) as the slab loads, so the next K loop must know how many stores follow
// its first slabs: every lane of every wave stores in each of the epilogue's store
// instructions (a lane without an output writes to a scratch area of the plan buffer),
// and they are issued from assembly, so that the compiler neither skips nor merges any.
template <bool GEMM1>
constexpr int kEpiStores = GEMM1 ? 3 * kTT : 4 * kTT;  // GEMM1: h (2 per token tile) + scale

template <int OFF = 0>
__device__ __forceinline__ void store32(void* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off offset:%2" ::"v"(p), "v"(v), "n"(OFF) : "memory");
}
template <int OFF = 0>
__device__ __forceinline__ void store64(void* p, uint64_t v) {
  asm volatile("global_store_dwordx2 %0, %1, off offset:%2" ::"v"(p), "v"(v), "n"(OFF) : "memory");
}
// LDS-only workgroup barrier (leaves the memory loads and stores in flight)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct Item {
  int g, M, m0, nb;
};

// The next work item from the per-XCD queues (see k_tiled), or false when every queue is
// exhausted.  Uniform over the workgroup; uses T.item and two barriers per queue entry.
template <bool GEMM1>
__device__ bool next_item(const TiledArgs& t, Tiles& T, int& q, int& left, Item& it) {
  const GemmArgs& p = GEMM1 ? t.g1 : t.g2;
  const BatchDims& d = p.d;
  const int nG = d.E + (d.Ish ? 1 : 0);
  const int n_sup = t.plan[GEMM1 ? 0 : 1];
  int* ctr = t.plan + kPlanCtr + (GEMM1 ? 0 : kXcds);
  while (left > 0) {
    if (threadIdx.x == 0) T.item = atomicAdd(ctr + q, 1);
    __syncthreads();
    const int k = __builtin_amdgcn_readfirstlane(T.item);
    __syncthreads();  // T.item is rewritten by the next round
    const int sup = q + kXcds * (k / kSlots), slot = k % kSlots;
    if (sup >= n_sup) {  // this queue is exhausted (uniform): move on to the next
      q = (q + 1) % kXcds;
      --left;
      continue;
    }
    // the group of super-tile sup: the last g with pstart[g] <= sup (groups without
    // super-tiles share their successor's start)
    int lo = 0, hi = nG - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (T.pstart[mid] <= sup) lo = mid; else hi = mid - 1;
    }
    const int g = __builtin_amdgcn_readfirstlane(lo);
    const int nbg = GEMM1 ? (g < d.E ? t.nb1_r : t.nb1_s) : t.nb2;
    const int ncb = (nbg + kSTN - 1) / kSTN;  // column super-blocks of g
    const int j = sup - T.pstart[g];
    const int tm = (j / ncb) * kSTM + slot / kSTN, nb = (j % ncb) * kSTN + slot % kSTN;
    const int M = __builtin_amdgcn_readfirstlane(T.prows[g]);
    if (tm * BM >= M || nb >= nbg) continue;  // an empty slot (uniform)
    // uniform values, held in scalar registers (the K loop needs every vector register)
    it = Item{g, M, __builtin_amdgcn_readfirstlane(tm * BM), __builtin_amdgcn_readfirstlane(nb)};
    return true;
  }
  return false;
}

// This GEMM's plan into LDS (read by next_item after its first barrier).
template <bool GEMM1>
__device__ __forceinline__ void load_plan(const TiledArgs& t, Tiles& T) {
  const BatchDims& d = (GEMM1 ? t.g1 : t.g2).d;
  const int nG = d.E + (d.Ish ? 1 : 0);
  const int* start = t.plan + (GEMM1 ? kPlanG1 : kPlanG2);
  for (int g = threadIdx.x; g <= nG; g += kThreads) {
    T.pstart[g] = start[g];
    if (g < nG) T.prows[g] = t.plan[kPlanRows + g];
  }
}

template <bool GEMM1>
__device__ __forceinline__ int item_kb(const GemmArgs& p, int g) {
  return (GEMM1 ? p.d.H : (g == p.d.E ? p.d.Ish : p.d.I)) >> 7;
}

// Issues an item's slab 0 into stage 0 and (when it has more) slab 1 into stage 1; the
// ring must be idle.
template <bool GEMM1, bool PK, int TT>
__device__ __forceinline__ void issue_first(const GemmArgs& p, const Item& it, const int* rows, Tiles& T) {
  const TileSrc<PK> src = make_src<GEMM1, PK, TT>(p, it.g, it.nb, rows, T);
  issue_slab<PK, TT>(src, 0, 0, T);
  if (item_kb<GEMM1>(p, it.g) > 1) issue_slab<PK, TT>(src, 1, 1, T);
}

// This wave's weight tiles: (GEMM1) gate rows wn*32 + 16*j and up rows 128 + wn*32 +
// 16*j (j = 0, 1); (GEMM2) rows wn*64 + 16*j.  Its token tiles: wm*16*TT + 16*tt (TT tiles per wave).
template <bool GEMM1>
__device__ __forceinline__ int wave_row(int wn, int j) {
  return GEMM1 ? ((j >> 1) * 128 + wn * 32 + 16 * (j & 1)) : (wn * 64 + 16 * j);
}

// acc[j][tt] = sum over K slabs of the MFMA result times (weight scale x token scale).
// On entry slab 0 (stage 0) and, if KB > 1, slab 1 (stage 1) are in flight, followed by
// exactly kEpiStores<GEMM1> stores of this wave (the previous item's epilogue, or
// placeholders before the first item).  From step 1 on, step kb issues slab kb + 1 into
// the stage read at step kb - 1.  Steps 0 and 1 are written out, so that every wait
// count is a constant and the loop itself is one uniform body.
template <bool GEMM1, bool PK, int TT>
__device__ __forceinline__ void kloop16(v4f (&acc)[4][TT], const TileSrc<PK>& src, Tiles& T, int KB) {
  constexpr bool t_packed = PK;
  constexpr int TR = 16 * TT;  // token rows per wave
  constexpr int S = kEpiStores<GEMM1>;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;
  const int wsel = GEMM1 ? -1 : (wn >> 1);  // GEMM2: this wave's 64 rows lie in block wn/2
  // Fragment offsets: tiles lie 16 or 128 rows apart, which leaves the swizzle term
  // (r >> 1) & 7 unchanged, so every fragment is a base (two registers per operand)
  // plus a constant the LDS instructions take as an immediate.
  const int r0 = wave_row<GEMM1>(wn, 0);
  const int w0 = t_packed ? wn * 8192 + lane * 16 : swz(r0 + r16, g4);
  const int w1 = t_packed ? w0 + 1024 : swz(r0 + r16, g4 + 4);
  const int a0 = swz(wm * TR + r16, g4), a1 = swz(wm * TR + r16, g4 + 4);
  auto wfrag_off = [&](int j, int h) {  // weight tile j, half h
    const int base = h ? w1 : w0;
    return t_packed ? base + 2 * j * 1024 : base + (wave_row<GEMM1>(wn, j) - r0) * kStride;
  };
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[j][tt] = v4f{0.f, 0.f, 0.f, 0.f};

  // LDS reads through an LDS-space pointer: per-lane offsets plus constants the LDS
  // instructions take as immediates
  const LDS_AS uint8_t* L = (const LDS_AS uint8_t*)(const uint8_t*)(&T);
  const int sxo = (wm * TR + r16) * 4;
  auto compute = [&](int st) {
    const LDS_AS uint8_t* ws_ = L + offsetof(Tiles, w) + st * (BN * kStride);
    const LDS_AS uint8_t* as_ = L + offsetof(Tiles, a) + st * (BM * kStride);
    const LDS_AS uint8_t* sx_ = L + offsetof(Tiles, sx) + st * (BM * 4) + sxo;
    const LDS_AS float* sw_ = reinterpret_cast<const LDS_AS float*>(L + offsetof(Tiles, sw) + st * 64 * 4);
    // the first token tile's fragments, then the weight fragments in the order the
    // MFMAs use them, so that the first MFMA waits for four reads, not ten
    u32x4 x0 = *reinterpret_cast<const LDS_AS u32x4*>(as_ + a0);
    u32x4 x1 = *reinterpret_cast<const LDS_AS u32x4*>(as_ + a1);
    u32x4 wf[8];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      wf[i] = *reinterpret_cast<const LDS_AS u32x4*>(ws_ + wfrag_off(i >> 1, i & 1));
      if (i == 1 || i == 3) __builtin_amdgcn_sched_barrier(0);
    }
    const float swj[2] = {sw_[0], sw_[1]};
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const v8i bv = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      const float sx = *reinterpret_cast<const LDS_AS float*>(sx_ + 64 * tt);
      if (tt + 1 < TT) {
        x0 = *reinterpret_cast<const LDS_AS u32x4*>(as_ + a0 + (tt + 1) * 16 * kStride);
        x1 = *reinterpret_cast<const LDS_AS u32x4*>(as_ + a1 + (tt + 1) * 16 * kStride);
      }
      auto mfma = [&](int j) {
        const v8i wv = {(int)wf[2 * j].x, (int)wf[2 * j].y, (int)wf[2 * j].z, (int)wf[2 * j].w,
                        (int)wf[2 * j + 1].x, (int)wf[2 * j + 1].y, (int)wf[2 * j + 1].z, (int)wf[2 * j + 1].w};
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, bv, v4f{0.f, 0.f, 0.f, 0.f}, MFMA_FMT_FP8,
                                                                MFMA_FMT_FP8, 0, E8M0_ONE, 0, E8M0_ONE);
      };
      auto promote = [&](int j, const v4f& r) {
        const float sc = swj[GEMM1 ? (j >> 1) : wsel] * sx;
        acc[j][tt][0] = fmaf(r[0], sc, acc[j][tt][0]);
        acc[j][tt][1] = fmaf(r[1], sc, acc[j][tt][1]);
        acc[j][tt][2] = fmaf(r[2], sc, acc[j][tt][2]);
        acc[j][tt][3] = fmaf(r[3], sc, acc[j][tt][3]);
      };
      // two MFMA results in flight: a promotion reads one while the next MFMA runs
      v4f r0 = mfma(0), r1 = mfma(1);
      promote(0, r0);
      r0 = mfma(2);
      promote(1, r1);
      r1 = mfma(3);
      promote(2, r0);
      promote(3, r1);
      // keep that order (MFMA, MFMA, a promotion with its scale product, ...)
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
  };
  // each wait: this wave's loads of the slab have landed (what was issued after it may
  // stay in flight), then the barrier: every wave's have
  if (KB > 1)
    wait_barrier<kLoadsOf<TT> + S>();
  else
    wait_barrier<S>();
  compute(0);
  if (KB == 1) return;
  wait_barrier<S>();
  if (KB > 2) issue_slab<PK, TT>(src, 2, 0, T);
  compute(1);
  for (int kb = 2; kb < KB; ++kb) {
    wait_barrier<0>();
    if (kb + 1 < KB) issue_slab<PK, TT>(src, kb + 1, (kb + 1) & 1, T);
    compute(kb & 1);
  }
}

// The kEpiStores<GEMM1> placeholder stores that stand in for an epilogue's before the
// first item's K loop.
template <bool GEMM1>
__device__ __forceinline__ void placeholder_stores(int* plan) {
  uint8_t* trash = reinterpret_cast<uint8_t*>(plan + kPlanTrash) + 8 * (threadIdx.x & 63);
#pragma unroll
  for (int i = 0; i < kEpiStores<GEMM1>; ++i) store32(trash, 0u);
}

// The epilogue of an item: exactly kEpiStores<GEMM1> store instructions per wave.  Lane
// (g4, r16) holds weight rows wave_row(wn, j) + 4*g4 + i of token wm*16*TT + 16*tt + r16.
template <bool GEMM1, int TT>
__device__ __forceinline__ void epilogue16(const GemmArgs& p, const Item& it, const int* rows, v4f (&acc)[4][TT],
                                           Tiles& T, int* plan) {
  constexpr int TR = 16 * TT;  // token rows per wave
  const BatchDims& d = p.d;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;
  // lanes without an output store here (1 KB: lane offsets up to 504 plus store offsets)
  uint8_t* trash = reinterpret_cast<uint8_t*>(plan + kPlanTrash) + 8 * lane;
  const bool shared = it.g == d.E;
  if constexpr (GEMM1) {
    // SwiGLU in place: acc[j] (gate, j = 0, 1) becomes h; acc[2 + j] (up) is then dead
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
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
      if (g4 == 0) T.amax[wn][wm * TR + 16 * tt + r16] = mx;
    }
    lds_barrier();
    const int hsc_stride = d.hstride >> 7;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int tr = wm * TR + 16 * tt + r16;
      const bool ok = it.m0 + tr < it.M;
      const int orow = shared ? d.R + rows[tr] : rows[tr];
      const float amax = fmaxf(fmaxf(T.amax[0][tr], T.amax[1][tr]), fmaxf(T.amax[2][tr], T.amax[3][tr]));
      const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
      const float inv = __builtin_amdgcn_rcpf(sc);
      uint32_t code[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = e4m3_scaled(acc[j][tt][i], inv);
        code[j] = pack4_e4m3(q[0], q[1], q[2], q[3]);
      }
      // this lane's h columns nb*128 + wn*32 + 16 j + 4 g4 .. + 3 (j = 0, 1: 16 bytes apart)
      uint8_t* hp = ok ? p.h + (int64_t)orow * d.hstride + it.nb * 128 + wn * 32 + 4 * g4 : trash;
      store32<0>(hp, code[0]);
      store32<16>(hp, code[1]);
      uint8_t* sp = ok && wn == 0 && g4 == 0 ? reinterpret_cast<uint8_t*>(p.hs + (int64_t)orow * hsc_stride + it.nb)
                                             : trash;
      store32<0>(sp, __float_as_uint(sc));
    }
    // a half-height item's stores are padded to the full count
#pragma unroll
    for (int i = 0; i < 3 * (kTT - TT); ++i) store32(trash, 0u);
  } else {
    // this wave's 64 columns are all inside H or all past it (H is a multiple of 128)
    const bool col_ok = it.nb * BN + wn * 64 < d.H;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int tr = wm * TR + 16 * tt + r16;
      const bool ok = col_ok && it.m0 + tr < it.M;
      // columns nb*BN + wn*64 + 16 j + 4 g4 .. + 3 (j = 0..3: 32 bytes apart)
      uint8_t* yp = ok ? reinterpret_cast<uint8_t*>(p.y + (int64_t)rows[tr] * d.H + it.nb * BN + wn * 64 + 4 * g4)
                       : trash;
      uint64_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = pack2_bf16(acc[j][tt][0], acc[j][tt][1]) | ((uint64_t)pack2_bf16(acc[j][tt][2], acc[j][tt][3]) << 32);
      store64<0>(yp, v[0]);
      store64<32>(yp, v[1]);
      store64<64>(yp, v[2]);
      store64<96>(yp, v[3]);
    }
#pragma unroll
    for (int i = 0; i < 4 * (kTT - TT); ++i) store32(trash, 0u);
  }
}

// An item whose token tile holds at most BM / 2 rows (an expert's ragged last tile) runs
// half-height: its rows split over all eight waves (64 each, TT = kTT / 2), so that it
// takes about half a full item's time instead of leaving half the waves' MFMAs idle.
__device__ __forceinline__ bool half_item(const Item& it) { return it.M - it.m0 <= BM / 2; }

// One item of the persistent loop, TT token tiles per wave: its K loop, then the next
// item from the queues, whose row table is built and first two slabs issued before this
// item's epilogue.  Returns false (after the epilogue) when the queues are exhausted.
template <bool GEMM1, bool PK, int TT>
__device__ __forceinline__ bool step16(const TiledArgs& t, Tiles& T, int& q, int& left, Item& it, int& sb) {
  const GemmArgs& p = GEMM1 ? t.g1 : t.g2;
  v4f acc[4][TT];
  {
    const TileSrc<PK> src = make_src<GEMM1, PK, TT>(p, it.g, it.nb, T.rows[sb], T);
    kloop16<GEMM1, PK, TT>(acc, src, T, item_kb<GEMM1>(p, it.g));
  }
  Item nx;
  // its barriers also end every wave's reads of the ring
  const bool more = next_item<GEMM1>(t, T, q, left, nx);
  if (more) {
    segments(p, nx.g, T.seg);
    __syncthreads();
    row_table<GEMM1>(p, nx.g, nx.M, nx.m0, T.seg, T.rows[sb ^ 1]);
    if (half_item(nx))
      issue_first<GEMM1, PK, kTT / 2>(p, nx, T.rows[sb ^ 1], T);
    else
      issue_first<GEMM1, PK, kTT>(p, nx, T.rows[sb ^ 1], T);
  }
  epilogue16<GEMM1, TT>(p, it, T.rows[sb], acc, T, t.plan);
  if (more) {
    it = nx;
    sb ^= 1;
  }
  return more;
}

// The persistent loop of the default path.
template <bool GEMM1, bool PK>
__device__ void run16(const TiledArgs& t, Tiles& T) {
  const GemmArgs& p = GEMM1 ? t.g1 : t.g2;
  int q = blockIdx.x % kXcds, left = kXcds;
  Item it;
  if (!next_item<GEMM1>(t, T, q, left, it)) return;
  int sb = 0;  // T.rows[sb]: the current item's row table
  segments(p, it.g, T.seg);
  __syncthreads();
  row_table<GEMM1>(p, it.g, it.M, it.m0, T.seg, T.rows[sb]);
  if (half_item(it))
    issue_first<GEMM1, PK, kTT / 2>(p, it, T.rows[sb], T);
  else
    issue_first<GEMM1, PK, kTT>(p, it, T.rows[sb], T);
  placeholder_stores<GEMM1>(t.plan);
  for (;;) {
    const bool more = half_item(it) ? step16<GEMM1, PK, kTT / 2>(t, T, q, left, it, sb)
                                    : step16<GEMM1, PK, kTT>(t, T, q, left, it, sb);
    if (!more) break;
  }
}

// Persistent grid: the items of one GEMM from the per-XCD queues.  Queue x holds
// super-tiles x, x + 8, ...; its counter k names slot k % 32 of its (k / 32)-th one.
// Workgroup b runs on XCD b % 8 (the GPU's round-robin placement; any other placement
// only costs locality).  Slots past an expert's last token tile or column block are
// empty.  A workgroup leaves when every queue is exhausted.
template <bool GEMM1, bool M32, bool PK>
__global__ __launch_bounds__(kThreads, 1) void k_tiled(TiledArgs t) {
  __shared__ Tiles T;
  if (GEMM1 && threadIdx.x < MOE_MAX_SRC) {
    T.src.x[threadIdx.x] = t.g1.src.x[threadIdx.x];
    T.src.xs[threadIdx.x] = t.g1.src.xs[threadIdx.x];
  }
  load_plan<GEMM1>(t, T);  // both published by next_item's first barrier
  if constexpr (!M32) {
    run16<GEMM1, PK>(t, T);
  } else {
    const GemmArgs& p = GEMM1 ? t.g1 : t.g2;
    int q = blockIdx.x % kXcds, left = kXcds;
    Item it;
    while (next_item<GEMM1>(t, T, q, left, it)) {
      segments(p, it.g, T.seg);
      __syncthreads();
      tile_item_m32<GEMM1, PK>(p, it.g, it.M, it.m0, it.nb, T);
      __syncthreads();
    }
  }
}

template <bool GEMM1>
hipError_t launch_one(const TiledArgs& a, int grid, hipStream_t st) {
  const dim3 g(grid), b(kThreads);
  if (a.m32 && a.packed)
    hipLaunchKernelGGL((k_tiled<GEMM1, true, true>), g, b, 0, st, a);
  else if (a.m32)
    hipLaunchKernelGGL((k_tiled<GEMM1, true, false>), g, b, 0, st, a);
  else if (a.packed)
    hipLaunchKernelGGL((k_tiled<GEMM1, false, true>), g, b, 0, st, a);
  else
    hipLaunchKernelGGL((k_tiled<GEMM1, false, false>), g, b, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tiled(const TiledArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_one<true>(a, grid, st)) != hipSuccess) return e;
  return launch_one<false>(a, grid, st);
}

int tiled_plan_words() { return kPlanTrash + kTrashWords; }
