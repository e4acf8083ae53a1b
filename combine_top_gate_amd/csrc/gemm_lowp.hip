// Grouped GEMMs over the expert windows, FP8 e4m3 activations x FP8 (128x128 block
// scales) or MXFP4 (e8m0 1x32 scales) weights, on gfx950 MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4; and the W4A16 variant (kFmtW4A16): bf16
// activations x MXFP4 weights decoded to bf16 in registers, on v_mfma_f32_16x16x32_bf16.
//
// GEMM1: a = x W13^T over the window rows of one expert, SwiGLU h = silu(gate) * up,
//        then h is requantised to e4m3 with one fp32 scale per 128 columns of a row
//        (W4A16: h is stored bf16).
// GEMM2: y = h W2^T, stored bf16.
// ("GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4 Grouped GEMM via
// CUDA Green Contexts", full text: block-scaled MMA with operand swap, fused SwiGLU,
// requantization, optional shared experts; "One-Sided Expert-Parallel All-to-All for
// Mixture-of-Experts Inference over NVLink", abstract: windows are read in place.)
//
// Decode shapes give an expert a few dozen rows against thousands of weight rows: the
// layer is bound by streaming the weights from HBM once.  So the weights go in the
// MFMA's 16-row A slot and the tokens in its 16-column B slot (operand swap), each
// wave owns 4 tiles of 16 weight rows and streams them K slab by K slab (128 deep)
// into registers, one slab ahead, and reads its token fragments straight from L2
// (an expert's rows are shared by the workgroups of that expert, which all run on one
// XCD).  Weight scales sit in lanes and token scales in LDS (staged once per pass), so
// the K loop's only memory operations are the slab loads, and it has no barrier.  One MFMA covers exactly
// one 128-wide scale block, so its fp32 result is promoted with (weight scale x token
// scale) before it is added to the accumulator.
//
// Weights come row-major or "packed" (moe_pack_weights): packed, each wave's weights
// are one contiguous stream in the order the wave consumes them, 1 KB per load
// instruction -- measured on MI355X, such streams read at ~6.9 TB/s against
// ~5.3-6.1 TB/s for 16 rows x 64 B per instruction.
//
// MFMA operand layout on gfx950 (16x16x128, measured): lane l serves row/column
// l%16; with g = l/16, an FP8 operand holds k = 16g..16g+15 in bytes 0..15 and
// k = 64+16g..64+16g+15 in bytes 16..31; an FP4 operand holds k = 32g..32g+31 as
// nibbles (element 2i in the low nibble of byte i) and lane l's e8m0 scale covers
// exactly those 32 k.  The result's lane l, register i is row 4g+i, column l%16.
#include <algorithm>

#include "dispatch_chunk.h"
#include "kernels.h"
#include "pack_layout.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define GLOBAL __attribute__((address_space(1)))

// Loads through the global address space (generic pointers would become flat loads,
// which also count against the LDS counter).
__device__ __forceinline__ u32x4 gload16(const uint8_t* p) { return *(const GLOBAL u32x4*)p; }
__device__ __forceinline__ u32x4 gload16_nt(const uint8_t* p) {
  return __builtin_nontemporal_load((const GLOBAL u32x4*)p);
}
__device__ __forceinline__ float gloadf(const float* p) { return *(const GLOBAL float*)p; }
__device__ __forceinline__ uint32_t gload32(const uint8_t* p) { return *(const GLOBAL uint32_t*)p; }
__device__ __forceinline__ uint32_t gload8(const uint8_t* p) { return *(const GLOBAL uint8_t*)p; }

// A kernel variant: weight storage and the activations' form.  kFmtW4A16 stores MXFP4
// weights like MOE_FP4_E2M1 but takes bf16 activations and keeps h in bf16.
template <int WFMT>
struct WeightFmt;
template <>
struct WeightFmt<MOE_FP8_E4M3> {
  static constexpr int kStore = MOE_FP8_E4M3;
  static constexpr int kLoads = 2;       // 16-byte loads per lane per 16-row tile per K slab
  static constexpr int kSlabBytes = 128; // bytes of one row per K slab
  static constexpr int kMfmaFmt = MFMA_FMT_FP8;
  static constexpr bool kA16 = false;    // activations (and h) bf16 instead of FP8 + 1x128 scales
};
template <>
struct WeightFmt<MOE_FP4_E2M1> {
  static constexpr int kStore = MOE_FP4_E2M1;
  static constexpr int kLoads = 1;
  static constexpr int kSlabBytes = 64;
  static constexpr int kMfmaFmt = MFMA_FMT_FP4;
  static constexpr bool kA16 = false;
};
template <>
struct WeightFmt<kFmtW4A16> {
  static constexpr int kStore = MOE_FP4_E2M1;
  static constexpr int kLoads = 1;
  static constexpr int kSlabBytes = 64;
  static constexpr int kMfmaFmt = MFMA_FMT_FP4;
  static constexpr bool kA16 = true;
};
template <int WFMT>
constexpr bool kFp4W = WeightFmt<WFMT>::kStore == MOE_FP4_E2M1;
template <int WFMT>
constexpr bool kA16 = WeightFmt<WFMT>::kA16;

// Where one wave's weights (4 tiles of 16 rows) come from.
template <int WFMT, bool PACKED>
struct WSrc {
  const uint8_t* row[4];   // row-major: this lane's row of each tile, + 16*g (k = 0)
  const uint8_t* erow[4];  // row-major FP4: this lane's e8m0 bytes of each tile, + g
  const uint8_t* base;     // packed: this wave's stream, + 16*lane
  const uint8_t* ebase;    // packed FP4: this wave's e8m0 stream, + 4*lane
  float fsv[2][2];         // FP8: weight scales of the tiles' two 128-row blocks, lane l
                           //      holding K slab l (fsv[.][0]) and 64 + l (fsv[.][1])
  int fsel[4];             // FP8: tile -> block 0 or 1
};

// FP8: this wave's two weight-scale rows into lanes (KB <= 128), read back per slab with
// v_readlane, so the K loop issues no scale loads at all.
template <int WFMT, bool PACKED>
__device__ __forceinline__ void load_wscales(WSrc<WFMT, PACKED>& ws, const float* row0, const float* row1, int KB) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kb = lane + 64 * j;
    ws.fsv[0][j] = kb < KB ? row0[kb] : 0.f;
    ws.fsv[1][j] = kb < KB ? row1[kb] : 0.f;
  }
}

__device__ __forceinline__ float lane_value(const float (&v)[2], int kb) {
  const int lo = __builtin_amdgcn_readlane(__float_as_int(v[0]), kb & 63);
  const int hi = __builtin_amdgcn_readlane(__float_as_int(v[1]), kb & 63);
  return __int_as_float(kb < 64 ? lo : hi);
}

// One K slab of one wave's weights.
template <int WFMT>
struct WSlab {
  u32x4 w[4][WeightFmt<WFMT>::kLoads];
  uint32_t e;  // FP4: e8m0 of tile mt in byte mt
};

template <int WFMT, bool PACKED>
__device__ __forceinline__ void load_wslab(WSlab<WFMT>& s, const WSrc<WFMT, PACKED>& ws, int kb) {
  constexpr int WL = WeightFmt<WFMT>::kLoads;
  if constexpr (PACKED) {
    const uint8_t* p = ws.base + (int64_t)kb * (4 * WL * 1024);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int h = 0; h < WL; ++h) s.w[mt][h] = gload16_nt(p + (mt * WL + h) * 1024);
    if constexpr (kFp4W<WFMT>) s.e = gload32(ws.ebase + (int64_t)kb * 256);
  } else {
    constexpr int SB = WeightFmt<WFMT>::kSlabBytes;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint8_t* p = ws.row[mt] + (int64_t)kb * SB;
      s.w[mt][0] = gload16_nt(p);
      if constexpr (WL == 2) s.w[mt][1] = gload16_nt(p + 64);
    }
    if constexpr (kFp4W<WFMT>) {
      uint32_t e = 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) e |= gload8(ws.erow[mt] + kb * 4) << (8 * mt);
      s.e = e;
    }
  }
}

// A pass's token tiles (16*NT rows) are staged K slab by K slab in LDS, shared by the
// workgroup's four waves (each wave multiplies the same tokens with its own weight
// rows).  A staged row takes the slab's bytes (128 FP8, 256 bf16) + 16 of padding: a
// row stride of 4 (mod 64) dwords keeps the B-operand reads (16 rows of one lane group
// per 128-bit LDS read cycle) free of bank conflicts.
template <bool A16>
struct TokFmt {
  static constexpr int kRowBytes = A16 ? 256 : 128;  // bytes of one token row per K slab
  static constexpr int kStride = kRowBytes + 16;      // staged row stride
  static constexpr int kChunks = kRowBytes / 16;      // 16-byte chunks per staged row
  static constexpr int kElem = A16 ? 2 : 1;           // bytes per activation element
};

// This thread's share of staging one K slab: chunk c = (threadIdx.x + 256 i) mod
// (16 NT kChunks) is bytes 16 (c % kChunks) .. +15 of token row c / kChunks.  Threads
// past the last chunk repeat one (same bytes to the same place), so the loads and
// stores carry no per-thread condition: a divergent branch around them would make the
// compiler wait for every load in flight, weights included, before the store.
template <int NT, bool A16>
struct TokStage {
  static constexpr int C = (NT * 16 * TokFmt<A16>::kChunks + 255) / 256;
  const uint8_t* src[C];  // the chunk at K slab 0
  int dst[C];             // byte offset in a staging buffer
};

// One thread's staging registers for one K slab.
template <int NT, bool A16>
using TokRegs = u32x4[TokStage<NT, A16>::C];

template <int NT, bool A16>
__device__ __forceinline__ void load_tok(TokRegs<NT, A16>& tv, const TokStage<NT, A16>& ts, int kb) {
#pragma unroll
  for (int i = 0; i < TokStage<NT, A16>::C; ++i) tv[i] = gload16(ts.src[i] + (int64_t)kb * TokFmt<A16>::kRowBytes);
}

template <int NT, bool A16>
__device__ __forceinline__ void store_tok(uint8_t* buf, const TokRegs<NT, A16>& tv, const TokStage<NT, A16>& ts) {
#pragma unroll
  for (int i = 0; i < TokStage<NT, A16>::C; ++i) *reinterpret_cast<u32x4*>(buf + ts.dst[i]) = tv[i];
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// W4A16, one K slab: the weights stay MXFP4 in registers (the FP4 loads above, lane l
// holding k = 32g..32g+31 of row l%16 and that block's e8m0 scale) and are decoded to
// bf16 with the scale applied (v_cvt_scalef32_pk_bf16_fp4, exact: an e2m1 value times a
// power of two), 8 k at a time, for v_mfma_f32_16x16x32_bf16 (lane l: row/column l%16,
// k = 8g..8g+7 of its 32).  MFMA c of the slab pairs instruction k-slot (g, i) with
// k = 32g + 8c + i on both sides, so the token fragment is bytes 64g + 16c .. +15 of the
// staged bf16 row.  The accumulator chains through the slab's four MFMAs; no promotion.
template <int NT>
__device__ __forceinline__ void compute_slab_a16(v4f (&acc)[4][NT], const u32x4 (&w)[4], uint32_t e8,
                                                 const uint8_t* tb) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
  float scl[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint32_t e = (e8 >> (8 * mt)) & 0xFFu;
    scl[mt] = __uint_as_float(e ? e << 23 : 0x00400000u);  // 2^(e - 127); e = 0 is 2^-127
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    bf16x8 av[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint32_t wd = c == 0 ? w[mt].x : c == 1 ? w[mt].y : c == 2 ? w[mt].z : w[mt].w;
      const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl[mt], 0);
      const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl[mt], 1);
      const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl[mt], 2);
      const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, scl[mt], 3);
      av[mt] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(tb + (nt * 16 + r16) * TokFmt<true>::kStride + 64 * g4 + 16 * c);
      const bf16x8 bv = __builtin_bit_cast(bf16x8, t);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bv, acc[mt][nt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // one k group's decoded weights live at a time
  }
}

// The weight scales of K slab kb for this lane's two weight-scale rows (FP8 weights;
// MXFP4 weights carry theirs in the MFMA).
template <int WFMT, bool PACKED>
__device__ __forceinline__ void slab_wscales(float (&fs)[2], const WSrc<WFMT, PACKED>& ws, int kb) {
  fs[0] = fs[1] = 1.f;
  if constexpr (WFMT == MOE_FP8_E4M3) {
    fs[0] = lane_value(ws.fsv[0], kb);
    fs[1] = lane_value(ws.fsv[1], kb);
  }
}

// The four MFMAs of token tile nt (fragments t0, t1: bytes 16g..16g+15 and 64+16g.. of
// this lane's token row in the slab) against the wave's weight slab, each promoted into
// acc with its weight scale times the token scale tsc.
template <int WFMT, bool PACKED, int NT>
__device__ __forceinline__ void mfma_tile(v4f (&acc)[4][NT], const WSlab<WFMT>& s, const WSrc<WFMT, PACKED>& ws,
                                          const float (&fs)[2], float tsc, int nt, u32x4 t0, u32x4 t1) {
  const v8i bv = {(int)t0.x, (int)t0.y, (int)t0.z, (int)t0.w, (int)t1.x, (int)t1.y, (int)t1.z, (int)t1.w};
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    v8i av;
    if constexpr (WeightFmt<WFMT>::kLoads == 2)
      av = v8i{(int)s.w[mt][0].x, (int)s.w[mt][0].y, (int)s.w[mt][0].z, (int)s.w[mt][0].w,
               (int)s.w[mt][1].x, (int)s.w[mt][1].y, (int)s.w[mt][1].z, (int)s.w[mt][1].w};
    else
      av = v8i{(int)s.w[mt][0].x, (int)s.w[mt][0].y, (int)s.w[mt][0].z, (int)s.w[mt][0].w, 0, 0, 0, 0};
    const int ea = kFp4W<WFMT> ? (int)((s.e >> (8 * mt)) & 0xFFu) : E8M0_ONE;
    const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        av, bv, v4f{0.f, 0.f, 0.f, 0.f}, WeightFmt<WFMT>::kMfmaFmt, MFMA_FMT_FP8, 0, ea, 0, E8M0_ONE);
    const float sc = (WFMT == MOE_FP8_E4M3 ? fs[ws.fsel[mt]] : 1.f) * tsc;
    acc[mt][nt][0] = fmaf(r[0], sc, acc[mt][nt][0]);
    acc[mt][nt][1] = fmaf(r[1], sc, acc[mt][nt][1]);
    acc[mt][nt][2] = fmaf(r[2], sc, acc[mt][nt][2]);
    acc[mt][nt][3] = fmaf(r[3], sc, acc[mt][nt][3]);
  }
}

// MFMAs of one slab: weights from registers, token fragments from the staged slab tb.
template <int WFMT, bool PACKED, int NT>
__device__ __forceinline__ void compute_slab(v4f (&acc)[4][NT], const WSlab<WFMT>& s, const WSrc<WFMT, PACKED>& ws,
                                             const float* s_tsc, int kb, const uint8_t* tb) {
  if constexpr (kA16<WFMT>) {
    const u32x4 w[4] = {s.w[0][0], s.w[1][0], s.w[2][0], s.w[3][0]};
    compute_slab_a16<NT>(acc, w, s.e, tb);
    return;
  }
  float fs[2];
  slab_wscales(fs, ws, kb);
  const int lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint8_t* tr = tb + (nt * 16 + r16) * TokFmt<false>::kStride + 16 * g4;
    const u32x4 t0 = *reinterpret_cast<const u32x4*>(tr);
    const u32x4 t1 = *reinterpret_cast<const u32x4*>(tr + 64);
    mfma_tile<WFMT, PACKED, NT>(acc, s, ws, fs, s_tsc[kb * (16 * NT) + nt * 16 + r16], nt, t0, t1);
    __builtin_amdgcn_sched_barrier(0);  // one token tile's fragments live at a time
  }
}

// acc[mt][nt] = promoted sum over all K slabs.  Weights: two register slabs, the next
// one in flight while the current one is consumed (a third slab costs more in spills
// than it gains, measured for FP4 and FP8).  Tokens: two LDS buffers; the slab after
// the current one is loaded into registers as each step starts and written to the
// other buffer after the step's MFMAs, and one barrier per step publishes it.  Token
// loads are issued ahead of the weight loads of the same step, so waiting for them
// leaves the weights in flight.  s_tsc holds the pass's token scales, [kb][16*NT].
// On entry w0 holds (in flight) the weights of slab 0.
template <int WFMT, bool PACKED, int NT>
__device__ __forceinline__ void mainloop(v4f (&acc)[4][NT], const WSrc<WFMT, PACKED>& ws,
                                         const TokStage<NT, kA16<WFMT>>& ts, uint8_t* s_tok, const float* s_tsc, int KB,
                                         WSlab<WFMT>& w0) {
  constexpr bool A16 = kA16<WFMT>;
  constexpr int BUF = 16 * NT * TokFmt<A16>::kStride;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  TokRegs<NT, A16> tv;
  load_tok<NT, A16>(tv, ts, 0);
  store_tok<NT, A16>(s_tok, tv, ts);
  __syncthreads();
  // one K step that loads slab kb + 1 (`next` receives its weights)
  auto step = [&](int kb, WSlab<WFMT>& cur, WSlab<WFMT>& next) {
    load_tok<NT, A16>(tv, ts, kb + 1);
    load_wslab(next, ws, kb + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute_slab<WFMT, PACKED, NT>(acc, cur, ws, s_tsc, kb, s_tok + (kb & 1) * BUF);
    __builtin_amdgcn_sched_barrier(0);
    store_tok<NT, A16>(s_tok + ((kb + 1) & 1) * BUF, tv, ts);
    __syncthreads();
  };
  // the last step: nothing left to load
  auto last = [&](int kb, WSlab<WFMT>& cur) {
    compute_slab<WFMT, PACKED, NT>(acc, cur, ws, s_tsc, kb, s_tok + (kb & 1) * BUF);
    __syncthreads();
  };
  // The loop body holds no condition around a load: at a join of paths with and without
  // the next slab's loads in flight, the compiler's wait counts would have to hold for
  // both, and so would wait for those loads inside the step meant to overlap them.
  WSlab<WFMT> w1;
  int kb = 0;
  for (; kb + 2 < KB; kb += 2) {
    step(kb, w0, w1);
    step(kb + 1, w1, w0);
  }
  if (kb + 2 == KB) {
    step(kb, w0, w1);
    last(kb + 1, w1);
  } else {
    last(kb, w0);
  }
}

// The K loop with each lane's token fragments loaded straight from L2 into registers,
// one slab ahead, in operand order (16 bytes at k = 16g and 64 + 16g of its row per 16-token
// tile): no LDS staging and no barrier per step, so the four waves of a workgroup run
// independently.  FP8 activations, at most 3 token tiles (the registers of two fragment
// sets).  trow[nt]: this lane's token row of tile nt, at k = 0.
template <int NT>
using TokFrag = u32x4[NT][2];
template <int NT>
__device__ __forceinline__ void load_frag(TokFrag<NT>& f, const uint8_t* const (&trow)[NT], int kb) {
  const int g4 = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint8_t* r = trow[nt] + (int64_t)kb * 128 + 16 * g4;
    f[nt][0] = gload16(r);
    f[nt][1] = gload16(r + 64);
  }
}
template <int WFMT, bool PACKED, int NT>
__device__ __forceinline__ void compute_direct(v4f (&acc)[4][NT], const WSlab<WFMT>& s, const WSrc<WFMT, PACKED>& ws,
                                               const float* s_tsc, int kb, const TokFrag<NT>& f) {
  float fs[2];
  slab_wscales(fs, ws, kb);
  const int r16 = threadIdx.x & 15;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    mfma_tile<WFMT, PACKED, NT>(acc, s, ws, fs, s_tsc[kb * (16 * NT) + nt * 16 + r16], nt, f[nt][0], f[nt][1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}
template <int WFMT, bool PACKED, int NT>
__device__ __forceinline__ void mainloop_direct(v4f (&acc)[4][NT], const WSrc<WFMT, PACKED>& ws,
                                                const uint8_t* const (&trow)[NT], const float* s_tsc, int KB,
                                                WSlab<WFMT>& w0) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  TokFrag<NT> fa, fb;
  load_frag<NT>(fa, trow, 0);
  // tokens of slab kb + 1 are issued ahead of its weights, so the wait for slab kb's
  // weights covers its tokens and leaves slab kb + 1 in flight
  auto step = [&](int kb, WSlab<WFMT>& cur, WSlab<WFMT>& next, const TokFrag<NT>& fc, TokFrag<NT>& fn) {
    load_frag<NT>(fn, trow, kb + 1);
    load_wslab(next, ws, kb + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute_direct<WFMT, PACKED, NT>(acc, cur, ws, s_tsc, kb, fc);
    __builtin_amdgcn_sched_barrier(0);
  };
  // no condition around a load inside the loop (see mainloop)
  WSlab<WFMT> w1;
  int kb = 0;
  for (; kb + 2 < KB; kb += 2) {
    step(kb, w0, w1, fa, fb);
    step(kb + 1, w1, w0, fb, fa);
  }
  if (kb + 2 == KB) {
    step(kb, w0, w1, fa, fb);
    compute_direct<WFMT, PACKED, NT>(acc, w1, ws, s_tsc, kb + 1, fb);
  } else {
    compute_direct<WFMT, PACKED, NT>(acc, w0, ws, s_tsc, kb, fa);
  }
}

constexpr int kMaxKB = MOE_MAX_DIM / 128;  // K slabs (the weight-scale lanes hold 128)
constexpr int kMaxTok = 6 * 16;            // tokens per pass

// Dynamic LDS of the decode GEMM kernels, sized per launch for K slabs and at most
// NTMAX token tiles per pass: the pass's token scales [KB][16*NT] fp32 (none for bf16
// activations), then the two token staging buffers: a few tens of KB instead of the
// worst case.
extern __shared__ __align__(16) uint8_t g_lds[];
__host__ __device__ constexpr int lds_tsc_bytes(int KB, int ntmax, bool a16 = false) {
  return a16 ? 0 : (KB * 16 * ntmax * 4 + 15) / 16 * 16;
}
__host__ __device__ constexpr int lds_bytes(int KB, int ntmax, bool a16 = false) {
  return lds_tsc_bytes(KB, ntmax, a16) + 2 * 16 * ntmax * (a16 ? TokFmt<true>::kStride : TokFmt<false>::kStride);
}

// The pass's token scales into LDS, s_tsc[kb][nt*16 + r16] = scale of this lane's token
// of tile nt at K slab kb; the 16 (wave, g) lane groups split the K slabs.
template <int NT>
__device__ __forceinline__ void stage_token_scales(float* s_tsc, const float* const (&tsc)[NT], int KB) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  for (int kb = wave * 4 + g4; kb < KB; kb += 16)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) s_tsc[kb * (16 * NT) + nt * 16 + r16] = gloadf(tsc[nt] + kb);
}

// Flat work list: routed expert g has nb_r entries, then the shared expert nb_s.
// routed_first (GEMM1): workgroups 0 .. E*nb_r-1 take the routed entries and the later
// ones the shared expert's, each range spread over the XCDs on its own, so that when the
// routed entries fill the GPU the shared expert's short chunks run after all of them
// (and a routed expert with a second pass starts in the first round) instead of routed
// entries being left for a second round.
__device__ __forceinline__ void work_item(const BatchDims& d, int nb_r, int nb_s, int b, int& g, int& nb,
                                          bool routed_first = false) {
  const int nr = d.E * nb_r;
  if (routed_first) {
    if (b < nr) {
      const int L = xcd_remap(b, nr);
      g = L / nb_r;
      nb = L - g * nb_r;
    } else {
      g = d.E;
      nb = xcd_remap(b - nr, nb_s);
    }
    return;
  }
  const int L = xcd_remap(b, nr + nb_s);
  if (L < nr) {
    g = L / nb_r;
    nb = L - g * nb_r;
  } else {
    g = d.E;
    nb = L - nr;
  }
}

// Where an expert's rows live: source s's bucket holds rows pre[s] .. pre[s+1]-1 of the
// expert window, starting at window row row0[s].  Built once per work item from one
// parallel load per source (wave 0), so every later row lookup is an LDS read.
struct SegTable {
  int pre[MOE_MAX_SRC + 1];
  int row0[MOE_MAX_SRC];
};

// Fills t for group g (all threads call; ends with a barrier); returns the group's rows.
__device__ __forceinline__ int load_segments(const GemmArgs& p, int g, SegTable& t) {
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
      t.pre[s] = inc - c;
      t.row0[s] = s * d.T_s * d.k + o;
    }
    if (s == d.S - 1) t.pre[d.S] = inc;
  }
  __syncthreads();
  return g < d.E ? t.pre[d.S] : d.T;
}

__device__ __forceinline__ int seg_row(const SegTable& t, int S, int m) {
  int s = 0;
  while (s + 1 < S && m >= t.pre[s + 1]) ++s;
  return t.row0[s] + (m - t.pre[s]);
}

// SENTINEL handshake of the routed experts' GEMM1 ("GC-MoE", token-ring handshake:
// the GEMM polls what dispatch publishes instead of waiting for its kernel to end).
// Lanes s < S of wave 0 poll flag[s] with relaxed loads and sleeps until it holds the
// epoch -- every source when t is null, else only the sources with rows for this
// group -- and then take one agent-scope acquire fence; the barrier orders the other
// waves after it.  A wait that exceeds spin_limit polls gives up: the work item is
// skipped and MOE_DEVERR_TIMEOUT latched.  Uniform over the workgroup.
__device__ __forceinline__ bool sentinel_wait(const GemmArgs& p, const uint32_t* flag, const SegTable* t) {
  __shared__ int s_fail;
  if (threadIdx.x == 0) s_fail = 0;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const bool need = s < p.d.S && (t == nullptr || t->pre[s + 1] > t->pre[s]);
    if (need) {
      uint32_t it = 0;
      while (__hip_atomic_load(flag + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != p.epoch) {
        if (++it > p.spin_limit) {
          s_fail = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  const bool ok = s_fail == 0;
  if (!ok && threadIdx.x == 0) atomicOr(p.err, MOE_DEVERR_TIMEOUT);
  return ok;
}

// Where token row mm of group g lives: its bytes (K slab 0), its scale row (none for
// bf16 activations), and the h / y row its result goes to.
template <bool GEMM1, bool A16>
__device__ __forceinline__ void token_row(const GemmArgs& p, const SegTable& t, int g, int mm, const uint8_t*& row,
                                          const float*& sc, int& r) {
  const BatchDims& d = p.d;
  const bool shared = g == d.E;
  constexpr int EB = TokFmt<A16>::kElem;
  sc = nullptr;
  if (GEMM1 && shared) {
    const int s = mm / d.T_s, tt = mm - s * d.T_s;
    row = p.src.x[s] + (int64_t)tt * d.H * EB;
    if constexpr (!A16) sc = p.src.xs[s] + (int64_t)tt * (d.H >> 7);
    r = d.R + mm;
  } else {
    r = shared ? d.R + mm : seg_row(t, d.S, mm);
    const int stride = GEMM1 ? d.H : d.hstride;
    row = p.a + (int64_t)r * stride * EB;
    if constexpr (!A16) sc = p.as + (int64_t)r * (stride >> 7);
  }
}

// Token rows of one pass for this lane (column r16 of each 16-token tile): scales and
// output rows (-1 past the expert's end).  Rows past the end read the pass's first
// row (their results are not stored).
template <int NT, bool GEMM1, bool A16>
__device__ __forceinline__ void pass_rows(const GemmArgs& p, const SegTable& t, int g, int M, int m0,
                                          const float* (&tsc)[NT], int (&orow)[NT],
                                          const uint8_t* (*trow)[NT] = nullptr) {
  const int r16 = threadIdx.x & 15;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int m = m0 + nt * 16 + r16;
    const uint8_t* row;
    int r;
    token_row<GEMM1, A16>(p, t, g, m < M ? m : m0, row, tsc[nt], r);
    orow[nt] = m < M ? r : -1;
    if (trow) (*trow)[nt] = row;
  }
}

// This thread's chunks of the pass's token staging (TokStage).
template <int NT, bool GEMM1, bool A16>
__device__ __forceinline__ void stage_rows(const GemmArgs& p, const SegTable& t, int g, int M, int m0,
                                           TokStage<NT, A16>& ts) {
  constexpr int CH = TokFmt<A16>::kChunks;
#pragma unroll
  for (int i = 0; i < TokStage<NT, A16>::C; ++i) {
    const unsigned c = (threadIdx.x + 256u * i) % (16u * NT * CH);
    const int row = (int)(c / CH);
    ts.dst[i] = row * TokFmt<A16>::kStride + 16 * (int)(c % CH);
    const int m = m0 + row;
    const uint8_t* rp;
    const float* sc;
    int r;
    token_row<GEMM1, A16>(p, t, g, m < M ? m : m0, rp, sc, r);
    ts.src[i] = rp + 16 * (int)(c % CH);
  }
}

// ------------------------------------------------------------------ GEMM1
// w0: the pass's first weight slab; issued here unless `issued` (the caller issued it
// earlier, so that its latency overlaps the caller's own work).
template <int WFMT, bool PACKED, int NT, bool DIRECT = false>
__device__ __forceinline__ void gemm1_pass(const GemmArgs& p, const WSrc<WFMT, PACKED>& ws, const SegTable& t,
                                           int g, int nb, int M, int m0, float (*s_amax)[kMaxTok], float* s_tsc,
                                           uint8_t* s_tok, WSlab<WFMT>& w0, bool issued) {
  const BatchDims& d = p.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int KB = d.H >> 7;
  constexpr bool A16 = kA16<WFMT>;
  const float* tsc[NT];
  int orow[NT];
  TokStage<NT, A16> ts;
  if (!issued) load_wslab(w0, ws, 0);  // the first weight slab is in flight during the pass setup
  __builtin_amdgcn_sched_barrier(0);
  static_assert(!DIRECT || (!A16 && NT <= 3), "direct token loads: FP8 activations, at most 3 tiles");
  const uint8_t* trow[NT];
  pass_rows<NT, true, A16>(p, t, g, M, m0, tsc, orow, &trow);
  if constexpr (!DIRECT) stage_rows<NT, true, A16>(p, t, g, M, m0, ts);
  if constexpr (!A16) stage_token_scales<NT>(s_tsc, tsc, KB);
  __syncthreads();
  v4f acc[4][NT];
  if constexpr (DIRECT)
    mainloop_direct<WFMT, PACKED, NT>(acc, ws, trow, s_tsc, KB, w0);
  else
    mainloop<WFMT, PACKED, NT>(acc, ws, ts, s_tok, s_tsc, KB, w0);

  if constexpr (A16) {
    // SwiGLU, h stored bf16: this lane holds rows rb + 16t + 4*g4 + i of token column
    // nt*16 + r16, i.e. 4 consecutive h elements of that token's row
    const int rb = nb * 128 + 32 * wave;
    uint16_t* hb = reinterpret_cast<uint16_t*>(p.h);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (orow[nt] < 0) continue;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = silu(acc[t][nt][i]) * acc[2 + t][nt][i];
        *reinterpret_cast<uint2*>(hb + (int64_t)orow[nt] * d.hstride + rb + 16 * t + 4 * g4) =
            make_uint2(bf16_bits(v[0]) | (bf16_bits(v[1]) << 16), bf16_bits(v[2]) | (bf16_bits(v[3]) << 16));
      }
    }
    __syncthreads();  // the token staging buffers are reused by the next pass
    return;
  }
  // SwiGLU; this lane holds rows rb + 16t + 4*g4 + i (t = 0, 1) of token column nt*16 + r16
  float hv[2][NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float mx = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = silu(acc[t][nt][i]) * acc[2 + t][nt][i];
        hv[t][nt][i] = v;
        mx = fmaxf(mx, fabsf(v));
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (g4 == 0) s_amax[wave][nt * 16 + r16] = mx;
  }
  __syncthreads();
  // requantise: one fp32 scale per 128 columns (this workgroup's block nb) of each row
  const int rb = nb * 128 + 32 * wave;
  const int hsc_stride = d.hstride >> 7;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (orow[nt] < 0) continue;
    const int tk = nt * 16 + r16;
    const float amax = fmaxf(fmaxf(s_amax[0][tk], s_amax[1][tk]), fmaxf(s_amax[2][tk], s_amax[3][tk]));
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
    const float inv = __builtin_amdgcn_rcpf(sc);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = e4m3_scaled(hv[t][nt][i], inv);
      *reinterpret_cast<uint32_t*>(p.h + (int64_t)orow[nt] * d.hstride + rb + 16 * t + 4 * g4) =
          pack4_e4m3(q[0], q[1], q[2], q[3]);
    }
    if (wave == 0 && g4 == 0) p.hs[(int64_t)orow[nt] * hsc_stride + nb] = sc;
  }
  __syncthreads();  // s_amax and s_tsc are reused by the next pass
}

// One GEMM1 work item: column block nb (128 gate + 128 up rows) of expert group g, over
// all of the group's rows.  Every thread of the workgroup calls it.
// prologue (SENTINEL, dispatch fused into this launch): the item's first weight slab and
// its weight scales are issued, then this workgroup runs dispatch chunk `chunk` of `da`
// (if chunk >= 0; every chunk of the dispatch is some workgroup's), and only then does it
// wait for the counts and rows its expert needs -- so the dispatch runs on every CU at
// the start of the launch, under the latency of the first weight loads.
struct NoPrologue {
  static constexpr bool kOn = false;
  __device__ void operator()() const {}
};
struct DispatchPrologue {
  static constexpr bool kOn = true;
  const DispatchArgs& da;
  int chunk, chunks;  // chunk < 0: none for this workgroup
  __device__ void operator()() const {
    if (chunk >= 0) dispatch_chunk(da, chunk / chunks, chunk % chunks, chunks, *reinterpret_cast<DispatchSmem*>(g_lds));
  }
};

// The one-tile passes of the small-batch kernels (at most two token tiles per pass,
// FP8 activations) load their token fragments straight into registers; in the kernels
// for larger batches such passes are rare and the staged loop alone measured faster.
template <int NTMAX, int WFMT>
constexpr bool kDirect1 = NTMAX == 2 && !kA16<WFMT>;

template <int NTMAX, int WFMT, bool PACKED, class Prologue = NoPrologue>
__device__ __forceinline__ void gemm1_item(const GemmArgs& p, int g, int nb_item, float (*s_amax)[kMaxTok],
                                           float* s_tsc, uint8_t* s_tok, SegTable& seg,
                                           const Prologue& prologue = Prologue{}) {
  const BatchDims& d = p.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  int nb = nb_item;
  const bool shared = g == d.E;
  const int inter = shared ? d.Ish : d.I;
  // the shared expert reads the source buffers, so only routed groups wait
  const bool sentinel = p.rflag != nullptr && !shared;
  // the shared expert's rows are split into chunks, each its own work item
  int shc = 0;
  if (shared) {
    shc = nb % p.sh_chunks;
    nb /= p.sh_chunks;
  }
  const int K = d.H, KB = K >> 7;
  constexpr bool FP4 = kFp4W<WFMT>;
  constexpr int SF = WeightFmt<WFMT>::kStore;
  const uint8_t* W = shared ? p.w_sh : p.w + (int64_t)g * p.w_stride;
  const uint8_t* WSb = static_cast<const uint8_t*>(shared ? p.ws_sh : p.ws) +
                       (shared ? 0 : (int64_t)g * p.ws_stride * (FP4 ? 1 : 4));
  WSrc<WFMT, PACKED> ws;
  const int rb = nb * 128 + 32 * wave;  // this wave's gate rows rb..rb+31; up rows inter + same
  if constexpr (PACKED) {
    ws.base = W + pack_w13_offset(SF, K, nb, wave, 0) + 16 * lane;
    if constexpr (FP4) ws.ebase = WSb + pack_e13_offset(K, nb, wave, 0) + 4 * lane;
  } else {
    const int64_t wrow = FP4 ? (K >> 1) : K;
    const int rows[4] = {rb, rb + 16, inter + rb, inter + rb + 16};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      ws.row[mt] = W + (int64_t)(rows[mt] + r16) * wrow + 16 * g4;
      if constexpr (FP4) ws.erow[mt] = WSb + (int64_t)(rows[mt] + r16) * (K >> 5) + g4;
    }
  }
  WSlab<WFMT> w0;
  constexpr bool pro = Prologue::kOn;
  if constexpr (pro) {
    load_wslab(w0, ws, 0);  // in flight across the dispatch chunk and the waits
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!FP4) {
    const float* FS = reinterpret_cast<const float*>(WSb);
    // gate rows: block nb; up rows: block I/128 + nb
    load_wscales(ws, FS + (int64_t)nb * KB, FS + (int64_t)((inter >> 7) + nb) * KB, KB);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ws.fsel[mt] = mt >> 1;
  }
  if constexpr (pro) {
    prologue();
    __syncthreads();  // the dispatch's LDS is the passes' LDS
  }
  // prologue form: one wait, for every source's rows (their last writer also published
  // the counts, so one acquire covers both); else the counts first, then the rows of the
  // sources that hold rows of this group, with the weight scales in flight meanwhile
  if (sentinel && !sentinel_wait(p, pro ? p.dflag : p.rflag, nullptr)) return;
  const int M = load_segments(p, g, seg);
  int mb = 0, me = M;
  if (shared) {
    mb = shc * p.sh_chunk_rows;
    me = min(M, mb + p.sh_chunk_rows);
  }
  if (M == 0) return;  // no rows: no weight traffic (uniform over the workgroup)
  if (!pro && sentinel && !sentinel_wait(p, p.dflag, &seg)) return;

  for (int m0 = mb; m0 < me; m0 += 16 * NTMAX) {
    const int nt = min(NTMAX, (me - m0 + 15) >> 4);
    const bool issued = pro && m0 == mb;
    switch (nt) {
      case 1: gemm1_pass<WFMT, PACKED, 1, kDirect1<NTMAX, WFMT>>(p, ws, seg, g, nb, me, m0, s_amax, s_tsc, s_tok, w0, issued); break;
      case 2: if constexpr (NTMAX >= 2) gemm1_pass<WFMT, PACKED, 2>(p, ws, seg, g, nb, me, m0, s_amax, s_tsc, s_tok, w0, issued); break;
      case 3: if constexpr (NTMAX >= 3) gemm1_pass<WFMT, PACKED, 3>(p, ws, seg, g, nb, me, m0, s_amax, s_tsc, s_tok, w0, issued); break;
      case 4: if constexpr (NTMAX >= 4) gemm1_pass<WFMT, PACKED, 4>(p, ws, seg, g, nb, me, m0, s_amax, s_tsc, s_tok, w0, issued); break;
      case 5: if constexpr (NTMAX >= 5) gemm1_pass<WFMT, PACKED, 5>(p, ws, seg, g, nb, me, m0, s_amax, s_tsc, s_tok, w0, issued); break;
      default: if constexpr (NTMAX >= 6) gemm1_pass<WFMT, PACKED, 6>(p, ws, seg, g, nb, me, m0, s_amax, s_tsc, s_tok, w0, issued); break;
    }
  }
}

// nchunks > 0 (SENTINEL, dispatch fused into this launch): workgroup b < nchunks runs
// dispatch chunk b (of `chunks` per source) in its prologue (gemm1_item); workgroups past
// the last work item (when chunks outnumber items) run only their chunk.  Every chunk is
// run by one of the lowest-numbered workgroups, which a GPU places first, and a chunk
// never waits for anything, so every flag a workgroup waits on is published by a
// workgroup that is already running.
template <int NTMAX, int WFMT, bool PACKED, bool FUSED>
__global__ __launch_bounds__(256, 2) void k_gemm1_lowp(GemmArgs p, DispatchArgs da, int nchunks, int chunks) {
  __shared__ float s_amax[4][kMaxTok];
  __shared__ SegTable seg;
  float* s_tsc = reinterpret_cast<float*>(g_lds);
  uint8_t* s_tok = g_lds + lds_tsc_bytes(p.d.H >> 7, NTMAX, kA16<WFMT>);
  const int b = blockIdx.x;
  const int items = p.d.E * (p.d.I >> 7) + (p.d.Ish >> 7) * p.sh_chunks;
  if constexpr (FUSED) {
    if (b >= items) {
      if (b < nchunks) dispatch_chunk(da, b / chunks, b % chunks, chunks, *reinterpret_cast<DispatchSmem*>(g_lds));
      return;
    }
  }
  int g, nb;
  work_item(p.d, p.d.I >> 7, (p.d.Ish >> 7) * p.sh_chunks, b, g, nb, true);
  if constexpr (FUSED)
    gemm1_item<NTMAX, WFMT, PACKED>(p, g, nb, s_amax, s_tsc, s_tok, seg,
                                    DispatchPrologue{da, b < nchunks ? b : -1, chunks});
  else
    gemm1_item<NTMAX, WFMT, PACKED>(p, g, nb, s_amax, s_tsc, s_tok, seg);
}

// ------------------------------------------------------------------ combine in GEMM2
// Option: the top-k weighted combine runs in GEMM2's epilogue instead of as its own
// kernel (the fused form the pages set against their split design: "GC-MoE:
// Decoupling MoE Communication and Computation with CUDA Green Contexts", "Why Expert
// Parallelism Is Inefficient in MoE Decoding").  A work item (group g, output columns
// nb*256 .. +255) counts, for each of its rows, one contribution of that row's token
// to those columns: an atomic counter per (token, column block) at agent scope, taken
// after the item's y stores have been made visible at agent scope (one write-back of the
// XCD's L2 per item).  The item whose count completes a token's set -- its slots with a
// row, plus the shared expert's row -- reads the token's y rows, which come from other
// experts' items on other XCDs, with agent-coherent loads (no L2 invalidation), and
// forms out[t][nb*256 .. +255] from them with the combine
// kernel's arithmetic (fp32 FMAs in slot order, the shared row last with weight 1,
// bf16 rounding), so its output is bit-identical to that kernel's.  It then resets the
// counter: every counter is back at zero when the launch ends, and no pass clears them
// between calls.  Tokens with no contribution at all (no slot with a row, no shared
// expert) get zero rows from workgroups past the last work item.

// Contributions that complete token t: its slots with a window row, plus the shared row.
__device__ __forceinline__ int token_need(const GemmArgs& p, int t) {
  const int k = p.d.k;
  int n = p.d.Ish > 0 ? 1 : 0;
  for (int j = 0; j < k; ++j) n += p.dst_row[(int64_t)t * k + j] >= 0 ? 1 : 0;
  return n;
}

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const uint4& y, float w) {
  const uint32_t u[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] = fmaf(w, bf16_to_f32(u[q] & 0xFFFFu), acc[2 * q]);
    acc[2 * q + 1] = fmaf(w, bf16_to_f32(u[q] >> 16), acc[2 * q + 1]);
  }
}

// 16 bytes of a y row written by another work item, read coherently at agent scope (four
// relaxed agent-scope loads: they miss any stale copy in this XCD's L2, so no L2
// invalidation is needed).  The caller issues them only after its counter update has seen
// every writer's, and each writer made its rows visible at agent scope before its update.
__device__ __forceinline__ uint4 load_coherent16(const uint16_t* p) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
  uint4 v;
  v.x = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.y = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.z = __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.w = __hip_atomic_load(q + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

// out[t][c .. c+7] from the token's y rows (one 16-byte piece per lane).
__device__ __forceinline__ void combine_piece(const GemmArgs& p, int t, int c) {
  const BatchDims& d = p.d;
  if (c >= d.H) return;
  const int k = d.k;
  const int32_t* rmap = p.dst_row + (int64_t)t * k;
  const float* wmap = p.topk_w + (int64_t)t * k;
  const uint16_t* yc = p.y + c;
  float acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = 0.f;
  for (int j0 = 0; j0 < k; j0 += 8) {  // eight slots' rows in flight at a time, added in slot order
    int rows[8];
    uint4 yv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rows[j] = j0 + j < k ? rmap[j0 + j] : -1;
#pragma unroll
    for (int j = 0; j < 8; ++j) yv[j] = load_coherent16(yc + (int64_t)max(rows[j], 0) * d.H);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (rows[j] >= 0) add_bf16x8(acc, yv[j], wmap[j0 + j]);
  }
  if (d.Ish) add_bf16x8(acc, load_coherent16(yc + (int64_t)(d.R + t) * d.H), 1.0f);
  uint4 o;
  o.x = pack2_bf16(acc[0], acc[1]);
  o.y = pack2_bf16(acc[2], acc[3]);
  o.z = pack2_bf16(acc[4], acc[5]);
  o.w = pack2_bf16(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(p.out + (int64_t)t * d.H + c) = o;
}

// After a GEMM2 item's passes: count its rows [mb, me) of group g towards their tokens'
// column block nb and combine the tokens it completes.  Every thread calls it.
__device__ __forceinline__ void combine_tail(const GemmArgs& p, int g, int nb, int mb, int me, const SegTable& seg) {
  __shared__ int s_list[256];
  __shared__ int s_n;
  const BatchDims& d = p.d;
  const int nbh = (d.H + 255) >> 8;
  release_workgroup_stores();  // the item's y rows, visible at agent scope before any count
  for (int m0 = mb; m0 < me; m0 += 256) {
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    const int m = m0 + (int)threadIdx.x;
    if (m < me) {
      const int t = g < d.E ? p.row_src[seg_row(seg, d.S, m)] / d.k : m;
      uint32_t* cp = p.ccnt + (int64_t)t * nbh + nb;
      const uint32_t old = __hip_atomic_fetch_add(cp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int)old + 1 == token_need(p, t)) {
        __hip_atomic_store(cp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
        s_list[atomicAdd(&s_n, 1)] = t;
      }
    }
    __syncthreads();
    const int n = s_n;
    for (int i = (int)threadIdx.x >> 5; i < n; i += 8) combine_piece(p, s_list[i], nb * 256 + 8 * (threadIdx.x & 31));
    __syncthreads();  // s_n and s_list are reused
  }
}

// Workgroups past the last work item: zero output rows of the tokens [b*256, +256) with
// no contribution (only possible without a shared expert).
__device__ __forceinline__ void combine_zero_rows(const GemmArgs& p, int b) {
  __shared__ int s_list[256];
  __shared__ int s_n;
  const BatchDims& d = p.d;
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  const int t = b * 256 + (int)threadIdx.x;
  if (t < d.T && token_need(p, t) == 0) s_list[atomicAdd(&s_n, 1)] = t;
  __syncthreads();
  const int n = s_n, per_row = d.H >> 3;
  for (int i = (int)threadIdx.x; i < n * per_row; i += 256) {
    const int tt = s_list[i / per_row], c = 8 * (i % per_row);
    *reinterpret_cast<uint4*>(p.out + (int64_t)tt * d.H + c) = make_uint4(0u, 0u, 0u, 0u);
  }
}

// ------------------------------------------------------------------ GEMM2
template <int WFMT, bool PACKED, int NT, bool DIRECT = false>
__device__ __forceinline__ void gemm2_pass(const GemmArgs& p, const WSrc<WFMT, PACKED>& ws, const SegTable& t,
                                           int g, int rb, bool active, int K, int M, int m0, float* s_tsc,
                                           uint8_t* s_tok) {
  const BatchDims& d = p.d;
  const int lane = threadIdx.x & 63, g4 = lane >> 4;
  const int KB = K >> 7;
  constexpr bool A16 = kA16<WFMT>;
  const float* tsc[NT];
  int orow[NT];
  TokStage<NT, A16> ts;
  WSlab<WFMT> w0;
  load_wslab(w0, ws, 0);  // the first weight slab is in flight during the pass setup
  __builtin_amdgcn_sched_barrier(0);
  static_assert(!DIRECT || (!A16 && NT <= 3), "direct token loads: FP8 activations, at most 3 tiles");
  const uint8_t* trow[NT];
  pass_rows<NT, false, A16>(p, t, g, M, m0, tsc, orow, &trow);
  if constexpr (!DIRECT) stage_rows<NT, false, A16>(p, t, g, M, m0, ts);
  if constexpr (!A16) stage_token_scales<NT>(s_tsc, tsc, KB);
  __syncthreads();
  v4f acc[4][NT];
  // a wave past a ragged end of H repeats the last tile's rows and stores nothing
  if constexpr (DIRECT)
    mainloop_direct<WFMT, PACKED, NT>(acc, ws, trow, s_tsc, KB, w0);
  else
    mainloop<WFMT, PACKED, NT>(acc, ws, ts, s_tok, s_tsc, KB, w0);
  __syncthreads();  // s_tsc is reused by the next pass
  if (!active) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (orow[nt] < 0) continue;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint32_t lo = bf16_bits(acc[mt][nt][0]) | (bf16_bits(acc[mt][nt][1]) << 16);
      const uint32_t hi = bf16_bits(acc[mt][nt][2]) | (bf16_bits(acc[mt][nt][3]) << 16);
      *reinterpret_cast<uint2*>(p.y + (int64_t)orow[nt] * d.H + rb + 16 * mt + 4 * g4) = make_uint2(lo, hi);
    }
  }
}

// One GEMM2 work item: output rows nb*256 .. +255 of expert group g, over all of the
// group's rows.  Every thread of the workgroup calls it.
template <int NTMAX, int WFMT, bool PACKED, bool FUSEC = false>
__device__ __forceinline__ void gemm2_item(const GemmArgs& p, int g, int nb_item, float* s_tsc, uint8_t* s_tok,
                                           SegTable& seg) {
  const BatchDims& d = p.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  int nb = nb_item, chunk = 0;
  if (g == d.E) {  // the shared expert's rows are split into chunks, each its own work item
    chunk = nb % p.sh_chunks;
    nb /= p.sh_chunks;
  }
  const int rb0 = nb * 256 + 64 * wave;
  const bool active = rb0 < d.H;      // a ragged last tile: such waves compute rows rb.. again

  const int rb = active ? rb0 : d.H - 64;
  const bool shared = g == d.E;
  const int K = shared ? d.Ish : d.I, KB = K >> 7;
  const int M = load_segments(p, g, seg);
  if (M == 0) return;
  const int mb = g == d.E ? chunk * p.sh_chunk_rows : 0;
  const int me = g == d.E ? min(M, mb + p.sh_chunk_rows) : M;

  constexpr bool FP4 = kFp4W<WFMT>;
  constexpr int SF = WeightFmt<WFMT>::kStore;
  const uint8_t* W = shared ? p.w_sh : p.w + (int64_t)g * p.w_stride;
  const uint8_t* WSb = static_cast<const uint8_t*>(shared ? p.ws_sh : p.ws) +
                       (shared ? 0 : (int64_t)g * p.ws_stride * (FP4 ? 1 : 4));
  WSrc<WFMT, PACKED> ws;
  if constexpr (PACKED) {
    ws.base = W + pack_w2_offset(SF, K, nb, wave, 0) + 16 * lane;
    if constexpr (FP4) ws.ebase = WSb + pack_e2_offset(K, nb, wave, 0) + 4 * lane;
  } else {
    const int64_t wrow = FP4 ? (K >> 1) : K;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = rb + 16 * mt + r16;
      ws.row[mt] = W + (int64_t)row * wrow + 16 * g4;
      if constexpr (FP4) ws.erow[mt] = WSb + (int64_t)row * (K >> 5) + g4;
    }
  }
  if constexpr (!FP4) {
    // this wave's 64 rows sit in one 128-row scale block
    const float* FS = reinterpret_cast<const float*>(WSb) + (int64_t)(rb >> 7) * KB;
    load_wscales(ws, FS, FS, KB);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ws.fsel[mt] = 0;
  }

  for (int m0 = mb; m0 < me; m0 += 16 * NTMAX) {
    const int nt = min(NTMAX, (me - m0 + 15) >> 4);
    switch (nt) {
      case 1: gemm2_pass<WFMT, PACKED, 1, kDirect1<NTMAX, WFMT>>(p, ws, seg, g, rb, active, K, me, m0, s_tsc, s_tok); break;
      case 2: if constexpr (NTMAX >= 2) gemm2_pass<WFMT, PACKED, 2>(p, ws, seg, g, rb, active, K, me, m0, s_tsc, s_tok); break;
      case 3: if constexpr (NTMAX >= 3) gemm2_pass<WFMT, PACKED, 3>(p, ws, seg, g, rb, active, K, me, m0, s_tsc, s_tok); break;
      case 4: if constexpr (NTMAX >= 4) gemm2_pass<WFMT, PACKED, 4>(p, ws, seg, g, rb, active, K, me, m0, s_tsc, s_tok); break;
      case 5: if constexpr (NTMAX >= 5) gemm2_pass<WFMT, PACKED, 5>(p, ws, seg, g, rb, active, K, me, m0, s_tsc, s_tok); break;
      default: if constexpr (NTMAX >= 6) gemm2_pass<WFMT, PACKED, 6>(p, ws, seg, g, rb, active, K, me, m0, s_tsc, s_tok); break;
    }
  }
  if constexpr (FUSEC) combine_tail(p, g, nb, mb, me, seg);
}

template <int NTMAX, int WFMT, bool PACKED, bool FUSEC = false>
__global__ __launch_bounds__(256, 2) void k_gemm2_lowp(GemmArgs p) {
  __shared__ SegTable seg;
  float* s_tsc = reinterpret_cast<float*>(g_lds);
  uint8_t* s_tok = g_lds + lds_tsc_bytes(p.d.hstride >> 7, NTMAX, kA16<WFMT>);
  const int nbh = (p.d.H + 255) >> 8;  // 256 output rows per workgroup, 64 per wave
  const int nb_s = p.d.Ish ? nbh * p.sh_chunks : 0;
  if constexpr (FUSEC) {
    const int items = p.d.E * nbh + nb_s;
    if ((int)blockIdx.x >= items) {
      if (!p.d.Ish) combine_zero_rows(p, (int)blockIdx.x - items);
      return;
    }
  }
  int g, nb;
  work_item(p.d, nbh, nb_s, blockIdx.x, g, nb);
  gemm2_item<NTMAX, WFMT, PACKED, FUSEC>(p, g, nb, s_tsc, s_tok, seg);
}

// ------------------------------------------------------------------ persistent
// Both GEMMs in one launch.  Work items -- GEMM1 column blocks, then GEMM2 row blocks
// -- are pulled from atomic queues: one per XCD (queue x serves the expert groups
// g = x, x + 8, ... so an expert's token rows stay in that XCD's L2) or a single
// queue (when experts are few or their loads very uneven).  A GEMM2 item of group g
// first waits until all GEMM1 items of g have published their h rows (release
// counter, agent scope).  Items are dequeued GEMM1-first, so a waited-on item has
// always been taken by a running workgroup: no wait can deadlock.  The last
// workgroup to leave resets the queues and counters for the next call.
__device__ __forceinline__ int items1_of(const ExpertsArgs& a, int g) {
  return g < a.g1.d.E ? a.nb1_r : a.nb1_s * a.g1.sh_chunks;
}
__device__ __forceinline__ int items2_of(const ExpertsArgs& a, int g) {
  return g < a.g1.d.E ? a.nb2 : a.nb2 * a.g1.sh_chunks;
}

// the q-th queue's groups are q, q + step, ...; returns (kind, g, nb) of entry i, kind 0 = none
__device__ __forceinline__ int decode_item(const ExpertsArgs& a, int q, int step, int i, int& g, int& nb) {
  const int nG = a.g1.d.E + (a.g1.d.Ish ? 1 : 0);
  for (int gg = q; gg < nG; gg += step) {
    const int n = items1_of(a, gg);
    if (i < n) { g = gg; nb = i; return 1; }
    i -= n;
  }
  for (int gg = q; gg < nG; gg += step) {
    const int n = items2_of(a, gg);
    if (i < n) { g = gg; nb = i; return 2; }
    i -= n;
  }
  return 0;
}

// FUSEC: the combine runs in the GEMM2 items' epilogue (a.g2.ccnt set), and the zero rows
// of tokens with no contribution are written by the workgroups as they leave.
template <int NTMAX, int WFMT, bool PACKED, bool FUSEC = false>
__global__ __launch_bounds__(256, 2) void k_experts_lowp(ExpertsArgs a) {
  __shared__ float s_amax[4][kMaxTok];
  __shared__ int s_item, s_go;
  __shared__ SegTable seg;
  float* s_tsc = reinterpret_cast<float*>(g_lds);
  uint8_t* s_tok = g_lds + lds_tsc_bytes(max(a.g1.d.H, a.g1.d.hstride) >> 7, NTMAX);
  const int q = a.per_xcd ? (blockIdx.x & 7) : 0, step = a.per_xcd ? 8 : 1;
  uint32_t* head = a.sched + q;
  uint32_t* exits = a.sched + 8;
  uint32_t* done1 = a.sched + 16;
  for (;;) {
    if (threadIdx.x == 0) s_item = (int)atomicAdd(head, 1u);
    __syncthreads();
    const int i = s_item;
    int g = 0, nb = 0;
    const int kind = decode_item(a, q, step, i, g, nb);
    if (kind == 0) break;  // uniform over the workgroup
    if (kind == 1) {
      gemm1_item<NTMAX, WFMT, PACKED>(a.g1, g, nb, s_amax, s_tsc, s_tok, seg);
      release_workgroup_stores();  // every wave's h stores, visible at agent scope
      if (threadIdx.x == 0) __hip_atomic_fetch_add(done1 + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (threadIdx.x == 0) {
        const uint32_t need = (uint32_t)items1_of(a, g);
        uint32_t it = 0;
        // poll without acquiring (an acquire invalidates caches other waves still use),
        // then acquire once
        while (__hip_atomic_load(done1 + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
          if (++it > a.spin_limit) break;
          __builtin_amdgcn_s_sleep(8);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_go = it <= a.spin_limit;
        if (!s_go) atomicOr(a.g1.err, MOE_DEVERR_TIMEOUT);
      }
      __syncthreads();
      if (s_go) gemm2_item<NTMAX, WFMT, PACKED, FUSEC>(a.g2, g, nb, s_tsc, s_tok, seg);
    }
    __syncthreads();  // s_item, s_go and the LDS tables are free again
  }
  if constexpr (FUSEC) {
    if (!a.g2.d.Ish)
      for (int tb = (int)blockIdx.x; tb * 256 < a.g2.d.T; tb += (int)gridDim.x) {
        combine_zero_rows(a.g2, tb);
        __syncthreads();  // its token list is rebuilt by the next round
      }
  }
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(exits, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {  // everyone else has left: reset for the next call
      const int nG = a.g1.d.E + (a.g1.d.Ish ? 1 : 0);
      for (int x = 0; x < 8; ++x) __hip_atomic_store(a.sched + x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int gg = 0; gg < nG; ++gg) __hip_atomic_store(done1 + gg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(exits, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int WFMT, bool PACKED>
hipError_t launch1(const GemmArgs& a, int nt, const DispatchArgs* fused, hipStream_t st) {
  DispatchArgs da{};
  int nchunks = 0, chunks = 0;
  if (fused) {
    da = *fused;
    chunks = dispatch_chunks(da);
    nchunks = da.S * chunks;
  }
  const int items = a.d.E * (a.d.I >> 7) + (a.d.Ish >> 7) * a.sh_chunks;
  const dim3 grid(std::max(items, nchunks)), block(256);
  const int KB = a.d.H >> 7;
  auto lds = [&](int ntmax) {
    const int b = lds_bytes(KB, ntmax, kA16<WFMT>);
    return (size_t)(nchunks && b < (int)sizeof(DispatchSmem) ? (int)sizeof(DispatchSmem) : b);
  };
  if (nchunks) {
    if (nt <= 2)
      hipLaunchKernelGGL((k_gemm1_lowp<2, WFMT, PACKED, true>), grid, block, lds(2), st, a, da, nchunks, chunks);
    else if (nt == 3)
      hipLaunchKernelGGL((k_gemm1_lowp<3, WFMT, PACKED, true>), grid, block, lds(3), st, a, da, nchunks, chunks);
    else if (nt == 4 || !kFp4W<WFMT>)
      hipLaunchKernelGGL((k_gemm1_lowp<4, WFMT, PACKED, true>), grid, block, lds(4), st, a, da, nchunks, chunks);
    else
      hipLaunchKernelGGL((k_gemm1_lowp<5, (kFp4W<WFMT> ? WFMT : MOE_FP4_E2M1), PACKED, true>), grid, block, lds(5), st,
                         a, da, nchunks, chunks);
  } else {
    if (nt <= 2)
      hipLaunchKernelGGL((k_gemm1_lowp<2, WFMT, PACKED, false>), grid, block, lds(2), st, a, da, 0, 0);
    else if (nt == 3)
      hipLaunchKernelGGL((k_gemm1_lowp<3, WFMT, PACKED, false>), grid, block, lds(3), st, a, da, 0, 0);
    else if (nt == 4 || !kFp4W<WFMT>)
      hipLaunchKernelGGL((k_gemm1_lowp<4, WFMT, PACKED, false>), grid, block, lds(4), st, a, da, 0, 0);
    else
      hipLaunchKernelGGL((k_gemm1_lowp<5, (kFp4W<WFMT> ? WFMT : MOE_FP4_E2M1), PACKED, false>), grid, block, lds(5),
                         st, a, da, 0, 0);
  }
  return hipGetLastError();
}

template <int WFMT, bool PACKED, bool FUSEC>
void launch2_nt(const GemmArgs& a, int nt, dim3 grid, hipStream_t st) {
  const int KB = a.d.hstride >> 7;
  constexpr bool A16 = kA16<WFMT>;
  const dim3 block(256);
  if (nt <= 2)
    hipLaunchKernelGGL((k_gemm2_lowp<2, WFMT, PACKED, FUSEC>), grid, block, lds_bytes(KB, 2, A16), st, a);
  else if (nt == 3)
    hipLaunchKernelGGL((k_gemm2_lowp<3, WFMT, PACKED, FUSEC>), grid, block, lds_bytes(KB, 3, A16), st, a);
  else if (nt == 4 || !kFp4W<WFMT>)
    hipLaunchKernelGGL((k_gemm2_lowp<4, WFMT, PACKED, FUSEC>), grid, block, lds_bytes(KB, 4, A16), st, a);
  else
    hipLaunchKernelGGL((k_gemm2_lowp<5, (kFp4W<WFMT> ? WFMT : MOE_FP4_E2M1), PACKED, FUSEC>), grid, block,
                       lds_bytes(KB, 5, A16), st, a);
}

// a.ccnt != null: the combine runs in the epilogue (plus a workgroup per 256 tokens for
// the zero rows of tokens with no contribution, when there is no shared expert).
template <int WFMT, bool PACKED>
hipError_t launch2(const GemmArgs& a, int nt, hipStream_t st) {
  const int nbh = (a.d.H + 255) >> 8;
  const int items = a.d.E * nbh + (a.d.Ish ? nbh * a.sh_chunks : 0);
  if (a.ccnt)
    launch2_nt<WFMT, PACKED, true>(a, nt, dim3(items + (a.d.Ish ? 0 : (a.d.T + 255) / 256)), st);
  else
    launch2_nt<WFMT, PACKED, false>(a, nt, dim3(items), st);
  return hipGetLastError();
}

template <int WFMT, bool PACKED, bool FUSEC>
void launch_experts_nt(const ExpertsArgs& a, int nt, int grid, hipStream_t st) {
  const int KB = std::max(a.g1.d.H, a.g1.d.hstride) >> 7;
  if (nt <= 2)
    hipLaunchKernelGGL((k_experts_lowp<2, WFMT, PACKED, FUSEC>), dim3(grid), dim3(256), lds_bytes(KB, 2), st, a);
  else if (nt == 3)
    hipLaunchKernelGGL((k_experts_lowp<3, WFMT, PACKED, FUSEC>), dim3(grid), dim3(256), lds_bytes(KB, 3), st, a);
  else
    hipLaunchKernelGGL((k_experts_lowp<4, WFMT, PACKED, FUSEC>), dim3(grid), dim3(256), lds_bytes(KB, 4), st, a);
}

template <int WFMT, bool PACKED>
hipError_t launch_experts(const ExpertsArgs& a, int nt, int grid, hipStream_t st) {
  if (a.g2.ccnt)
    launch_experts_nt<WFMT, PACKED, true>(a, nt, grid, st);
  else
    launch_experts_nt<WFMT, PACKED, false>(a, nt, grid, st);
  return hipGetLastError();
}

template <int WFMT, bool PACKED>
int experts_blocks_per_cu(int nt, int KB) {
  int n = 0;
  hipError_t e;
  if (nt <= 2)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_experts_lowp<2, WFMT, PACKED>, 256, lds_bytes(KB, 2));
  else if (nt == 3)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_experts_lowp<3, WFMT, PACKED>, 256, lds_bytes(KB, 3));
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_experts_lowp<4, WFMT, PACKED>, 256, lds_bytes(KB, 4));
  return e == hipSuccess ? n : 0;
}

}  // namespace

hipError_t launch_experts_lowp(const ExpertsArgs& a, int weight_fmt, int packed, int tok_tiles, int grid,
                               hipStream_t st) {
  if (weight_fmt == MOE_FP4_E2M1)
    return packed ? launch_experts<MOE_FP4_E2M1, true>(a, tok_tiles, grid, st)
                  : launch_experts<MOE_FP4_E2M1, false>(a, tok_tiles, grid, st);
  return packed ? launch_experts<MOE_FP8_E4M3, true>(a, tok_tiles, grid, st)
                : launch_experts<MOE_FP8_E4M3, false>(a, tok_tiles, grid, st);
}

int experts_lowp_blocks_per_cu(int weight_fmt, int packed, int tok_tiles, int k_slabs) {
  if (weight_fmt == MOE_FP4_E2M1)
    return packed ? experts_blocks_per_cu<MOE_FP4_E2M1, true>(tok_tiles, k_slabs)
                  : experts_blocks_per_cu<MOE_FP4_E2M1, false>(tok_tiles, k_slabs);
  return packed ? experts_blocks_per_cu<MOE_FP8_E4M3, true>(tok_tiles, k_slabs)
                : experts_blocks_per_cu<MOE_FP8_E4M3, false>(tok_tiles, k_slabs);
}

hipError_t launch_gemm1_lowp(const GemmArgs& a, int weight_fmt, int packed, int tok_tiles, hipStream_t st,
                             const DispatchArgs* fused) {
  if (weight_fmt == kFmtW4A16)
    return packed ? launch1<kFmtW4A16, true>(a, tok_tiles, fused, st) : launch1<kFmtW4A16, false>(a, tok_tiles, fused, st);
  if (weight_fmt == MOE_FP4_E2M1)
    return packed ? launch1<MOE_FP4_E2M1, true>(a, tok_tiles, fused, st)
                  : launch1<MOE_FP4_E2M1, false>(a, tok_tiles, fused, st);
  return packed ? launch1<MOE_FP8_E4M3, true>(a, tok_tiles, fused, st)
                : launch1<MOE_FP8_E4M3, false>(a, tok_tiles, fused, st);
}

hipError_t launch_gemm2_lowp(const GemmArgs& a, int weight_fmt, int packed, int tok_tiles, hipStream_t st) {
  if (weight_fmt == kFmtW4A16)
    return packed ? launch2<kFmtW4A16, true>(a, tok_tiles, st) : launch2<kFmtW4A16, false>(a, tok_tiles, st);
  if (weight_fmt == MOE_FP4_E2M1)
    return packed ? launch2<MOE_FP4_E2M1, true>(a, tok_tiles, st) : launch2<MOE_FP4_E2M1, false>(a, tok_tiles, st);
  return packed ? launch2<MOE_FP8_E4M3, true>(a, tok_tiles, st) : launch2<MOE_FP8_E4M3, false>(a, tok_tiles, st);
}
