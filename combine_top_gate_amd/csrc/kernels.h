// Launchers of the HIP kernels; the host API (api.hip) is their only caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

// ---- dispatch ---------------------------------------------------------------
// One launch: route (counts, offsets, row maps) and scatter of the token rows.
constexpr int kMaxDispatchPairs = 1024;  // (token, slot) pairs per dispatch workgroup
struct DispatchArgs {
  const int32_t* ids;  // [S][T_s][k]
  int32_t* cnt;        // [S][E]
  int32_t* off;        // [S][E]
  int32_t* dst_row;    // [S][T_s][k]
  int32_t* row_src;    // [S*T_s*k]
  uint32_t* err;
  SrcPtrs src;
  uint8_t* win;        // [R][row_bytes]
  float* wsc;          // [R][nsc] or null
  int S, T_s, k, E;
  int row_bytes;       // bytes per token row (multiple of 16)
  int nsc;             // scales per row (0 = none)
  int tpb;             // tokens per workgroup (tpb * k <= kMaxDispatchPairs)
  // SENTINEL publication (all null under FENCE): per-source epoch flags
  uint32_t* rflag;     // [S] counts and offsets written
  uint32_t* dflag;     // [S] every window row of the source written
  uint32_t* arrive;    // [S] arrival counters (zero between calls)
  uint32_t epoch;
  uint32_t delay_ticks;  // SENTINEL test aid: each chunk waits this many 100 MHz ticks after
                         // publishing the counts, before it writes its window rows (0 = none)
};
int dispatch_tokens_per_block(int T_s, int k, int blocks_wanted, int S);
int dispatch_chunks(const DispatchArgs& a);  // workgroups per source
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t st);

// ---- grouped GEMMs ----------------------------------------------------------
// One launch covers every routed expert and, when present, the shared expert
// (group index E), which reads token rows straight from the source buffers.
struct GemmArgs {
  BatchDims d;
  const int32_t* cnt;
  const int32_t* off;
  // weights: routed base + per-expert strides, and the shared expert
  const uint8_t* w;
  const void* ws;
  int64_t w_stride;   // bytes per routed expert
  int64_t ws_stride;  // scale elements per routed expert
  const uint8_t* w_sh;
  const void* ws_sh;
  // activation rows (GEMM1: the window; GEMM2: the h window) and their scales
  const uint8_t* a;
  const float* as;
  SrcPtrs src;        // GEMM1 shared expert rows
  // outputs
  uint8_t* h;         // GEMM1: [R+T][hstride]
  float* hs;          // GEMM1: [R+T][hstride/128]
  uint16_t* y;        // GEMM2 (bf16): [R+T][H]
  float* yf;          // GEMM2 (F32): [R+T][H]
  uint32_t* err;
  int sh_chunks;      // the shared expert's rows are split into this many work items
  int sh_chunk_rows;  // rows per chunk (multiple of 16)
  // SENTINEL (GEMM1 of the routed experts): wait for rflag/dflag[s] == epoch; null = FENCE
  const uint32_t* rflag;
  const uint32_t* dflag;
  uint32_t epoch;
  uint32_t spin_limit;
  // GEMM2 with the combine in its epilogue (bf16 y and out); null ccnt: no combine here
  uint32_t* ccnt;          // [T][ceil(H/256)] contributions counted per token and column block, zero between calls
  const int32_t* dst_row;  // [T][k] window row of each slot, -1 for none
  const int32_t* row_src;  // [R] flattened (token, slot) pair of each window row
  const float* topk_w;     // [T][k]
  uint16_t* out;           // [T][H]
};
// The W4A16 variant of the decode GEMMs: MXFP4 weights (stored as MOE_FP4_E2M1), bf16
// activations and bf16 h.  Passed as weight_fmt; not a moe_dtype.
constexpr int kFmtW4A16 = 16;
// weight_fmt: MOE_FP8_E4M3, MOE_FP4_E2M1 or kFmtW4A16; packed: weights in the pack_layout.h order;
// tok_tiles: most 16-token tiles per pass (2..4)
// fused: also run these dispatch chunks in the launch's first workgroups (SENTINEL)
hipError_t launch_gemm1_lowp(const GemmArgs& a, int weight_fmt, int packed, int tok_tiles, hipStream_t st,
                             const DispatchArgs* fused = nullptr);
hipError_t launch_gemm2_lowp(const GemmArgs& a, int weight_fmt, int packed, int tok_tiles, hipStream_t st);
// Both low-precision GEMMs in one persistent launch (work queues, see gemm_lowp.hip).
struct ExpertsArgs {
  GemmArgs g1, g2;
  uint32_t* sched;      // [0..7] queue heads, [8] exit count, [16 + g] finished GEMM1 items of group g
  int nb1_r, nb1_s;     // GEMM1 items of a routed / the shared group
  int nb2;              // GEMM2 items of any group
  int per_xcd;          // 1: eight queues, one per XCD; 0: one queue
  uint32_t spin_limit;  // bound of the wait for a group's GEMM1 items
};
hipError_t launch_experts_lowp(const ExpertsArgs& a, int weight_fmt, int packed, int tok_tiles, int grid,
                               hipStream_t st);
int experts_lowp_blocks_per_cu(int weight_fmt, int packed, int tok_tiles, int k_slabs);
// LDS-tiled GEMMs for large expert row counts (FP8 weights; gemm_tiled.hip): a plan
// kernel, then GEMM1 and GEMM2 on persistent grids fed by atomic work counters.
struct TiledArgs {
  GemmArgs g1, g2;
  int* plan;           // tiled_plan_words() ints of workspace
  int nb1_r, nb1_s;    // GEMM1 column blocks (128 gate + 128 up) of a routed / the shared group
  int nb2;             // GEMM2 row blocks of 256
  int packed;          // weights in the pack_layout.h order
  int m32;             // K loop on 32x32x64 MFMAs (else 16x16x128)
};
hipError_t launch_tiled(const TiledArgs& a, int grid, hipStream_t st);
int tiled_plan_words();
hipError_t launch_gemm1_f32(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm2_f32(const GemmArgs& a, hipStream_t st);

// ---- weight repack (pack_layout.h) -----------------------------------------
struct PackArgs {
  const uint8_t* src;  // row-major weights (or e8m0 scales), E experts
  uint8_t* dst;        // packed
  int64_t src_stride, dst_stride;  // bytes per expert
  int E;
  int wfmt;            // MOE_FP8_E4M3 or MOE_FP4_E2M1
  int gemm1;           // 1: W13 (2*inter rows), 0: W2 (N = H rows)
  int K;               // contraction length (elements)
  int N;               // rows of the source matrix
  int inter;           // GEMM1: I of this weight set
  int nblk;            // GEMM1: inter/128; GEMM2: ceil(H/256)
};
hipError_t launch_pack(const PackArgs& a, bool scales, hipStream_t st);

// ---- combine ----------------------------------------------------------------
struct CombineArgs {
  const int32_t* dst_row;  // [S][T_s][k]
  const float* topk_w;     // [S][T_s][k]
  const void* y;           // [R+T][H] bf16 or f32
  void* out;               // [S][T_s][H] in y's dtype, or e4m3 codes when out_scale is set
  int T, k, H, R;
  int has_shared;
  int y_f32;               // y (and a plain out) are fp32
  float* out_scale;        // null: out in y's dtype; else FP8 out, f32 [S][T_s][H/128]
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// ---- gating (ahead of dispatch) ----------------------------------------------
struct RouterArgs {
  const uint16_t* x;   // [T][H] bf16
  const uint16_t* wr;  // [E][H] bf16
  float* logits;       // [T][E]
  int T, H, E;         // H a multiple of 32
};
hipError_t launch_router(const RouterArgs& a, hipStream_t st);

// Split-K router: partial[s][t][e] = sum over K slice s of x[t][h] * wr[e][h].
struct RouterSplitArgs {
  const uint16_t* x;   // [T][H] bf16
  const uint16_t* wr;  // [E][H] bf16
  float* partial;      // [ks][T][E]
  int T, H, E, ks;
};
// The split (ks) and token-tile width the fused gate uses for a shape; ks <= kGateMaxSplit.
constexpr int kGateMaxSplit = 16;
int gate_split(int T, int H, int E);
hipError_t launch_router_split(const RouterSplitArgs& a, hipStream_t st);

struct TopkArgs {
  const float* logits;  // [ks][T][E] fp32 partial sums, added in slice order; E <= 256
  float* logits_out;    // [T][E] the sums, or NULL (only with ks > 1)
  int32_t* ids;         // [T][k]
  float* w;             // [T][k]
  int T, E, k, ks;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

// ---- buffer fill (fill.hip) ------------------------------------------------------
// p 16-byte aligned; bytes a multiple of 4 (the remainder is not written).
hipError_t launch_fill32(void* p, size_t bytes, uint32_t pattern, hipStream_t st);

// ---- measurement aid ----------------------------------------------------------
hipError_t launch_mfma_fp8_probe(float* sink, int blocks, int iters, hipStream_t st);
int mfma_fp8_probe_chains();
hipError_t launch_mfma_dot(bool a_fp4, const uint8_t* a, const uint8_t* b, float* out, hipStream_t st);
