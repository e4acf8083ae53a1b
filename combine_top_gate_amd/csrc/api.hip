// Host side of the C-ABI: argument validation, workspace, launch sequencing, timing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "kernels.h"
#include "pack_layout.h"

namespace {

thread_local char g_msg[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr int kStages = 5;  // dispatch, gemm1, gemm2, combine, layer
constexpr int kSchedWords = 16 + MOE_MAX_EXPERTS + 1 + 15;
constexpr uint32_t kSpinLimit = 1u << 22;  // persistent GEMM: ~0.2 s of s_sleep polling
constexpr uint32_t kSentinelSpin = 1u << 20;  // SENTINEL GEMM1: polls before a wait gives up
constexpr int kXcds = 8;                     // CU mask bits are spread over the XCDs
constexpr double kTiledRows = 192.0;       // mean rows per expert from which the tiled GEMM runs
constexpr int kMaxDelayUs = 10000;          // SENTINEL dispatch delay cap, far below the wait limit

}  // namespace

struct moe_ctx {
  moe_config cfg{};
  int device = 0;
  int64_t R_cap = 0, rows_cap = 0;
  int hstride = 0;  // elements per h row = max(I, Ish)
  int act_bytes = 0;  // bytes per activation (and h) element: 1 FP8, 2 bf16, 4 fp32
  int row_bytes = 0;
  // workspace
  uint8_t* win = nullptr;
  float* wsc = nullptr;
  uint8_t* h = nullptr;
  float* hs = nullptr;
  void* y = nullptr;
  int32_t* cnt = nullptr;
  int32_t* off = nullptr;
  int32_t* dst_row = nullptr;
  int32_t* row_src = nullptr;
  uint32_t* err = nullptr;
  uint32_t* sched = nullptr;  // persistent GEMM: queue heads, exit count, per-group counters
  int* plan = nullptr;        // tiled GEMM: tile table and work counters
  uint32_t* sync = nullptr;   // SENTINEL: rflag[MOE_MAX_SRC], dflag[..], arrive[..]
  uint32_t* ccnt = nullptr;   // combine in GEMM2: [max tokens][ceil(H/256)] counters, zero between calls
  int n_cu = 0;
  // SENTINEL with dispatch_cus > 0: dispatch and GEMM1 streams on disjoint CU sets and
  // their fork/join events; with 0, the dispatch runs inside the GEMM1 launch
  hipStream_t s_disp = nullptr, s_comp = nullptr;
  hipEvent_t ev_fork = nullptr, ev_disp = nullptr, ev_g1 = nullptr;
  int dispatch_cus = 0;
  uint32_t epoch = 0;
  uint32_t spin_limit = kSentinelSpin;
  int opt_stall = 0;
  int opt_poison = 0;           // fill windows, h and y with NaN codes before each layer call
  uint32_t delay_ticks = 0;     // SENTINEL dispatch delay (100 MHz ticks), a test aid
  // options
  int opt_persistent = 0, opt_tiles = 0, opt_queue = 0, opt_tiled = 0, opt_tiled_m32 = 0;
  int opt_fcombine = 0;  // the combine in the decode GEMM2's epilogue
  // state of the last dispatch
  int T_s = -1;
  SrcPtrs src{};
  // timing
  int timing_cap = 0, timing_n = 0;
  std::vector<hipEvent_t> ev;  // timing_cap x (kStages+1)
};

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

BatchDims dims(const moe_ctx* c, int T_s) {
  BatchDims d;
  d.S = c->cfg.n_src;
  d.T_s = T_s;
  d.k = c->cfg.topk;
  d.E = c->cfg.n_experts;
  d.H = c->cfg.hidden;
  d.I = c->cfg.inter;
  d.Ish = c->cfg.shared_inter;
  d.R = d.S * d.T_s * d.k;
  d.T = d.S * d.T_s;
  d.hstride = c->hstride;
  return d;
}

BatchDims dims(const moe_ctx* c) { return dims(c, c->T_s); }

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->n_src < 1 || c->n_src > MOE_MAX_SRC)
    return fail(MOE_ERR_INVALID_ARG, "n_src %d outside 1..%d", c->n_src, MOE_MAX_SRC);
  if (c->max_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "max_tokens %d < 0", c->max_tokens);
  if (c->hidden <= 0 || c->hidden % 128 || c->hidden > MOE_MAX_DIM)
    return fail(MOE_ERR_INVALID_ARG, "hidden %d is not a positive multiple of 128 up to %d", c->hidden, MOE_MAX_DIM);
  if (c->inter <= 0 || c->inter % 128 || c->inter > MOE_MAX_DIM)
    return fail(MOE_ERR_INVALID_ARG, "inter %d is not a positive multiple of 128 up to %d", c->inter, MOE_MAX_DIM);
  if (c->shared_inter < 0 || c->shared_inter % 128 || c->shared_inter > MOE_MAX_DIM)
    return fail(MOE_ERR_INVALID_ARG, "shared_inter %d is not a multiple of 128 up to %d", c->shared_inter,
                MOE_MAX_DIM);
  if (c->n_experts < 1 || c->n_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "n_experts %d outside 1..%d", c->n_experts, MOE_MAX_EXPERTS);
  if (c->topk < 1 || c->topk > MOE_MAX_TOPK || c->topk > c->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "topk %d outside 1..min(%d, n_experts)", c->topk, MOE_MAX_TOPK);
  const bool fp8 = c->act == MOE_FP8_E4M3 && (c->weight == MOE_FP8_E4M3 || c->weight == MOE_FP4_E2M1) &&
                   c->out == MOE_BF16;
  const bool f32 = c->act == MOE_F32 && c->weight == MOE_F32 && c->out == MOE_F32;
  const bool w4a16 = c->act == MOE_BF16 && c->weight == MOE_FP4_E2M1 && c->out == MOE_BF16;
  if (!fp8 && !f32 && !w4a16)
    return fail(MOE_ERR_INVALID_ARG,
                "dtype combination act=%d weight=%d out=%d is not one of (fp8, fp8|fp4, bf16), "
                "(bf16, fp4, bf16) or (f32, f32, f32)",
                c->act, c->weight, c->out);
  if (c->sched != MOE_SCHED_FENCE && c->sched != MOE_SCHED_SENTINEL)
    return fail(MOE_ERR_INVALID_ARG, "unknown schedule %d", c->sched);
  if (c->dispatch_cus < 0 || c->dispatch_cus % kXcds)
    return fail(MOE_ERR_INVALID_ARG, "dispatch_cus %d is not 0 or a positive multiple of %d", c->dispatch_cus,
                kXcds);
  const int64_t R = (int64_t)c->n_src * c->max_tokens * c->topk;
  if (R > (int64_t)1 << 30) return fail(MOE_ERR_INVALID_ARG, "window of %lld rows is too large", (long long)R);
  return MOE_OK;
}

// Most 16-token tiles per pass of the low-precision GEMMs (each pass takes only the
// tiles it needs): enough for a typical expert (mean rows + two standard deviations
// of a multinomial count) in one pass, 2..4.
int tok_tiles(const BatchDims& d, int opt, bool fp4) {
  if (opt) return opt;
  const double mean = (double)d.R / d.E;
  const double want = mean + 2.0 * std::sqrt(mean);
  int nt = (int)std::ceil(want / 16.0);
  return std::min(fp4 ? 5 : 4, std::max(2, nt));
}

void record(moe_ctx* c, int stage, hipStream_t st) {
  if (c->timing_n < c->timing_cap) (void)hipEventRecord(c->ev[(size_t)c->timing_n * (kStages + 1) + stage], st);
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "unknown moe_status";
}

const char* moe_last_error_message(void) { return g_msg; }

moe_status moe_create(const moe_config* cfg, moe_ctx** out) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  moe_ctx* c = new moe_ctx();
  c->cfg = *cfg;
  auto cleanup = [&](moe_status s) {
    moe_destroy(c);
    return s;
  };
  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) return cleanup(fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e)));
  const bool f32 = cfg->act == MOE_F32, fp8 = cfg->act == MOE_FP8_E4M3;
  const int S = cfg->n_src, Tc = cfg->max_tokens, k = cfg->topk, E = cfg->n_experts, H = cfg->hidden;
  c->R_cap = (int64_t)S * Tc * k;
  c->rows_cap = c->R_cap + (int64_t)S * Tc;
  c->hstride = std::max(cfg->inter, cfg->shared_inter);
  c->act_bytes = f32 ? 4 : fp8 ? 1 : 2;
  c->row_bytes = c->act_bytes * H;
  const size_t one = 1;
  auto alloc = [&](void** p, size_t bytes) {
    return hipMalloc(p, std::max(bytes, one));
  };
  if ((e = alloc((void**)&c->win, (size_t)c->R_cap * c->row_bytes)) != hipSuccess ||
      (e = alloc((void**)&c->wsc, fp8 ? (size_t)c->R_cap * (H / 128) * 4 : 0)) != hipSuccess ||
      (e = alloc((void**)&c->h, (size_t)c->rows_cap * c->hstride * c->act_bytes)) != hipSuccess ||
      (e = alloc((void**)&c->hs, fp8 ? (size_t)c->rows_cap * (c->hstride / 128) * 4 : 0)) != hipSuccess ||
      (e = alloc(&c->y, (size_t)c->rows_cap * H * (f32 ? 4 : 2))) != hipSuccess ||
      (e = alloc((void**)&c->cnt, (size_t)S * E * 4)) != hipSuccess ||
      (e = alloc((void**)&c->off, (size_t)S * E * 4)) != hipSuccess ||
      // + MOE_MAX_TOPK entries: the combine reads a token's row map as whole vectors of
      // 2, 4, 8 or 16 entries, past the last token's k (never used)
      (e = alloc((void**)&c->dst_row, ((size_t)S * Tc * k + MOE_MAX_TOPK) * 4)) != hipSuccess ||
      (e = alloc((void**)&c->row_src, (size_t)c->R_cap * 4)) != hipSuccess ||
      (e = alloc((void**)&c->err, 4)) != hipSuccess ||
      (e = alloc((void**)&c->sched, kSchedWords * 4)) != hipSuccess ||
      (e = alloc((void**)&c->plan, (size_t)tiled_plan_words() * 4)) != hipSuccess ||
      (e = alloc((void**)&c->sync, 3 * MOE_MAX_SRC * 4)) != hipSuccess ||
      (e = alloc((void**)&c->ccnt, (size_t)S * Tc * ((H + 255) / 256) * 4)) != hipSuccess)
    return cleanup(fail(MOE_ERR_HIP, "workspace allocation failed: %s", hipGetErrorString(e)));
  if ((e = hipMemset(c->err, 0, 4)) != hipSuccess || (e = hipMemset(c->cnt, 0, (size_t)S * E * 4)) != hipSuccess ||
      (e = hipMemset(c->sched, 0, kSchedWords * 4)) != hipSuccess ||
      (e = hipMemset(c->off, 0, (size_t)S * E * 4)) != hipSuccess ||
      (e = hipMemset(c->sync, 0, 3 * MOE_MAX_SRC * 4)) != hipSuccess ||
      (e = hipMemset(c->ccnt, 0, (size_t)S * Tc * ((H + 255) / 256) * 4)) != hipSuccess)
    return cleanup(fail(MOE_ERR_HIP, "hipMemset: %s", hipGetErrorString(e)));
  hipDeviceProp_t prop;
  if ((e = hipGetDeviceProperties(&prop, c->device)) != hipSuccess)
    return cleanup(fail(MOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e)));
  c->n_cu = prop.multiProcessorCount;
  if (cfg->sched == MOE_SCHED_SENTINEL && cfg->dispatch_cus > 0) {
    // two streams on disjoint CU sets: dispatch gets dispatch_cus CUs, GEMM1 the rest
    const int dcu = cfg->dispatch_cus;
    if (dcu >= c->n_cu)
      return cleanup(fail(MOE_ERR_INVALID_ARG, "dispatch_cus %d leaves no CU of %d for the GEMM", dcu, c->n_cu));
    c->dispatch_cus = dcu;
    std::vector<uint32_t> dm((c->n_cu + 31) / 32, 0u), cm(dm.size(), 0u);
    for (int i = 0; i < c->n_cu; ++i) (i < dcu ? dm : cm)[i >> 5] |= 1u << (i & 31);
    if ((e = hipExtStreamCreateWithCUMask(&c->s_disp, (uint32_t)dm.size(), dm.data())) != hipSuccess ||
        (e = hipExtStreamCreateWithCUMask(&c->s_comp, (uint32_t)cm.size(), cm.data())) != hipSuccess)
      return cleanup(fail(MOE_ERR_UNSUPPORTED, "CU-masked streams for SENTINEL: %s", hipGetErrorString(e)));
    if ((e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&c->ev_disp, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&c->ev_g1, hipEventDisableTiming)) != hipSuccess)
      return cleanup(fail(MOE_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e)));
  }
  *out = c;
  return MOE_OK;
}

moe_status moe_destroy(moe_ctx* c) {
  if (!c) return MOE_OK;
  (void)hipDeviceSynchronize();
  for (auto ev : c->ev) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : {c->ev_fork, c->ev_disp, c->ev_g1})
    if (ev) (void)hipEventDestroy(ev);
  for (hipStream_t st : {c->s_disp, c->s_comp})
    if (st) (void)hipStreamDestroy(st);
  void* bufs[] = {c->win,     c->wsc,     c->h,   c->hs,    c->y,    c->cnt,
                  c->off,     c->dst_row, c->row_src, c->err, c->sched, c->plan, c->sync, c->ccnt};
  for (void* b : bufs)
    if (b) (void)hipFree(b);
  delete c;
  return MOE_OK;
}

}  // extern "C"

// Validates the dispatch arguments and fills `da` (nothing is launched; T_s == 0 leaves
// da.T_s = 0).  publish: SENTINEL flags for this call's epoch; blocks: workgroups
// the chunks should spread over.
static moe_status check_dispatch(const moe_ctx* c, int32_t T_s, const void* const* x, const float* const* x_scale,
                                 const int32_t* ids) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  const moe_config& cf = c->cfg;
  if (T_s < 0 || T_s > cf.max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "tokens_per_src %d outside 0..max_tokens (%d)", T_s, cf.max_tokens);
  const bool fp8 = cf.act == MOE_FP8_E4M3;
  if (T_s > 0) {
    if (!x) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
    if (fp8 && !x_scale) return fail(MOE_ERR_INVALID_ARG, "x_scale is NULL for FP8 activations");
    if (!ids) return fail(MOE_ERR_INVALID_ARG, "ids is NULL");
    for (int s = 0; s < cf.n_src; ++s) {
      if (!x[s] || !aligned16(x[s])) return fail(MOE_ERR_INVALID_ARG, "x[%d] is NULL or not 16-byte aligned", s);
      if (fp8 && (!x_scale[s] || ((uintptr_t)x_scale[s] & 3u)))
        return fail(MOE_ERR_INVALID_ARG, "x_scale[%d] is NULL or misaligned", s);
    }
  }
  return MOE_OK;
}

static moe_status dispatch_prepare(moe_ctx* c, int32_t T_s, const void* const* x, const float* const* x_scale,
                                   const int32_t* ids, bool publish, int blocks, DispatchArgs& da) {
  const moe_status st = check_dispatch(c, T_s, x, x_scale, ids);
  if (st != MOE_OK) return st;
  const moe_config& cf = c->cfg;
  const bool fp8 = cf.act == MOE_FP8_E4M3;
  SrcPtrs src{};
  for (int s = 0; s < cf.n_src && T_s > 0; ++s) {
    src.x[s] = static_cast<const uint8_t*>(x[s]);
    src.xs[s] = fp8 ? x_scale[s] : nullptr;
  }
  c->T_s = T_s;
  c->src = src;
  da = DispatchArgs{};
  if (T_s == 0) return MOE_OK;
  da.ids = ids;
  da.cnt = c->cnt;
  da.off = c->off;
  da.dst_row = c->dst_row;
  da.row_src = c->row_src;
  da.err = c->err;
  da.src = src;
  da.win = c->win;
  da.wsc = fp8 ? c->wsc : nullptr;
  da.S = cf.n_src;
  da.T_s = T_s;
  da.k = cf.topk;
  da.E = cf.n_experts;
  da.row_bytes = c->row_bytes;
  da.nsc = fp8 ? cf.hidden / 128 : 0;
  da.tpb = dispatch_tokens_per_block(T_s, cf.topk, blocks, cf.n_src);
  if (publish) {
    da.rflag = c->sync;
    da.dflag = c->sync + MOE_MAX_SRC;
    da.arrive = c->sync + 2 * MOE_MAX_SRC;
    da.epoch = c->epoch;
    da.delay_ticks = c->delay_ticks;
  }
  return MOE_OK;
}

// Validates and launches the dispatch kernel (about four workgroups per CU it may use).
static moe_status dispatch_impl(moe_ctx* c, int32_t T_s, const void* const* x, const float* const* x_scale,
                                const int32_t* ids, hipStream_t stream, bool publish) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  DispatchArgs da;
  moe_status st = dispatch_prepare(c, T_s, x, x_scale, ids, publish, 4 * (publish ? c->dispatch_cus : c->n_cu), da);
  if (st != MOE_OK || da.T_s == 0) return st;
  HIP_TRY(launch_dispatch(da, stream));
  return MOE_OK;
}

extern "C" {

moe_status moe_dispatch(moe_ctx* c, int32_t T_s, const void* const* x, const float* const* x_scale,
                        const int32_t* ids, hipStream_t stream) {
  return dispatch_impl(c, T_s, x, x_scale, ids, stream, false);
}

static bool use_tiled(const moe_ctx* c, const BatchDims& d) {
  const moe_config& cf = c->cfg;
  if (cf.act == MOE_F32 || cf.weight == MOE_FP4_E2M1) return false;
  return c->opt_tiled == 1 || (c->opt_tiled == 0 && (double)d.R / d.E >= kTiledRows);
}

// SENTINEL overlaps dispatch with the decode GEMM1 (weight-streaming kernels, two
// launches); the tiled prefill, fp32 and persistent paths run in stream order.
static bool sentinel_applies(const moe_ctx* c, int T_s) {
  const bool persistent = c->opt_persistent && c->cfg.act != MOE_BF16;  // W4A16 always runs two kernels
  if (c->cfg.sched != MOE_SCHED_SENTINEL || c->cfg.act == MOE_F32 || persistent || T_s <= 0) return false;
  return !use_tiled(c, dims(c, T_s));
}

// The weight pointers of a call (nothing is launched).
static moe_status check_weights(const moe_ctx* c, const moe_weights* w) {
  const moe_config& cf = c->cfg;
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  const bool f32 = cf.act == MOE_F32, fp4 = cf.weight == MOE_FP4_E2M1;
  if (!w->w13 || !w->w2 || (!f32 && (!w->s13 || !w->s2)))
    return fail(MOE_ERR_INVALID_ARG, "routed expert weight or scale pointer is NULL");
  if (!aligned16(w->w13) || !aligned16(w->w2)) return fail(MOE_ERR_INVALID_ARG, "weights not 16-byte aligned");
  if (w->packed && f32) return fail(MOE_ERR_INVALID_ARG, "F32 weights have no packed form");
  if (w->packed && fp4 && (((uintptr_t)w->s13 | (uintptr_t)w->s2) & 3u))
    return fail(MOE_ERR_INVALID_ARG, "packed e8m0 scales must be 4-byte aligned");
  if (cf.shared_inter) {
    if (!w->sh_w13 || !w->sh_w2 || (!f32 && (!w->sh_s13 || !w->sh_s2)))
      return fail(MOE_ERR_INVALID_ARG, "shared expert weight or scale pointer is NULL");
    if (!aligned16(w->sh_w13) || !aligned16(w->sh_w2))
      return fail(MOE_ERR_INVALID_ARG, "shared weights not 16-byte aligned");
  }
  return MOE_OK;
}

// Test aid (MOE_OPT_POISON): windows, their scales, h, its scales and y filled with NaN
// codes of their formats, so that a kernel reading a row the call has not written
// produces NaN.
static moe_status poison(moe_ctx* c, hipStream_t stream) {
  const moe_config& cf = c->cfg;
  const bool f32 = cf.act == MOE_F32, fp8 = cf.act == MOE_FP8_E4M3;
  const uint32_t act = f32 ? 0x7FC00000u : fp8 ? 0x7F7F7F7Fu : 0x7FC07FC0u;  // e4m3 NaN 0x7F, bf16 NaN
  const uint32_t out = f32 ? 0x7FC00000u : 0x7FC07FC0u;
  const int H = cf.hidden;
  HIP_TRY(launch_fill32(c->win, (size_t)c->R_cap * c->row_bytes, act, stream));
  HIP_TRY(launch_fill32(c->h, (size_t)c->rows_cap * c->hstride * c->act_bytes, act, stream));
  HIP_TRY(launch_fill32(c->y, (size_t)c->rows_cap * H * (f32 ? 4 : 2), out, stream));
  if (fp8) {
    HIP_TRY(launch_fill32(c->wsc, (size_t)c->R_cap * (H / 128) * 4, 0x7FC00000u, stream));
    HIP_TRY(launch_fill32(c->hs, (size_t)c->rows_cap * (c->hstride / 128) * 4, 0x7FC00000u, stream));
  }
  return MOE_OK;
}

// sn: SENTINEL -- GEMM1 polls the dispatch's flags.  fused != null: the dispatch chunks
// run in the GEMM1 launch itself, on `stream`; otherwise GEMM1 runs on the compute
// stream and GEMM2 joins both streams back into `stream`.
// combine != null (moe_layer): {topk_w, out}; with MOE_OPT_FUSED_COMBINE on a path that
// takes it, GEMM2 also forms the combine and *combined is set.
struct CombineTarget {
  const float* topk_w;
  void* out;
  bool combined;
};
static moe_status gemm_stage(moe_ctx* c, const moe_weights* w, hipStream_t stream, bool timed, bool sn = false,
                             const DispatchArgs* fused = nullptr, CombineTarget* combine = nullptr) {
  const moe_config& cf = c->cfg;
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (c->T_s < 0) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm before any moe_dispatch");
  const bool f32 = cf.act == MOE_F32, fp4 = cf.weight == MOE_FP4_E2M1, a16 = cf.act == MOE_BF16;
  // the kernel variant: FP8 or MXFP4 weights with FP8 activations, or W4A16
  const int wf = a16 ? kFmtW4A16 : cf.weight;
  const moe_status wst = check_weights(c, w);
  if (wst != MOE_OK) return wst;
  if (c->T_s == 0) {
    if (timed) { record(c, 2, stream); }
    return MOE_OK;
  }
  const BatchDims d = dims(c);
  const int64_t H = cf.hidden, I = cf.inter;
  GemmArgs g{};
  g.d = d;
  g.cnt = c->cnt;
  g.off = c->off;
  g.src = c->src;
  g.err = c->err;
  const bool packed = w->packed != 0;
  // GEMM1
  g.w = static_cast<const uint8_t*>(w->w13);
  g.ws = w->s13;
  g.w_sh = static_cast<const uint8_t*>(w->sh_w13);
  g.ws_sh = w->sh_s13;
  if (f32) {
    g.w_stride = 2 * I * H * 4;
  } else if (fp4) {
    g.w_stride = packed_w13_bytes(MOE_FP4_E2M1, (int)H, (int)I);
    g.ws_stride = packed_e13_bytes((int)H, (int)I);
  } else {
    g.w_stride = packed_w13_bytes(MOE_FP8_E4M3, (int)H, (int)I);
    g.ws_stride = (2 * I / 128) * (H / 128);
  }
  g.a = c->win;
  g.as = c->wsc;
  g.h = c->h;
  g.hs = c->hs;
  // W4A16 with row-major weights: at most 4 token tiles (with 5 the kernels spill registers)
  const int nt = a16 && !packed ? std::min(4, tok_tiles(d, c->opt_tiles, fp4)) : tok_tiles(d, c->opt_tiles, fp4);
  // the shared expert (all T rows): chunks of at most one pass each, as separate work items
  g.sh_chunk_rows = 16 * nt;
  g.sh_chunks = d.Ish ? std::max(1, (d.T + g.sh_chunk_rows - 1) / g.sh_chunk_rows) : 1;
  GemmArgs g1 = g;
  // many rows per expert: the LDS-tiled, MFMA-bound kernels (FP8 weights)
  const bool tiled = use_tiled(c, d);
  if (d.Ish && !c->opt_tiles && !tiled && !f32 && (sn || a16 || !c->opt_persistent)) {
    // GEMM1 as its own launch: its shared-expert items run after every routed item (the
    // kernel's work order), in chunks of two token tiles, short items that spread over
    // the workgroups the routed items leave; GEMM2 keeps chunks of whole passes.
    // Measured at the 256-token layers, shared chunks of 5 / 4 / 2 / 1 tiles: GEMM1
    // MXFP4 171.8 / 157.8 / 147.5 / 147.5 us, W4A16 - / 162.5 / 164.5 / 165.8 us (with
    // whole-pass chunks among the routed items, as before: 168.8 and 237.5 us)
    g1.sh_chunk_rows = 32;
    g1.sh_chunks = (d.T + 31) / 32;
  }
  if (sn) {
    g1.rflag = c->sync;
    g1.dflag = c->sync + MOE_MAX_SRC;
    g1.epoch = c->opt_stall ? c->epoch ^ 0x80000000u : c->epoch;  // stall: an epoch never published
    g1.spin_limit = c->spin_limit;
    if (fused) {
      HIP_TRY(launch_gemm1_lowp(g1, wf, packed, nt, stream, fused));
      if (timed) record(c, 2, stream);
    } else {
      HIP_TRY(launch_gemm1_lowp(g1, wf, packed, nt, c->s_comp));
      if (timed) record(c, 2, c->s_comp);
      HIP_TRY(hipEventRecord(c->ev_g1, c->s_comp));
      HIP_TRY(hipStreamWaitEvent(stream, c->ev_disp, 0));
      HIP_TRY(hipStreamWaitEvent(stream, c->ev_g1, 0));
    }
  } else if (!tiled && (f32 || a16 || !c->opt_persistent)) {
    HIP_TRY(f32 ? launch_gemm1_f32(g1, stream) : launch_gemm1_lowp(g1, wf, packed, nt, stream));
    if (timed) record(c, 2, stream);
  }
  // GEMM2
  g.w = static_cast<const uint8_t*>(w->w2);
  g.ws = w->s2;
  g.w_sh = static_cast<const uint8_t*>(w->sh_w2);
  g.ws_sh = w->sh_s2;
  if (f32) {
    g.w_stride = H * I * 4;
  } else if (fp4) {
    g.w_stride = packed ? packed_w2_bytes(MOE_FP4_E2M1, (int)H, (int)I) : H * (I / 2);
    g.ws_stride = packed ? packed_e2_bytes((int)H, (int)I) : H * (I / 32);
  } else {
    g.w_stride = packed ? packed_w2_bytes(MOE_FP8_E4M3, (int)H, (int)I) : H * I;
    g.ws_stride = (H / 128) * (I / 128);
  }
  g.a = c->h;
  g.as = c->hs;
  g.y = static_cast<uint16_t*>(c->y);
  g.yf = static_cast<float*>(c->y);
  if (tiled) {
    TiledArgs ta{};
    ta.g1 = g1;
    ta.g2 = g;
    ta.plan = c->plan;
    ta.nb1_r = d.I / 128;
    ta.nb1_s = d.Ish / 128;
    ta.nb2 = (d.H + 255) / 256;
    ta.packed = packed;
    ta.m32 = c->opt_tiled_m32;
    HIP_TRY(launch_tiled(ta, c->n_cu, stream));
    if (timed) record(c, 2, stream);
    return MOE_OK;
  }
  if (!f32 && combine && c->opt_fcombine) {
    // the combine in GEMM2's epilogue (the decode kernels, two-kernel or persistent)
    g.ccnt = c->ccnt;
    g.dst_row = c->dst_row;
    g.row_src = c->row_src;
    g.topk_w = combine->topk_w;
    g.out = static_cast<uint16_t*>(combine->out);
    combine->combined = true;
  }
  if (f32 || a16 || !c->opt_persistent || sn) {
    HIP_TRY(f32 ? launch_gemm2_f32(g, stream) : launch_gemm2_lowp(g, wf, packed, nt, stream));
    return MOE_OK;
  }
  ExpertsArgs ea{};
  ea.g1 = g1;
  ea.g2 = g;
  ea.sched = c->sched;
  ea.nb1_r = d.I / 128;
  ea.nb1_s = d.Ish / 128;
  ea.nb2 = (d.H + 255) / 256;
  const double mean_rows = (double)d.R / d.E;
  ea.per_xcd = c->opt_queue ? c->opt_queue == 1 : (d.E >= 16 && mean_rows <= 256.0);
  ea.spin_limit = kSpinLimit;
  const int groups = d.E + (d.Ish ? 1 : 0);
  const int items = d.E * ea.nb1_r + ea.nb1_s * g.sh_chunks + d.E * ea.nb2 + (d.Ish ? ea.nb2 * g.sh_chunks : 0);
  (void)groups;
  const int per_cu = std::max(1, experts_lowp_blocks_per_cu(cf.weight, packed, nt, std::max(d.H, d.hstride) / 128));
  int grid = std::min(items, per_cu * c->n_cu);
  if (ea.per_xcd) grid = std::max(8, grid / 8 * 8);
  HIP_TRY(launch_experts_lowp(ea, cf.weight, packed, nt, grid, stream));
  if (timed) record(c, 2, stream);
  return MOE_OK;
}

moe_status moe_grouped_gemm(moe_ctx* c, const moe_weights* w, hipStream_t stream) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  return gemm_stage(c, w, stream, false);
}

moe_status moe_combine(moe_ctx* c, const float* topk_w, void* out, hipStream_t stream) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  if (c->T_s < 0) return fail(MOE_ERR_INVALID_ARG, "moe_combine before any moe_dispatch");
  if (c->T_s == 0) return MOE_OK;
  if (!topk_w || !out) return fail(MOE_ERR_INVALID_ARG, "topk_w or out is NULL");
  if (!aligned16(out)) return fail(MOE_ERR_INVALID_ARG, "out is not 16-byte aligned");
  const moe_config& cf = c->cfg;
  const BatchDims d = dims(c);
  CombineArgs a{c->dst_row, topk_w, c->y, out, d.T, d.k, d.H, d.R, cf.shared_inter > 0, cf.out == MOE_F32, nullptr};
  HIP_TRY(launch_combine(a, stream));
  return MOE_OK;
}

moe_status moe_combine_fp8(moe_ctx* c, const float* topk_w, uint8_t* out, float* out_scale, hipStream_t stream) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  if (c->T_s < 0) return fail(MOE_ERR_INVALID_ARG, "moe_combine_fp8 before any moe_dispatch");
  if (c->T_s == 0) return MOE_OK;
  if (!topk_w || !out || !out_scale) return fail(MOE_ERR_INVALID_ARG, "topk_w, out or out_scale is NULL");
  if (!aligned16(out) || ((uintptr_t)out_scale & 3u))
    return fail(MOE_ERR_INVALID_ARG, "out is not 16-byte aligned or out_scale not 4-byte aligned");
  const moe_config& cf = c->cfg;
  const BatchDims d = dims(c);
  CombineArgs a{c->dst_row, topk_w, c->y, out, d.T, d.k, d.H, d.R, cf.shared_inter > 0, cf.out == MOE_F32, out_scale};
  HIP_TRY(launch_combine(a, stream));
  return MOE_OK;
}

moe_status moe_layer(moe_ctx* c, int32_t T_s, const void* const* x, const float* const* x_scale,
                     const int32_t* ids, const float* topk_w, const moe_weights* w, void* out,
                     hipStream_t stream) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  moe_status st = check_weights(c, w);
  if (st != MOE_OK) return st;
  if (T_s > 0 && (!topk_w || !out)) return fail(MOE_ERR_INVALID_ARG, "topk_w or out is NULL");
  if (T_s > 0 && !aligned16(out)) return fail(MOE_ERR_INVALID_ARG, "out is not 16-byte aligned");
  st = check_dispatch(c, T_s, x, x_scale, ids);  // every argument is checked before anything is enqueued
  if (st != MOE_OK) return st;
  const bool timed = c->timing_n < c->timing_cap;
  const bool sn = sentinel_applies(c, T_s);
  if (sn || timed) {
    // a replayed graph would repeat this call's epoch, or its timing events
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(stream, &cs));
    if (cs != hipStreamCaptureStatusNone)
      return fail(MOE_ERR_INVALID_ARG, "%s cannot be captured into a graph",
                  sn ? "a SENTINEL layer call (per-call epoch)" : "a timed layer call");
  }
  if (c->opt_poison && T_s > 0) {
    st = poison(c, stream);
    if (st != MOE_OK) return st;
  }
  if (timed) record(c, 0, stream);
  DispatchArgs fused;
  const bool use_fused = sn && c->dispatch_cus == 0;
  if (use_fused) {
    // the dispatch chunks run in the prologue of the GEMM1 launch's first workgroups
    // (at most one chunk per CU's worth of workgroups)
    c->epoch = c->epoch + 1 ? c->epoch + 1 : 1;  // 0 (the flags' initial value) is never an epoch
    st = dispatch_prepare(c, T_s, x, x_scale, ids, true, c->n_cu / 2, fused);
    if (st != MOE_OK) return st;
    fused.rflag = nullptr;  // the GEMM1 workgroups wait for the rows flags only
    if (timed) record(c, 1, stream);
  } else if (sn) {
    // fork: dispatch and GEMM1 start together on their CU sets once `stream` is here
    HIP_TRY(hipEventRecord(c->ev_fork, stream));
    HIP_TRY(hipStreamWaitEvent(c->s_disp, c->ev_fork, 0));
    HIP_TRY(hipStreamWaitEvent(c->s_comp, c->ev_fork, 0));
    c->epoch = c->epoch + 1 ? c->epoch + 1 : 1;  // 0 (the flags' initial value) is never an epoch
    st = dispatch_impl(c, T_s, x, x_scale, ids, c->s_disp, true);
    if (st != MOE_OK) return st;
    if (timed) record(c, 1, c->s_disp);
    HIP_TRY(hipEventRecord(c->ev_disp, c->s_disp));
  } else {
    st = dispatch_impl(c, T_s, x, x_scale, ids, stream, false);
    if (st != MOE_OK) return st;
    if (timed) record(c, 1, stream);
  }
  CombineTarget ct{topk_w, out, false};
  st = gemm_stage(c, w, stream, timed, sn, use_fused ? &fused : nullptr, &ct);
  if (st != MOE_OK) return st;
  if (timed) record(c, 3, stream);
  if (!ct.combined) {
    st = moe_combine(c, topk_w, out, stream);
    if (st != MOE_OK) return st;
  }
  if (timed) {
    record(c, 4, stream);
    c->timing_n++;
  }
  return MOE_OK;
}

moe_status moe_get_routing(moe_ctx* c, int32_t* cnt, int32_t* off, int32_t* dst_row, int32_t* row_src,
                           hipStream_t stream) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  if (c->T_s < 0) return fail(MOE_ERR_INVALID_ARG, "no dispatch yet");
  const moe_config& cf = c->cfg;
  const size_t SE = (size_t)cf.n_src * cf.n_experts * 4, R = (size_t)cf.n_src * c->T_s * cf.topk * 4;
  if (cnt) HIP_TRY(hipMemcpyAsync(cnt, c->cnt, SE, hipMemcpyDeviceToDevice, stream));
  if (off) HIP_TRY(hipMemcpyAsync(off, c->off, SE, hipMemcpyDeviceToDevice, stream));
  if (dst_row && R) HIP_TRY(hipMemcpyAsync(dst_row, c->dst_row, R, hipMemcpyDeviceToDevice, stream));
  if (row_src && R) HIP_TRY(hipMemcpyAsync(row_src, c->row_src, R, hipMemcpyDeviceToDevice, stream));
  return MOE_OK;
}

moe_status moe_copy_buffer(moe_ctx* c, moe_buffer which, void* dst, size_t bytes, hipStream_t stream) {
  if (!c || !dst) return fail(MOE_ERR_INVALID_ARG, "ctx or dst is NULL");
  const bool f32 = c->cfg.act == MOE_F32, fp8 = c->cfg.act == MOE_FP8_E4M3;
  const int H = c->cfg.hidden;
  const void* src = nullptr;
  size_t cap = 0;
  switch (which) {
    case MOE_BUF_WINDOW: src = c->win; cap = (size_t)c->R_cap * c->row_bytes; break;
    case MOE_BUF_WSCALE: src = c->wsc; cap = fp8 ? (size_t)c->R_cap * (H / 128) * 4 : 0; break;
    case MOE_BUF_H: src = c->h; cap = (size_t)c->rows_cap * c->hstride * c->act_bytes; break;
    case MOE_BUF_HSCALE: src = c->hs; cap = fp8 ? (size_t)c->rows_cap * (c->hstride / 128) * 4 : 0; break;
    case MOE_BUF_Y: src = c->y; cap = (size_t)c->rows_cap * H * (f32 ? 4 : 2); break;
    default: return fail(MOE_ERR_INVALID_ARG, "unknown buffer %d", (int)which);
  }
  if (bytes > cap) return fail(MOE_ERR_INVALID_ARG, "%zu bytes requested, buffer holds %zu", bytes, cap);
  if (bytes) HIP_TRY(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, stream));
  return MOE_OK;
}

moe_status moe_packed_sizes(const moe_config* cfg, size_t sizes[8]) {
  if (!sizes) return fail(MOE_ERR_INVALID_ARG, "sizes is NULL");
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->weight == MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "F32 weights have no packed form");
  const int H = cfg->hidden, I = cfg->inter, Ish = cfg->shared_inter;
  const size_t E = cfg->n_experts;
  const bool fp4 = cfg->weight == MOE_FP4_E2M1;
  auto sc13 = [&](int inter) { return fp4 ? (size_t)packed_e13_bytes(H, inter) : (size_t)(2 * inter / 128) * (H / 128) * 4; };
  auto sc2 = [&](int inter) { return fp4 ? (size_t)packed_e2_bytes(H, inter) : (size_t)(H / 128) * (inter / 128) * 4; };
  sizes[0] = E * packed_w13_bytes(cfg->weight, H, I);
  sizes[1] = E * sc13(I);
  sizes[2] = E * packed_w2_bytes(cfg->weight, H, I);
  sizes[3] = E * sc2(I);
  sizes[4] = Ish ? (size_t)packed_w13_bytes(cfg->weight, H, Ish) : 0;
  sizes[5] = Ish ? sc13(Ish) : 0;
  sizes[6] = Ish ? (size_t)packed_w2_bytes(cfg->weight, H, Ish) : 0;
  sizes[7] = Ish ? sc2(Ish) : 0;
  return MOE_OK;
}

moe_status moe_pack_weights(moe_ctx* c, const moe_weights* src, const moe_weights* dst, hipStream_t stream) {
  if (!c || !src || !dst) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  const moe_config& cf = c->cfg;
  if (cf.weight == MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "F32 weights have no packed form");
  if (src->packed || !dst->packed) return fail(MOE_ERR_INVALID_ARG, "src must be row-major and dst packed");
  size_t sz[8];
  moe_status st = moe_packed_sizes(&cf, sz);
  if (st != MOE_OK) return st;
  const void* s8[8] = {src->w13, src->s13, src->w2, src->s2, src->sh_w13, src->sh_s13, src->sh_w2, src->sh_s2};
  const void* d8[8] = {dst->w13, dst->s13, dst->w2, dst->s2, dst->sh_w13, dst->sh_s13, dst->sh_w2, dst->sh_s2};
  for (int i = 0; i < 8; ++i)
    if (sz[i] && (!s8[i] || !d8[i])) return fail(MOE_ERR_INVALID_ARG, "weight buffer %d is NULL", i);
  for (int i = 0; i < 8; ++i)
    if (sz[i] && (!aligned16(s8[i]) || !aligned16(d8[i])))
      return fail(MOE_ERR_INVALID_ARG, "weight buffer %d is not 16-byte aligned", i);
  const int H = cf.hidden, wf = cf.weight;
  const bool fp4 = wf == MOE_FP4_E2M1;
  auto pack_set = [&](int E, int inter, int i13, int i2) -> moe_status {
    PackArgs a{};
    a.E = E;
    a.wfmt = wf;
    // W13: [2*inter][H]
    a.src = static_cast<const uint8_t*>(s8[i13]);
    a.dst = static_cast<uint8_t*>(const_cast<void*>(d8[i13]));
    a.src_stride = (int64_t)2 * inter * H / (fp4 ? 2 : 1);
    a.dst_stride = packed_w13_bytes(wf, H, inter);
    a.gemm1 = 1; a.K = H; a.N = 2 * inter; a.inter = inter; a.nblk = inter / 128;
    HIP_TRY(launch_pack(a, false, stream));
    if (fp4) {
      a.src = static_cast<const uint8_t*>(s8[i13 + 1]);
      a.dst = static_cast<uint8_t*>(const_cast<void*>(d8[i13 + 1]));
      a.src_stride = (int64_t)2 * inter * (H / 32);
      a.dst_stride = packed_e13_bytes(H, inter);
      HIP_TRY(launch_pack(a, true, stream));
    } else {
      HIP_TRY(hipMemcpyAsync(const_cast<void*>(d8[i13 + 1]), s8[i13 + 1], sz[i13 + 1], hipMemcpyDeviceToDevice, stream));
    }
    // W2: [H][inter]
    a.src = static_cast<const uint8_t*>(s8[i2]);
    a.dst = static_cast<uint8_t*>(const_cast<void*>(d8[i2]));
    a.src_stride = (int64_t)H * inter / (fp4 ? 2 : 1);
    a.dst_stride = packed_w2_bytes(wf, H, inter);
    a.gemm1 = 0; a.K = inter; a.N = H; a.inter = inter; a.nblk = (H + 255) / 256;
    HIP_TRY(launch_pack(a, false, stream));
    if (fp4) {
      a.src = static_cast<const uint8_t*>(s8[i2 + 1]);
      a.dst = static_cast<uint8_t*>(const_cast<void*>(d8[i2 + 1]));
      a.src_stride = (int64_t)H * (inter / 32);
      a.dst_stride = packed_e2_bytes(H, inter);
      HIP_TRY(launch_pack(a, true, stream));
    } else {
      HIP_TRY(hipMemcpyAsync(const_cast<void*>(d8[i2 + 1]), s8[i2 + 1], sz[i2 + 1], hipMemcpyDeviceToDevice, stream));
    }
    return MOE_OK;
  };
  st = pack_set(cf.n_experts, cf.inter, 0, 2);
  if (st != MOE_OK) return st;
  if (cf.shared_inter) st = pack_set(1, cf.shared_inter, 4, 6);
  return st;
}

moe_status moe_set_option(moe_ctx* c, moe_option opt, int32_t v) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  switch (opt) {
    case MOE_OPT_PERSISTENT_GEMM:
      if (v != 0 && v != 1) break;
      c->opt_persistent = v;
      return MOE_OK;
    case MOE_OPT_TOKEN_TILES:
      if (v != 0 && (v < 2 || v > 6)) break;
      c->opt_tiles = v;
      return MOE_OK;
    case MOE_OPT_QUEUE:
      if (v < 0 || v > 2) break;
      c->opt_queue = v;
      return MOE_OK;
    case MOE_OPT_TILED_GEMM:
      if (v < 0 || v > 2) break;
      c->opt_tiled = v;
      return MOE_OK;
    case MOE_OPT_SENTINEL_SPIN:
      if (v < 0) break;
      c->spin_limit = v ? (uint32_t)v : kSentinelSpin;
      return MOE_OK;
    case MOE_OPT_SENTINEL_STALL:
      if (v != 0 && v != 1) break;
      c->opt_stall = v;
      return MOE_OK;
    case MOE_OPT_TILED_MFMA:
      if (v != 0 && v != 1) break;
      c->opt_tiled_m32 = v;
      return MOE_OK;
    case MOE_OPT_POISON:
      if (v != 0 && v != 1) break;
      c->opt_poison = v;
      return MOE_OK;
    case MOE_OPT_EPOCH: {
      // the flags may hold any earlier epoch: clear them, with the device idle
      HIP_TRY(hipDeviceSynchronize());
      HIP_TRY(hipMemset(c->sync, 0, 3 * MOE_MAX_SRC * 4));
      c->epoch = (uint32_t)v;
      return MOE_OK;
    }
    case MOE_OPT_DISPATCH_DELAY:
      if (v < 0 || v > kMaxDelayUs) break;
      c->delay_ticks = (uint32_t)v * 100u;  // the real-time counter runs at 100 MHz
      return MOE_OK;
    case MOE_OPT_FUSED_COMBINE:
      if (v != 0 && v != 1) break;
      c->opt_fcombine = v;
      return MOE_OK;
  }
  return fail(MOE_ERR_INVALID_ARG, "option %d does not take value %d", (int)opt, v);
}

moe_status moe_router_logits(int32_t T, int32_t H, int32_t E, const void* x, const void* wr, float* logits,
                             hipStream_t stream) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T %d < 0", T);
  if (H <= 0 || H % 32) return fail(MOE_ERR_INVALID_ARG, "H %d is not a positive multiple of 32", H);
  if (E < 1 || E > MOE_MAX_GATE_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "E %d outside 1..%d", E, MOE_MAX_GATE_EXPERTS);
  if (T == 0) return MOE_OK;
  if (!x || !wr || !logits) return fail(MOE_ERR_INVALID_ARG, "x, wr or logits is NULL");
  if (!aligned16(x) || !aligned16(wr) || ((uintptr_t)logits & 3u))
    return fail(MOE_ERR_INVALID_ARG, "x and wr must be 16-byte aligned, logits 4-byte aligned");
  RouterArgs a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr), logits, T, H, E};
  HIP_TRY(launch_router(a, stream));
  return MOE_OK;
}

moe_status moe_topk_softmax(int32_t T, int32_t E, int32_t k, const float* logits, int32_t* ids, float* w,
                            hipStream_t stream) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T %d < 0", T);
  if (E < 1 || E > MOE_MAX_GATE_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "E %d outside 1..%d", E, MOE_MAX_GATE_EXPERTS);
  if (k < 1 || k > MOE_MAX_TOPK || k > E)
    return fail(MOE_ERR_INVALID_ARG, "k %d outside 1..min(%d, E)", k, MOE_MAX_TOPK);
  if (T == 0) return MOE_OK;
  if (!logits || !ids || !w) return fail(MOE_ERR_INVALID_ARG, "logits, ids or w is NULL");
  if (((uintptr_t)logits | (uintptr_t)ids | (uintptr_t)w) & 3u)
    return fail(MOE_ERR_INVALID_ARG, "logits, ids and w must be 4-byte aligned");
  TopkArgs a{logits, nullptr, ids, w, T, E, k, 1};
  HIP_TRY(launch_topk(a, stream));
  return MOE_OK;
}

size_t moe_gate_workspace_bytes(int32_t T, int32_t H, int32_t E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  return (size_t)gate_split(T, H, E) * (size_t)T * (size_t)E * sizeof(float);
}

}  // extern "C"

// Argument checks of the fused gate (nothing is enqueued); workspace may be null when
// need_ws is false.
static moe_status gate_check(int32_t T, int32_t H, int32_t E, int32_t k, const void* x, const void* wr,
                             const void* workspace, bool need_ws, const float* logits, const int32_t* ids,
                             const float* w) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T %d < 0", T);
  if (H <= 0 || H % 32) return fail(MOE_ERR_INVALID_ARG, "H %d is not a positive multiple of 32", H);
  if (E < 1 || E > MOE_MAX_GATE_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "E %d outside 1..%d", E, MOE_MAX_GATE_EXPERTS);
  if (k < 1 || k > MOE_MAX_TOPK || k > E)
    return fail(MOE_ERR_INVALID_ARG, "k %d outside 1..min(%d, E)", k, MOE_MAX_TOPK);
  if (T == 0) return MOE_OK;
  if (!x || !wr || (need_ws && !workspace) || !ids || !w)
    return fail(MOE_ERR_INVALID_ARG, "x, wr, workspace, ids or w is NULL");
  if (!aligned16(x) || !aligned16(wr) || (need_ws && !aligned16(workspace)))
    return fail(MOE_ERR_INVALID_ARG, "x, wr and workspace must be 16-byte aligned");
  if (((uintptr_t)ids | (uintptr_t)w | (uintptr_t)logits) & 3u)
    return fail(MOE_ERR_INVALID_ARG, "logits, ids and w must be 4-byte aligned");
  return MOE_OK;
}

// The two launches of the fused gate, partial sums in `part` (ks x T x E fp32).
static moe_status gate_launch(int32_t T, int32_t H, int32_t E, int32_t k, const void* x, const void* wr, float* part,
                              float* logits, int32_t* ids, float* w, hipStream_t stream) {
  const int ks = gate_split(T, H, E);
  RouterSplitArgs ra{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr), part, T, H, E, ks};
  HIP_TRY(launch_router_split(ra, stream));
  TopkArgs ta{part, logits, ids, w, T, E, k, ks};
  HIP_TRY(launch_topk(ta, stream));
  return MOE_OK;
}

// Scratch of moe_gate_noalloc: one array per GPU, in the library's device code, holding
// the router's partial sums.  In host code `scratch` only names the symbol; its device
// address (a different one on every GPU) comes from hipGetSymbolAddress, looked up once
// per device on the first call there and kept in g_scratch_dev.
static __device__ __align__(256) uint8_t scratch[MOE_GATE_NOALLOC_MAX_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices] = {};

static moe_status scratch_address(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

extern "C" {

moe_status moe_gate_noalloc(int32_t T, int32_t H, int32_t E, int32_t k, const void* x, const void* wr, float* logits,
                            int32_t* ids, float* w, hipStream_t stream) {
  moe_status st = gate_check(T, H, E, k, x, wr, nullptr, false, logits, ids, w);
  if (st != MOE_OK || T == 0) return st;
  const size_t need = moe_gate_workspace_bytes(T, H, E);
  if (need > MOE_GATE_NOALLOC_MAX_BYTES)
    return fail(MOE_ERR_INVALID_ARG, "this shape needs %zu bytes of scratch; moe_gate_noalloc holds %u", need,
                (unsigned)MOE_GATE_NOALLOC_MAX_BYTES);
  void* part = nullptr;
  st = scratch_address(&part);
  if (st != MOE_OK) return st;
  return gate_launch(T, H, E, k, x, wr, static_cast<float*>(part), logits, ids, w, stream);
}

moe_status moe_gate(int32_t T, int32_t H, int32_t E, int32_t k, const void* x, const void* wr, void* workspace,
                    size_t workspace_bytes, float* logits, int32_t* ids, float* w, hipStream_t stream) {
  moe_status st = gate_check(T, H, E, k, x, wr, workspace, true, logits, ids, w);
  if (st != MOE_OK || T == 0) return st;
  const size_t need = moe_gate_workspace_bytes(T, H, E);
  if (workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "workspace of %zu bytes; this shape needs %zu", workspace_bytes, need);
  return gate_launch(T, H, E, k, x, wr, static_cast<float*>(workspace), logits, ids, w, stream);
}

int64_t moe_mfma_fp8_probe(float* sink, int32_t blocks, int32_t iters, hipStream_t stream) {
  if (!sink || ((uintptr_t)sink & 3u) || blocks < 1 || iters < 1) {
    fail(MOE_ERR_INVALID_ARG, "sink must be a 4-byte aligned device pointer; blocks, iters >= 1");
    return -1;
  }
  if (launch_mfma_fp8_probe(sink, blocks, iters, stream) != hipSuccess) {
    fail(MOE_ERR_HIP, "probe launch failed");
    return -1;
  }
  return (int64_t)blocks * 4 * iters * mfma_fp8_probe_chains() * (2 * 16 * 16 * 128);
}

moe_status moe_mfma_dot16x16(moe_dtype a_fmt, const uint8_t* a, const uint8_t* b, float* out, hipStream_t stream) {
  if (a_fmt != MOE_FP8_E4M3 && a_fmt != MOE_FP4_E2M1)
    return fail(MOE_ERR_INVALID_ARG, "a_fmt must be MOE_FP8_E4M3 or MOE_FP4_E2M1");
  if (!a || !b || !out || ((uintptr_t)out & 3u)) return fail(MOE_ERR_INVALID_ARG, "a, b or out is NULL or out misaligned");
  HIP_TRY(launch_mfma_dot(a_fmt == MOE_FP4_E2M1, a, b, out, stream));
  return MOE_OK;
}

moe_status moe_last_device_error(moe_ctx* c, uint32_t* bits) {
  if (!c || !bits) return fail(MOE_ERR_INVALID_ARG, "ctx or bits is NULL");
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(bits, c->err, 4, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemset(c->err, 0, 4));
  if (*bits & MOE_DEVERR_TIMEOUT) {
    // a GEMM2 item the persistent kernel skipped never counted its rows: start the fused
    // combine's counters from zero again (the device is idle)
    const size_t nbh = (size_t)(c->cfg.hidden + 255) / 256;
    HIP_TRY(hipMemset(c->ccnt, 0, (size_t)c->cfg.n_src * c->cfg.max_tokens * nbh * 4));
  }
  return MOE_OK;
}

moe_status moe_set_timing(moe_ctx* c, int32_t max_calls) {
  if (!c || max_calls < 0) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL or max_calls < 0");
  HIP_TRY(hipDeviceSynchronize());
  for (auto ev : c->ev) (void)hipEventDestroy(ev);
  c->ev.assign((size_t)max_calls * (kStages + 1), nullptr);
  for (auto& ev : c->ev) HIP_TRY(hipEventCreate(&ev));
  c->timing_cap = max_calls;
  c->timing_n = 0;
  return MOE_OK;
}

moe_status moe_read_timing(moe_ctx* c, float* ms, int32_t* n_calls) {
  if (!c || !ms || !n_calls) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  for (int i = 0; i < kStages; ++i) ms[i] = 0.f;
  for (int n = 0; n < c->timing_n; ++n) {
    hipEvent_t* e = &c->ev[(size_t)n * (kStages + 1)];
    HIP_TRY(hipEventSynchronize(e[4]));
    float t;
    // events: 0 start, 1 after dispatch, 2 after GEMM1, 3 after GEMM2, 4 after combine
    for (int i = 0; i < 4; ++i) {
      HIP_TRY(hipEventElapsedTime(&t, e[i], e[i + 1]));
      ms[i] += t;
    }
    HIP_TRY(hipEventElapsedTime(&t, e[0], e[4]));
    ms[4] += t;
  }
  *n_calls = c->timing_n;
  c->timing_n = 0;
  return MOE_OK;
}

}  // extern "C"
