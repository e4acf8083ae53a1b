// Grouped GEMMs over the expert windows, FP8 e4m3 activations x FP8 (128x128 block
// scales) or MXFP4 (e8m0 1x32 scales) weights, on gfx950 MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4.
//
// GEMM1: a = x W13^T over the window rows of one expert, SwiGLU h = silu(gate) * up,
//        then h is requantised to e4m3 with one fp32 scale per 128 columns of a row.
// GEMM2: y = h W2^T, stored bf16.
// ("GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4 Grouped GEMM via
// CUDA Green Contexts", full text: block-scaled MMA with operand swap, fused SwiGLU,
// requantization, optional shared experts; "One-Sided Expert-Parallel All-to-All for
// Mixture-of-Experts Inference over NVLink", abstract: windows are read in place.)
//
// Decode shapes give each expert a few dozen rows against thousands of weight rows,
// so the weights go in the MFMA's 16-row A slot and the tokens in its 16-column B
// slot (operand swap).  Each wave streams its weight rows straight from HBM into
// registers in the MFMA operand layout, two 128-deep K slabs ahead; the workgroup's
// token rows (at most 16*NT of them per pass) go through LDS once per K slab and are
// shared by the four waves.  One MFMA covers exactly one 128-wide scale block, so
// its fp32 result is promoted with (weight scale x token scale) before it is added
// to the accumulator.  Experts with more rows than one pass take several passes.
//
// MFMA operand layout on gfx950 (16x16x128, measured): lane l serves row/column
// l%16; with g = l/16, an FP8 operand holds k = 16g..16g+15 in bytes 0..15 and
// k = 64+16g..64+16g+15 in bytes 16..31; an FP4 operand holds k = 32g..32g+31 as
// nibbles (element 2i in the low nibble of byte i) and lane l's e8m0 scale covers
// exactly those 32 k.  The result's lane l, register i is row 4g+i, column l%16.
#include "kernels.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTokStride = 144;  // LDS bytes per staged 128-byte token slab row (+16 against bank conflicts)

template <int WFMT>
struct WeightFmt;
template <>
struct WeightFmt<MOE_FP8_E4M3> {
  static constexpr int kLoads = 2;  // 16-byte loads per lane per 16-row tile per K slab
  static constexpr int kSlabBytes = 128;
  static constexpr int kMfmaFmt = MFMA_FMT_FP8;
};
template <>
struct WeightFmt<MOE_FP4_E2M1> {
  static constexpr int kLoads = 1;
  static constexpr int kSlabBytes = 64;
  static constexpr int kMfmaFmt = MFMA_FMT_FP4;
};

// Per-pass token table: where each of the pass's rows is read from and written to.
template <int NTOK>
struct TokTable {
  const uint8_t* arow[NTOK];
  const float* asc[NTOK];
  int orow[NTOK];
};

// Weight-side state of one wave: 4 tiles of 16 weight rows.
template <int WFMT>
struct WaveWeights {
  const uint8_t* row[4];    // this lane's weight row of each tile (at k = 0)
  const float* fscale[4];   // FP8: scale row of each tile's 128-row block, [kb]
  const uint8_t* escale[4]; // FP4: this lane's e8m0 bytes, [kb*4]
};

template <int WFMT>
__device__ __forceinline__ void load_w(u32x4 (&dst)[4][WeightFmt<WFMT>::kLoads],
                                       const WaveWeights<WFMT>& ww, int kb, int g4) {
  constexpr int SB = WeightFmt<WFMT>::kSlabBytes;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint8_t* p = ww.row[mt] + (int64_t)kb * SB + 16 * g4;
    dst[mt][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    if constexpr (WeightFmt<WFMT>::kLoads == 2)
      dst[mt][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 64));
  }
}

// Main loop of one pass: acc[mt][nt] += promoted MFMA results over all K slabs.
// Token rows come from tab; row_stride is the byte stride of the activation rows,
// KB the number of 128-deep K slabs.  Every thread of the workgroup calls this.
template <int NT, int WFMT>
__device__ __forceinline__ void mainloop(v4f (&acc)[4][NT], const WaveWeights<WFMT>& ww,
                                         const TokTable<16 * NT>& tab,
                                         uint8_t (*s_tok)[16 * NT * kTokStride],
                                         float (*s_tsc)[16 * NT], int KB, bool wave_active) {
  constexpr int NTOK = 16 * NT;
  constexpr int PIECES = NTOK * 8;  // 16-byte pieces of one token slab
  constexpr int TLD = (PIECES + 255) / 256;
  constexpr int WL = WeightFmt<WFMT>::kLoads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int g4 = lane >> 4, r16 = lane & 15;

#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

  u32x4 treg[TLD];
  float tsreg = 0.f;
  auto load_tok = [&](int kb) {
#pragma unroll
    for (int i = 0; i < TLD; ++i) {
      const int q = tid + 256 * i;
      if (q < PIECES) {
        const uint8_t* ar = tab.arow[q >> 3];
        treg[i] = ar ? *reinterpret_cast<const u32x4*>(ar + (int64_t)kb * 128 + (q & 7) * 16)
                     : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < NTOK) {
      const float* as = tab.asc[tid];
      tsreg = as ? as[kb] : 0.f;
    }
  };
  auto store_tok = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TLD; ++i) {
      const int q = tid + 256 * i;
      if (q < PIECES) *reinterpret_cast<u32x4*>(&s_tok[buf][(q >> 3) * kTokStride + (q & 7) * 16]) = treg[i];
    }
    if (tid < NTOK) s_tsc[buf][tid] = tsreg;
  };

  u32x4 wA[4][WL], wB[4][WL], wC[4][WL];
  load_tok(0);
  if (wave_active) {
    load_w<WFMT>(wA, ww, 0, g4);
    if (KB > 1) load_w<WFMT>(wB, ww, 1, g4);
  }
  store_tok(0);
  __syncthreads();

  auto step = [&](int kb, const u32x4 (&cur)[4][WL], u32x4 (&nxt)[4][WL]) {
    if (kb + 1 < KB) load_tok(kb + 1);
    if (wave_active) {
      if (kb + 2 < KB) load_w<WFMT>(nxt, ww, kb + 2, g4);
      const int buf = kb & 1;
      float fs[4];
      int es[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if constexpr (WFMT == MOE_FP8_E4M3) {
          fs[mt] = ww.fscale[mt][kb];
          es[mt] = E8M0_ONE;
        } else {
          fs[mt] = 1.f;
          es[mt] = ww.escale[mt][kb * 4];
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint8_t* tp = &s_tok[buf][(nt * 16 + r16) * kTokStride + 16 * g4];
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(tp);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(tp + 64);
        const v8i bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                        (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        const float sx = s_tsc[buf][nt * 16 + r16];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          v8i av;
          if constexpr (WL == 2)
            av = v8i{(int)cur[mt][0].x, (int)cur[mt][0].y, (int)cur[mt][0].z, (int)cur[mt][0].w,
                     (int)cur[mt][1].x, (int)cur[mt][1].y, (int)cur[mt][1].z, (int)cur[mt][1].w};
          else
            av = v8i{(int)cur[mt][0].x, (int)cur[mt][0].y, (int)cur[mt][0].z, (int)cur[mt][0].w,
                     0, 0, 0, 0};
          const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              av, bv, v4f{0.f, 0.f, 0.f, 0.f}, WeightFmt<WFMT>::kMfmaFmt, MFMA_FMT_FP8, 0, es[mt], 0,
              E8M0_ONE);
          const float sc = fs[mt] * sx;
          acc[mt][nt][0] = fmaf(r[0], sc, acc[mt][nt][0]);
          acc[mt][nt][1] = fmaf(r[1], sc, acc[mt][nt][1]);
          acc[mt][nt][2] = fmaf(r[2], sc, acc[mt][nt][2]);
          acc[mt][nt][3] = fmaf(r[3], sc, acc[mt][nt][3]);
        }
      }
    }
    if (kb + 1 < KB) store_tok((kb + 1) & 1);
    __syncthreads();
  };

  for (int kb = 0; kb < KB; kb += 3) {
    step(kb, wA, wC);
    if (kb + 1 < KB) step(kb + 1, wB, wA);
    if (kb + 2 < KB) step(kb + 2, wC, wB);
  }
}

// Flat work list: routed expert g has nb_r entries, then the shared expert nb_s.
__device__ __forceinline__ void work_item(const BatchDims& d, int nb_r, int nb_s, int& g, int& nb) {
  const int total = d.E * nb_r + nb_s;
  const int L = xcd_remap(blockIdx.x, total);
  if (L < d.E * nb_r) {
    g = L / nb_r;
    nb = L - g * nb_r;
  } else {
    g = d.E;
    nb = L - d.E * nb_r;
  }
}

__device__ __forceinline__ int group_rows(const GemmArgs& p, int g) {
  if (g == p.d.E) return p.d.T;
  int M = 0;
  for (int s = 0; s < p.d.S; ++s) M += p.cnt[s * p.d.E + g];
  return M;
}

// ------------------------------------------------------------------ GEMM1
template <int NT, int WFMT>
__global__ __launch_bounds__(256, 2) void k_gemm1_lowp(GemmArgs p) {
  constexpr int NTOK = 16 * NT;
  __shared__ __align__(16) uint8_t s_tok[2][NTOK * kTokStride];
  __shared__ float s_tsc[2][NTOK];
  __shared__ TokTable<NTOK> tab;
  __shared__ float s_amax[4][NTOK];

  const BatchDims& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  int g, nb;
  work_item(d, d.I >> 7, d.Ish >> 7, g, nb);
  const bool shared = g == d.E;
  const int inter = shared ? d.Ish : d.I;
  const int M = group_rows(p, g);
  if (M == 0) return;  // no rows: no weight traffic (uniform over the workgroup)

  const int K = d.H, KB = K >> 7;
  constexpr bool FP4 = WFMT == MOE_FP4_E2M1;
  const int64_t wrow = FP4 ? (K >> 1) : K;
  const uint8_t* W = shared ? p.w_sh : p.w + (int64_t)g * p.w_stride;
  WaveWeights<WFMT> ww;
  const int rb = nb * 128 + 32 * wave;  // this wave's gate rows: rb..rb+31; up rows: inter + same
  const int rows[4] = {rb, rb + 16, inter + rb, inter + rb + 16};
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = rows[mt] + r16;
    ww.row[mt] = W + (int64_t)row * wrow;
    if constexpr (FP4) {
      const uint8_t* E8 = static_cast<const uint8_t*>(shared ? p.ws_sh : p.ws) + (shared ? 0 : (int64_t)g * p.ws_stride);
      ww.escale[mt] = E8 + (int64_t)row * (K >> 5) + g4;
      ww.fscale[mt] = nullptr;
    } else {
      const float* FS = static_cast<const float*>(shared ? p.ws_sh : p.ws) + (shared ? 0 : (int64_t)g * p.ws_stride);
      ww.fscale[mt] = FS + (int64_t)(rows[mt] >> 7) * KB;
      ww.escale[mt] = nullptr;
    }
  }

  const int seg = d.T_s * d.k;
  const int hsc_stride = d.hstride >> 7;
  for (int m0 = 0; m0 < M; m0 += NTOK) {
    if (tid < NTOK) {
      const int m = m0 + tid;
      const uint8_t* ar = nullptr;
      const float* as = nullptr;
      int orow = -1;
      if (m < M) {
        if (shared) {
          const int s = m / d.T_s, t = m - s * d.T_s;
          ar = p.src.x[s] + (int64_t)t * K;
          as = p.src.xs[s] + (int64_t)t * KB;
          orow = d.R + m;
        } else {
          const int r = routed_row(p.cnt, p.off, d.S, d.E, seg, g, m);
          ar = p.a + (int64_t)r * K;
          as = p.as + (int64_t)r * KB;
          orow = r;
        }
      }
      tab.arow[tid] = ar;
      tab.asc[tid] = as;
      tab.orow[tid] = orow;
    }
    __syncthreads();

    v4f acc[4][NT];
    mainloop<NT, WFMT>(acc, ww, tab, s_tok, s_tsc, KB, true);

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
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int tk = nt * 16 + r16;
      const int orow = tab.orow[tk];
      if (orow < 0) continue;
      const float amax = fmaxf(fmaxf(s_amax[0][tk], s_amax[1][tk]), fmaxf(s_amax[2][tk], s_amax[3][tk]));
      const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(hv[t][nt][i] / sc, -448.0f), 448.0f);
        const uint32_t packed = pack4_e4m3(q[0], q[1], q[2], q[3]);
        *reinterpret_cast<uint32_t*>(p.h + (int64_t)orow * d.hstride + rb + 16 * t + 4 * g4) = packed;
      }
      if (wave == 0 && g4 == 0) p.hs[(int64_t)orow * hsc_stride + nb] = sc;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ GEMM2
template <int NT, int WFMT>
__global__ __launch_bounds__(256, 2) void k_gemm2_lowp(GemmArgs p) {
  constexpr int NTOK = 16 * NT;
  __shared__ __align__(16) uint8_t s_tok[2][NTOK * kTokStride];
  __shared__ float s_tsc[2][NTOK];
  __shared__ TokTable<NTOK> tab;

  const BatchDims& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int nbh = (d.H + 255) >> 8;  // 256 output rows per workgroup
  int g, nb;
  work_item(d, nbh, d.Ish ? nbh : 0, g, nb);
  const bool shared = g == d.E;
  const int K = shared ? d.Ish : d.I, KB = K >> 7;
  const int M = group_rows(p, g);
  if (M == 0) return;

  constexpr bool FP4 = WFMT == MOE_FP4_E2M1;
  const int64_t wrow = FP4 ? (K >> 1) : K;
  const uint8_t* W = shared ? p.w_sh : p.w + (int64_t)g * p.w_stride;
  const int rb = nb * 256 + 64 * wave;  // this wave's output rows rb..rb+63
  const bool active = rb < d.H;
  WaveWeights<WFMT> ww;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = active ? rb + 16 * mt + r16 : 0;
    ww.row[mt] = W + (int64_t)row * wrow;
    if constexpr (FP4) {
      const uint8_t* E8 = static_cast<const uint8_t*>(shared ? p.ws_sh : p.ws) + (shared ? 0 : (int64_t)g * p.ws_stride);
      ww.escale[mt] = E8 + (int64_t)row * (K >> 5) + g4;
      ww.fscale[mt] = nullptr;
    } else {
      const float* FS = static_cast<const float*>(shared ? p.ws_sh : p.ws) + (shared ? 0 : (int64_t)g * p.ws_stride);
      ww.fscale[mt] = FS + (int64_t)((active ? rb : 0) >> 7) * KB;
      ww.escale[mt] = nullptr;
    }
  }

  const int seg = d.T_s * d.k;
  const int hsc_stride = d.hstride >> 7;
  for (int m0 = 0; m0 < M; m0 += NTOK) {
    if (tid < NTOK) {
      const int m = m0 + tid;
      const uint8_t* ar = nullptr;
      const float* as = nullptr;
      int orow = -1;
      if (m < M) {
        const int r = shared ? d.R + m : routed_row(p.cnt, p.off, d.S, d.E, seg, g, m);
        ar = p.a + (int64_t)r * d.hstride;
        as = p.as + (int64_t)r * hsc_stride;
        orow = r;
      }
      tab.arow[tid] = ar;
      tab.asc[tid] = as;
      tab.orow[tid] = orow;
    }
    __syncthreads();

    v4f acc[4][NT];
    mainloop<NT, WFMT>(acc, ww, tab, s_tok, s_tsc, KB, active);

    if (active) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int orow = tab.orow[nt * 16 + r16];
        if (orow < 0) continue;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint32_t lo = bf16_bits(acc[mt][nt][0]) | (bf16_bits(acc[mt][nt][1]) << 16);
          const uint32_t hi = bf16_bits(acc[mt][nt][2]) | (bf16_bits(acc[mt][nt][3]) << 16);
          *reinterpret_cast<uint2*>(p.y + (int64_t)orow * d.H + rb + 16 * mt + 4 * g4) = make_uint2(lo, hi);
        }
      }
    }
    __syncthreads();
  }
}

template <int WFMT>
hipError_t launch1(const GemmArgs& a, int nt, hipStream_t st) {
  const dim3 grid(a.d.E * (a.d.I >> 7) + (a.d.Ish >> 7)), block(256);
  switch (nt) {
    case 1: hipLaunchKernelGGL((k_gemm1_lowp<1, WFMT>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemm1_lowp<2, WFMT>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_gemm1_lowp<3, WFMT>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_gemm1_lowp<4, WFMT>), grid, block, 0, st, a); break;
    case 5: hipLaunchKernelGGL((k_gemm1_lowp<5, WFMT>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_gemm1_lowp<6, WFMT>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

template <int WFMT>
hipError_t launch2(const GemmArgs& a, int nt, hipStream_t st) {
  const int nbh = (a.d.H + 255) >> 8;
  const dim3 grid(a.d.E * nbh + (a.d.Ish ? nbh : 0)), block(256);
  switch (nt) {
    case 1: hipLaunchKernelGGL((k_gemm2_lowp<1, WFMT>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemm2_lowp<2, WFMT>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_gemm2_lowp<3, WFMT>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_gemm2_lowp<4, WFMT>), grid, block, 0, st, a); break;
    case 5: hipLaunchKernelGGL((k_gemm2_lowp<5, WFMT>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_gemm2_lowp<6, WFMT>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1_lowp(const GemmArgs& a, int weight_fmt, int tok_tiles, hipStream_t st) {
  return weight_fmt == MOE_FP4_E2M1 ? launch1<MOE_FP4_E2M1>(a, tok_tiles, st)
                                    : launch1<MOE_FP8_E4M3>(a, tok_tiles, st);
}

hipError_t launch_gemm2_lowp(const GemmArgs& a, int weight_fmt, int tok_tiles, hipStream_t st) {
  return weight_fmt == MOE_FP4_E2M1 ? launch2<MOE_FP4_E2M1>(a, tok_tiles, st)
                                    : launch2<MOE_FP8_E4M3>(a, tok_tiles, st);
}
