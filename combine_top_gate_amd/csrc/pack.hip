// Device-side repack of row-major expert weights into the GEMM's streaming order
// (pack_layout.h).  One thread per 16-byte destination piece (weights) or per 4-byte
// destination word (FP4 e8m0 scales); a pure permutation of bytes.
#include "kernels.h"
#include "pack_layout.h"

namespace {

__global__ __launch_bounds__(256) void k_pack_w(PackArgs a) {
  const int wl = pack_wl(a.wfmt);
  const int KB = a.K >> 7;
  const int64_t rowb = a.wfmt == MOE_FP4_E2M1 ? a.K / 2 : a.K;  // bytes per source row
  // pieces per expert: blocks * 4 waves * KB * 4 tiles * wl * 64 lanes
  const int64_t per_e = (int64_t)a.nblk * 4 * KB * 4 * wl * 64;
  const int64_t total = per_e * a.E;
  for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int e = (int)(i / per_e);
    int64_t j = i - e * per_e;
    const int lane = (int)(j & 63); j >>= 6;
    const int h = (int)(j % wl); j /= wl;
    const int mt = (int)(j & 3); j >>= 2;
    const int kb = (int)(j % KB); j /= KB;
    const int wave = (int)(j & 3); j >>= 2;
    const int blk = (int)j;
    const int r = lane & 15, g = lane >> 4;
    const int row = a.gemm1 ? pack_row13(a.inter, blk, wave, mt, r) : pack_row2(blk, wave, mt, r);
    if (row >= a.N) continue;
    const int64_t col = a.wfmt == MOE_FP4_E2M1 ? (int64_t)kb * 64 + 16 * g : (int64_t)kb * 128 + 64 * h + 16 * g;
    const uint4 v = *reinterpret_cast<const uint4*>(a.src + e * a.src_stride + row * rowb + col);
    const int64_t dst = e * a.dst_stride + pack_w_offset(a.wfmt, a.K, blk, wave, kb) + (mt * wl + h) * 1024 + lane * 16;
    *reinterpret_cast<uint4*>(a.dst + dst) = v;
  }
}

__global__ __launch_bounds__(256) void k_pack_e(PackArgs a) {
  const int KB = a.K >> 7;
  const int64_t per_e = (int64_t)a.nblk * 4 * KB * 64;  // 4-byte words per expert
  const int64_t total = per_e * a.E;
  for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int e = (int)(i / per_e);
    int64_t j = i - e * per_e;
    const int lane = (int)(j & 63); j >>= 6;
    const int kb = (int)(j % KB); j /= KB;
    const int wave = (int)(j & 3); j >>= 2;
    const int blk = (int)j;
    const int r = lane & 15, g = lane >> 4;
    uint32_t word = 0;
    for (int mt = 0; mt < 4; ++mt) {
      const int row = a.gemm1 ? pack_row13(a.inter, blk, wave, mt, r) : pack_row2(blk, wave, mt, r);
      const uint32_t b = row < a.N ? a.src[e * a.src_stride + (int64_t)row * (a.K / 32) + kb * 4 + g] : 127u;
      word |= b << (8 * mt);
    }
    *reinterpret_cast<uint32_t*>(a.dst + e * a.dst_stride + pack_e_offset(a.K, blk, wave, kb) + lane * 4) = word;
  }
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, bool scales, hipStream_t st) {
  if (a.E == 0) return hipSuccess;
  if (scales)
    hipLaunchKernelGGL(k_pack_e, dim3(2048), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_pack_w, dim3(4096), dim3(256), 0, st, a);
  return hipGetLastError();
}
