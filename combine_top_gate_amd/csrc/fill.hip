// Fill of a device buffer with a repeated 32-bit pattern (a kernel, not a memset, so
// that a captured graph replays it like any other kernel).  Used to poison the
// context's windows, h and y with NaN codes before a layer call (a test option).
#include "kernels.h"

namespace {

typedef unsigned int fill_vec4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_fill32(uint32_t* p, size_t words, uint32_t pattern) {
  const size_t vecs = words >> 2;
  const fill_vec4 v = {pattern, pattern, pattern, pattern};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < vecs; i += stride)
    reinterpret_cast<fill_vec4*>(p)[i] = v;
  for (size_t i = (vecs << 2) + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) p[i] = pattern;
}

}  // namespace

hipError_t launch_fill32(void* p, size_t bytes, uint32_t pattern, hipStream_t st) {
  const size_t words = bytes >> 2;
  if (words == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>(1024, (words / 4 + 255) / 256 + 1);
  hipLaunchKernelGGL(k_fill32, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<uint32_t*>(p), words, pattern);
  return hipGetLastError();
}
