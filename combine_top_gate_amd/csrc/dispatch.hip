// Dispatch kernel: one workgroup per (chunk of tokens, source); the work itself is
// dispatch_chunk() (dispatch_chunk.h).
#include <algorithm>

#include "dispatch_chunk.h"

namespace {

__global__ __launch_bounds__(kDispatchThreads) void k_dispatch(DispatchArgs a) {
  __shared__ DispatchSmem sm;
  dispatch_chunk(a, blockIdx.y, blockIdx.x, gridDim.x, sm);
}

}  // namespace

int dispatch_chunks(const DispatchArgs& a) { return (a.T_s + a.tpb - 1) / a.tpb; }

int dispatch_tokens_per_block(int T_s, int k, int blocks_wanted, int S) {
  // enough workgroups to spread the copy, at most kMaxDispatchPairs pairs each
  const int per = (T_s * S + blocks_wanted - 1) / std::max(1, blocks_wanted);
  return std::max(1, std::min(std::max(1, per), kMaxDispatchPairs / k));
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_dispatch, dim3(dispatch_chunks(a), a.S), dim3(kDispatchThreads), 0, st, a);
  return hipGetLastError();
}
