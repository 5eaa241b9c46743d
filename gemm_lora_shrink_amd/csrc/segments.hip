// The segment build kernel: one workgroup runs the block-level build of
// segments_block.h -- 1024 threads in general, 256 for small batches
// (T <= kSmallT, S <= 256), where fewer waves mean shorter per-key table walks
// and cheaper barriers.
#include "segments_block.h"

namespace lora {

namespace {

constexpr int kThreadsLarge = 1024;
constexpr int kThreadsSmall = 256;
constexpr int kSmallT = 1024;
constexpr int kLdsPerm = 8192;  // perm positions mirrored in LDS

template <int kThreads>
__global__ __launch_bounds__(kThreads) void build_segments_kernel(const int32_t* __restrict__ idx, int T, int S,
                                                                  int mode, int32_t* __restrict__ rec) {
  __shared__ SegShared<kThreads, kLdsPerm> sh;
  build_segments_block<kThreads, kLdsPerm>(idx, T, S, mode, rec, sh);
}

}  // namespace

hipError_t launch_build_segments(const int32_t* idx, int32_t T, int32_t S, int32_t mode, int32_t* rec,
                                 hipStream_t stream) {
  if (T <= kSmallT && S <= kThreadsSmall)
    hipLaunchKernelGGL(build_segments_kernel<kThreadsSmall>, dim3(1), dim3(kThreadsSmall), 0, stream, idx, T, S,
                       mode, rec);
  else
    hipLaunchKernelGGL(build_segments_kernel<kThreadsLarge>, dim3(1), dim3(kThreadsLarge), 0, stream, idx, T, S,
                       mode, rec);
  return hipGetLastError();
}

}  // namespace lora
