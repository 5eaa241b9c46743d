// Loading an adapter into a fixed slot ("Add multi-LoRA support", Features:
// a tiered cache whose GPU tier is a fixed number of slots, and adapters of
// different ranks).  A slot of a stacked tensor is a dense [rows][cols]
// region; an adapter's matrix is smaller (rank r <= r_max), and everything
// past it must be zero so that kernels reading the padded region (or ranks
// clamped differently) see no stale values of the slot's previous adapter.
// One element per thread, destination-ordered (coalesced stores):
//   dst[i][j] = (i < m_rows && j < m_cols) ? M[i][j] : 0
// with M = src or src transposed.
#include "common.h"

namespace lora {

namespace {

template <typename Word>
__global__ __launch_bounds__(256) void copy_padded_kernel(const Word* __restrict__ src, int64_t src_ld, int transpose,
                                                          int64_t m_rows, int64_t m_cols, Word* __restrict__ dst,
                                                          int64_t dst_rows, int64_t dst_cols, int64_t dst_ld) {
  const int64_t n = dst_rows * dst_cols;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / dst_cols, j = e - i * dst_cols;
    Word w = 0;
    if (i < m_rows && j < m_cols) w = transpose ? src[j * src_ld + i] : src[i * src_ld + j];
    dst[i * dst_ld + j] = w;
  }
}

}  // namespace

hipError_t launch_copy_padded(int elem_bytes, const void* src, int64_t src_ld, int transpose, int64_t m_rows,
                              int64_t m_cols, void* dst, int64_t dst_rows, int64_t dst_cols, int64_t dst_ld,
                              hipStream_t stream) {
  const int64_t n = dst_rows * dst_cols;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)(ceil_div(n, 256) < 4096 ? ceil_div(n, 256) : 4096);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(copy_padded_kernel<uint32_t>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint32_t*>(src), src_ld, transpose, m_rows, m_cols,
                       static_cast<uint32_t*>(dst), dst_rows, dst_cols, dst_ld);
  else
    hipLaunchKernelGGL(copy_padded_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), src_ld, transpose, m_rows, m_cols,
                       static_cast<uint16_t*>(dst), dst_rows, dst_cols, dst_ld);
  return hipGetLastError();
}

}  // namespace lora
