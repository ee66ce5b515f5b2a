// kv_window_advance: the copy that advances a linear (non-ring) cache window by n tokens, the
// per-call whole-cache work of the read-time design that the ring replaces (Runway Characters
// abstract: the cache's whole-window work moved out of every call; cpdf.ai blog, section "Como
// rodar 57B em tempo real com batch size 1": the ring advances the window without copies).
//
// dst = src[n:] followed by fresh[0:n], rows of row_bytes bytes.  One pass of 16-byte units:
// unit u < (window - n) * row_units reads src at unit u + n * row_units, the others read fresh.
// Four units per thread are loaded before any is stored, so each wavefront keeps four 1 KB
// loads in flight; the grid is sized to a few waves per compute unit and strides over the rest.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvring {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void window_advance_kernel(const uint4* __restrict__ src,
                                                                      const uint4* __restrict__ fresh,
                                                                      uint4* __restrict__ dst,
                                                                      int64_t kept, int64_t shift,
                                                                      int64_t total) {
  const int64_t stride = (int64_t)gridDim.x * kCopyThreads * kCopyUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kCopyThreads * kCopyUnroll + threadIdx.x; base < total;
       base += stride) {
    uint4 x[kCopyUnroll];
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t u = base + (int64_t)j * kCopyThreads;
      if (u < total) x[j] = u < kept ? src[u + shift] : fresh[u - kept];
    }
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t u = base + (int64_t)j * kCopyThreads;
      if (u < total) dst[u] = x[j];
    }
  }
}

}  // namespace

hipError_t launch_window_advance(const void* src, void* dst, const void* fresh, int32_t window,
                                 int32_t n, int64_t row_bytes, hipStream_t stream) {
  const int64_t row_units = row_bytes / 16;
  const int64_t total = (int64_t)window * row_units;
  if (total == 0) return hipSuccess;
  const int64_t per_block = (int64_t)kCopyThreads * kCopyUnroll;
  int64_t blocks = (total + per_block - 1) / per_block;
  if (blocks > 256 * 8) blocks = 256 * 8;
  hipLaunchKernelGGL(window_advance_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                     static_cast<const uint4*>(src), static_cast<const uint4*>(fresh),
                     static_cast<uint4*>(dst), (int64_t)(window - n) * row_units,
                     (int64_t)n * row_units, total);
  return hipGetLastError();
}

}  // namespace kvring
