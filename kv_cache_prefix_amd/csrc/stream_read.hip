// A plain streaming read: the achievable HBM read rate a bandwidth-bound kernel of this
// library is measured against (the roofline's "ceiling" beside the 8 TB/s rating). It
// reads a buffer once with 16-byte non-temporal loads, as the decode kernels read K/V,
// and does no other work.
#include "kernels.h"

namespace pion {
namespace {

constexpr int kReadUnroll = 4;  // 16-byte loads in flight per lane and iteration
typedef unsigned rd_u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride over 16-byte pieces; each lane folds what it read into one word and stores
// it only when that word equals `magic` (never, for any realistic buffer), so the loads
// cannot be removed and nothing but the reads reaches memory.
__global__ __launch_bounds__(256) void stream_read_kernel(const rd_u32x4 *__restrict__ src,
                                                          int64_t n16, uint32_t magic,
                                                          uint32_t *__restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    rd_u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const rd_u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == magic) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  // 8 workgroups of 256 lanes per CU (2 per SIMD), each lane 4 pieces in flight
  const int64_t want = (n16 + 256 * kReadUnroll - 1) / (256 * kReadUnroll);
  const unsigned grid = (unsigned)(want < 2048 ? want : 2048);
  note_launch("stream_read_kernel");
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, s, (const rd_u32x4 *)buf, n16,
                     0x9E3779B9u, sink);
  return hipGetLastError();
}

}  // namespace pion
