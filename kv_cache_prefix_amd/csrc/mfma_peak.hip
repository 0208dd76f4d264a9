// A plain stream of fp16 matrix products: the dense MFMA rate the chip sustains when
// every SIMD issues them back to back (its clock then settles below the rated one). The
// batched-Q kernels use the same v_mfma_f32_32x32x16_f16 and are measured against this
// beside the rated peak. No memory traffic and no vector work besides the products.
#include "kernels.h"

namespace pion {
namespace {

typedef _Float16 pk_half8 __attribute__((ext_vector_type(8)));
typedef float pk_f16v __attribute__((ext_vector_type(16)));

constexpr int kPeakChains = 4;      // independent accumulators per wave
constexpr int kPeakWgPerCu = 4;     // workgroups of 4 waves per CU: 4 waves per SIMD
constexpr double kFlopsPerMfma = 2.0 * 32 * 32 * 16;

// Every wave runs iters rounds of kPeakChains independent products; the operands are
// small lane-dependent values (the sums stay far from overflow for any iters that fits an
// int), and the accumulators are folded into one word that is stored only when it equals
// `magic`, so the products cannot be removed and nothing reaches memory.
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, uint32_t magic,
                                                        uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  pk_half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)((float)((lane + e) & 63) * 0x1p-16f);
    b[e] = (_Float16)((float)((lane ^ e) & 63) * 0x1p-16f);
  }
  pk_f16v acc[kPeakChains];
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (__float_as_uint(s) == magic) sink[0] = magic;
}

}  // namespace

hipError_t launch_mfma_peak(int iters, double *flops, uint32_t *sink, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)cus * kPeakWgPerCu;
  *flops = (double)grid * 4 * kPeakChains * (double)iters * kFlopsPerMfma;
  note_launch("mfma_peak_kernel");
  // 0x7F800001 is a NaN pattern: finite sums never match it
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(grid), dim3(256), 0, s, iters, 0x7F800001u, sink);
  return hipGetLastError();
}

}  // namespace pion
