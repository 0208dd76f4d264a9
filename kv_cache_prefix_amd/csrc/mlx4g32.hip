// mlx4g32 encoder: int4 codes, group 32, affine, fp16 scale and bias per group, the
// scale rounded to fp16 before the codes are chosen ("Shared KV Cache Serving",
// Quantized tier - mlx4g32; V-store page, The mlx4g32 tier).
//
// Per group, in fp32 with IEEE round-to-nearest-even on every op:
//   mn = min x, mx = max x, s = fp16((mx - mn) / 15), b = fp16(mn),
//   q = clamp(rint((x - b) / s), 0, 15), or all zero when s == 0.
// Element i of a row goes to word i/8 at bits 4*(i%8).
//
// Layout: one lane per uint32 code word (8 elements, 16 input bytes), so four
// consecutive lanes hold one group; min/max combine across those four lanes. Loads are
// 16 B per lane and stores 4 B per lane, contiguous across the wave. Division is the
// correctly rounded fp32 divide and there is no contraction, so the codes are bit-exact
// with any IEEE fp32 evaluation of the steps above.
#include "kernels.h"

#include <hip/hip_fp16.h>

namespace pion {
namespace {

__global__ __launch_bounds__(256) void quantize_mlx4g32_kernel(const uint16_t *__restrict__ x,
                                                               int64_t nwords,
                                                               uint32_t *__restrict__ codes,
                                                               uint16_t *__restrict__ scales,
                                                               uint16_t *__restrict__ biases,
                                                               int sb_stride) {
#pragma clang fp contract(off)
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = t < nwords;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (valid) raw = *(const uint4 *)(x + t * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[2 * c] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[c] & 0xffffu));
    v[2 * c + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[c] >> 16));
  }
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    mn = fminf(mn, v[e]);
    mx = fmaxf(mx, v[e]);
  }
  // the four lanes of a group are lanes 4k..4k+3 of the same wave
  mn = fminf(mn, __shfl_xor(mn, 1));
  mn = fminf(mn, __shfl_xor(mn, 2));
  mx = fmaxf(mx, __shfl_xor(mx, 1));
  mx = fmaxf(mx, __shfl_xor(mx, 2));

  const float range = mx - mn;
  const float s32 = __fdiv_rn(range, 15.0f);
  const __half s16 = __float2half_rn(s32);
  const __half b16 = __float2half_rn(mn);
  const float s = __half2float(s16);
  const float b = __half2float(b16);
  uint32_t word = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float diff = v[e] - b;
      const float tq = __fdiv_rn(diff, s);
      const float q = fminf(fmaxf(rintf(tq), 0.0f), 15.0f);
      word |= (uint32_t)q << (4 * e);
    }
  }
  if (valid) {
    codes[t] = word;
    if ((t & 3) == 0) {
      scales[(t >> 2) * sb_stride] = __builtin_bit_cast(uint16_t, s16);
      biases[(t >> 2) * sb_stride] = __builtin_bit_cast(uint16_t, b16);
    }
  }
}

}  // namespace

hipError_t launch_quantize_mlx4g32(const uint16_t *x, int64_t rows, int D, uint32_t *codes,
                                   uint16_t *scales, uint16_t *biases, int sb_stride,
                                   hipStream_t s) {
  const int64_t nwords = rows * (D / 8);
  if (nwords <= 0) return hipSuccess;
  if (sb_stride != 1 && sb_stride != 2) return hipErrorInvalidValue;
  const int64_t blocks = (nwords + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_mlx4g32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x,
                     nwords, codes, scales, biases, sb_stride);
  return hipGetLastError();
}

}  // namespace pion
