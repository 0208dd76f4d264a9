// mlx4g32 encoder: int4 codes, group 32, affine, fp16 scale and bias per group, the
// scale rounded to fp16 before the codes are chosen ("Shared KV Cache Serving",
// Quantized tier - mlx4g32; V-store page, The mlx4g32 tier).
//
// Per group, in fp32 with IEEE round-to-nearest-even on every op:
//   mn = min x, mx = max x, s = fp16((mx - mn) / 15), b = fp16(mn),
//   q = clamp(rint((x - b) / s), 0, 15), or all zero when s == 0.
// The minimum and maximum order -0 below +0, so the bias of a group whose minimum is
// zero is -0 exactly when the group holds a -0. Inputs must be finite.
// Element i of a row goes to word i/8 at bits 4*(i%8).
//
// Layout: one lane per uint32 code word (8 elements, 16 input bytes), so four
// consecutive lanes hold one group; min/max combine across those four lanes. Loads are
// 16 B per lane and stores 4 B per lane, contiguous across the wave. The scale uses the
// correctly rounded fp32 divide; the codes round the correctly rounded quotient (a
// product with the reciprocal where that provably rounds the same, else the divide), and
// there is no contraction, so the codes are bit-exact with any IEEE fp32 evaluation of
// the steps above.
#include "kernels.h"

#include <hip/hip_fp16.h>

namespace pion {
namespace {

// v from the lane given by a quad_perm DPP control (all rows and banks)
template <int CTRL>
__device__ __forceinline__ float quad_xor(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// Encode code word t (elements 8t .. 8t+7) from its 16 loaded bytes; the four words of
// a group are in one lane quad.
__device__ __forceinline__ void encode_word(uint4 raw, int64_t t, bool valid,
                                            uint32_t *__restrict__ codes,
                                            uint16_t *__restrict__ scales,
                                            uint16_t *__restrict__ biases, int sb_stride) {
#pragma clang fp contract(off)
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
  // the four lanes of a group are a lane quad (4k..4k+3): quad_perm moves
  mn = fminf(mn, quad_xor<0xB1>(mn));  // lane ^ 1
  mn = fminf(mn, quad_xor<0x4E>(mn));  // lane ^ 2
  mx = fmaxf(mx, quad_xor<0xB1>(mx));
  mx = fmaxf(mx, quad_xor<0x4E>(mx));
  // Signed zeros: -0 orders below +0, so a zero minimum is -0 when the group holds a -0
  // and a zero maximum is +0 when it holds a +0 (fminf / fmaxf return either zero).
  // Rare, and the branch is wave-uniform.
  if (__builtin_amdgcn_ballot_w64(mn == 0.0f || mx == 0.0f)) {
    int negz = 0, posz = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      negz |= (int)((w[c] & 0xffffu) == 0x8000u) | (int)((w[c] >> 16) == 0x8000u);
      posz |= (int)((w[c] & 0xffffu) == 0u) | (int)((w[c] >> 16) == 0u);
    }
    negz |= __builtin_bit_cast(int, quad_xor<0xB1>(__builtin_bit_cast(float, negz)));
    negz |= __builtin_bit_cast(int, quad_xor<0x4E>(__builtin_bit_cast(float, negz)));
    posz |= __builtin_bit_cast(int, quad_xor<0xB1>(__builtin_bit_cast(float, posz)));
    posz |= __builtin_bit_cast(int, quad_xor<0x4E>(__builtin_bit_cast(float, posz)));
    if (mn == 0.0f) mn = negz ? -0.0f : 0.0f;
    if (mx == 0.0f) mx = posz ? 0.0f : -0.0f;
  }

  const float range = mx - mn;
  const float s32 = __fdiv_rn(range, 15.0f);
  const __half s16 = __float2half_rn(s32);
  const __half b16 = __float2half_rn(mn);
  const float s = __half2float(s16);
  const float b = __half2float(b16);
  uint32_t word = 0;
  if (s != 0.0f) {
    // rint of the correctly rounded quotient diff / s, without a divide per element:
    // with r = fl(1 / s), fl(diff * r) is within 3 * 2^-24 * |diff / s| of fl(diff / s)
    // (three roundings of relative size <= 2^-24), so the two round to the same integer
    // unless a half-integer lies that close; such elements (and non-finite ones) take the
    // correctly rounded divide.
    const float r = __fdiv_rn(1.0f, s);
    float diff[8], tq[8];
    bool near = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      diff[e] = v[e] - b;
      tq[e] = diff[e] * r;
      const float gap = fabsf(tq[e] - (floorf(tq[e]) + 0.5f));  // to the nearest half-integer
      near |= !(gap > fabsf(tq[e]) * 0x1p-20f);                 // NaN counts as near
    }
    // rare: a wave-uniform branch, so the divides run only for waves that need them
    if (__builtin_amdgcn_ballot_w64(near)) {
      if (near) {
#pragma unroll
        for (int e = 0; e < 8; ++e) tq[e] = __fdiv_rn(diff[e], s);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q = fminf(fmaxf(rintf(tq[e]), 0.0f), 15.0f);
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

// One code word per lane: lane t of the grid encodes word t.
__global__ __launch_bounds__(256) void quantize_mlx4g32_kernel(const uint16_t *__restrict__ x,
                                                               int64_t nwords,
                                                               uint32_t *__restrict__ codes,
                                                               uint16_t *__restrict__ scales,
                                                               uint16_t *__restrict__ biases,
                                                               int sb_stride) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = t < nwords;
  const uint4 raw = valid ? *(const uint4 *)(x + t * 8) : make_uint4(0, 0, 0, 0);
  encode_word(raw, t, valid, codes, scales, biases, sb_stride);
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
  note_launch("quantize_mlx4g32_kernel");
  hipLaunchKernelGGL(quantize_mlx4g32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x,
                     nwords, codes, scales, biases, sb_stride);
  return hipGetLastError();
}

}  // namespace pion
