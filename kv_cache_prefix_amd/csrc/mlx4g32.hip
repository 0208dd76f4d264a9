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
// 16 B per lane and stores 4 B per lane, contiguous across the wave.
//
// Arithmetic, each step equal to its IEEE fp32 round-to-nearest-even counterpart:
//   x - b        one fused v_fma_mix (x fp16, times 1, minus b): a single rounding;
//   range / 15   q = fl(range * c), c = fl(1/15), then fl(q + fma(-q, 15, range) * c)
//                by two fmas: equal to the correctly rounded quotient for every
//                non-negative finite fp32 range (checked exhaustively on the host);
//   (x - b) / s  rounds to the same integer as t = fl((x - b) * rcp(s)) unless t lies
//                within 2^-16 of a half-integer: v_rcp_f32 is within 1 ulp of 1/s for
//                every fp16 s (checked on the device), so |t - fl((x - b)/s)| <=
//                2^-22 |t| and |t| < 22.5 (s >= range / 22.5 even where s rounds to an
//                fp16 subnormal); such elements take the correctly rounded divide (a
//                wave-uniform branch, rare);
//   rint, clamp  v_med3 to [0, 15], then v_cvt_pk_u8_f32 (round to nearest even, as
//                checked on the device) packs four codes per word: even elements in one
//                word, odd ones in another, merged as lo | hi << 4.
// No contraction elsewhere, so the codes are bit-exact with any IEEE fp32 evaluation
// of the steps above.
#include "mlx4g32.h"

#include <hip/hip_fp16.h>

namespace pion {
namespace {

// v from the lane given by a quad_perm DPP control (all rows and banks)
template <int CTRL>
__device__ __forceinline__ float quad_xor(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

__device__ __forceinline__ float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));

// Packed fp16 min / max of two words (inputs are finite: no quieting needed).
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
  uint32_t d;
  __asm__("v_pk_min_f16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  uint32_t d;
  __asm__("v_pk_max_f16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
// fl(x - b) for the fp16 x in the low (HI = 0) or high half of w: one fused operation
// (x * 1 + nb, nb = -b), rounded once
template <int HI>
__device__ __forceinline__ float sub_f16(uint32_t w, float nb) {
  float d;
  if constexpr (HI)
    __asm__("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(nb));
  else
    __asm__("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(nb));
  return d;
}

// Encode code word t (elements 8t .. 8t+7) from its 16 loaded bytes; the four words of
// a group are in one lane quad. SBW: scale and bias share a 32-bit word (scale low).
template <bool SBW>
__device__ __forceinline__ void encode_word(uint4 raw, int64_t t, bool valid,
                                            uint32_t *__restrict__ codes,
                                            uint16_t *__restrict__ scales,
                                            uint16_t *__restrict__ biases, int sb_stride) {
#pragma clang fp contract(off)
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  // group min and max in one packed fp16 word (min, -max), so that one packed min
  // per step reduces both: over the lane's four words, then over the lane quad
  // (4k..4k+3) by quad_perm moves
  const uint32_t m2 = pk_min(pk_min(w[0], w[1]), pk_min(w[2], w[3]));
  const uint32_t x2 = pk_max(pk_max(w[0], w[1]), pk_max(w[2], w[3])) ^ 0x80008000u;  // -max
  uint32_t pm = pk_min(__builtin_amdgcn_perm(x2, m2, 0x05040100u),   // (m2.lo, x2.lo)
                       __builtin_amdgcn_perm(x2, m2, 0x07060302u));  // (m2.hi, x2.hi)
  pm = pk_min(pm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pm, 0xB1, 0xF, 0xF, true));  // lane ^ 1
  pm = pk_min(pm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pm, 0x4E, 0xF, 0xF, true));  // lane ^ 2
  float mn = h2f((uint16_t)(pm & 0xffffu));
  float mx = -h2f((uint16_t)(pm >> 16));
  // Signed zeros: -0 orders below +0, so a zero minimum is -0 when the group holds a -0
  // and a zero maximum is +0 when it holds a +0 (the min / max above return either zero).
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
  const float c15 = 1.0f / 15.0f;  // fl(1/15)
  const float q15 = range * c15;
  const float s32 = __builtin_fmaf(__builtin_fmaf(-q15, 15.0f, range), c15, q15);
  const __half s16 = __float2half_rn(s32);
  const __half b16 = __float2half_rn(mn);  // exact: mn is one of the fp16 inputs
  const float s = __half2float(s16);
  const float nb = -__half2float(b16);
  uint32_t word = 0;
  if (s != 0.0f) {
    const float r = __builtin_amdgcn_rcpf(s);
    float diff[8], tq[8], dh[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      diff[2 * c] = sub_f16<0>(w[c], nb);
      diff[2 * c + 1] = sub_f16<1>(w[c], nb);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tq[e] = diff[e] * r;
      dh[e] = fabsf(__builtin_amdgcn_fractf(tq[e]) - 0.5f);  // distance to k + 1/2
    }
    // the smallest distance (the compiler forms three-input mins)
    float dmin = fminf(fminf(fminf(dh[0], dh[1]), fminf(dh[2], dh[3])),
                       fminf(fminf(dh[4], dh[5]), fminf(dh[6], dh[7])));
    const bool near = !(dmin > 0x1p-16f);
    // rare: a wave-uniform branch, so the divides run only for waves that need them
    if (__builtin_amdgcn_ballot_w64(near)) {
      if (near) {
#pragma unroll
        for (int e = 0; e < 8; ++e) tq[e] = __fdiv_rn(diff[e], s);
      }
    }
    uint32_t ev = 0, od = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ev = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(tq[2 * k], 0.0f, 15.0f), k, ev);
      od = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(tq[2 * k + 1], 0.0f, 15.0f), k, od);
    }
    word = ev | (od << 4);
  }
  if (valid) {
    __builtin_nontemporal_store(word, codes + t);
    if ((t & 3) == 0) {
      const uint16_t sb = __builtin_bit_cast(uint16_t, s16), bb = __builtin_bit_cast(uint16_t, b16);
      if constexpr (SBW) {
        __builtin_nontemporal_store((uint32_t)sb | ((uint32_t)bb << 16),
                                    (uint32_t *)scales + (t >> 2));
      } else {
        scales[(t >> 2) * sb_stride] = sb;
        biases[(t >> 2) * sb_stride] = bb;
      }
    }
  }
}

// One tensor's input rows and output arrays.
struct QuantTensor {
  const uint16_t *x;
  uint32_t *codes;
  uint16_t *scales, *biases;
};

// One code word per lane and chunk: workgroup x encodes the kWords chunks of 256 words
// from word 256 kWords x, lane i word 256 (kWords x + k) + i of chunk k; all chunks'
// loads are issued before the first is encoded (more bytes in flight per wave). Grid row
// y encodes tensor y (a, or b for y = 1: the K and V of a store in one launch).
constexpr int kWords = 4;
template <bool SBW>
__global__ __launch_bounds__(256) void quantize_mlx4g32_kernel(QuantTensor qa, QuantTensor qb,
                                                               int64_t nwords, int sb_stride) {
  const QuantTensor q = blockIdx.y ? qb : qa;
  const uint16_t *__restrict__ x = q.x;
  uint32_t *__restrict__ codes = q.codes;
  uint16_t *__restrict__ scales = q.scales;
  uint16_t *__restrict__ biases = q.biases;
  const int64_t t0 = (int64_t)blockIdx.x * (256 * kWords) + threadIdx.x;
  uint4 raw[kWords];
#pragma unroll
  for (int k = 0; k < kWords; ++k) {
    const int64_t t = t0 + 256 * k;
    if (t < nwords) {
      const nt_u32x4 v = __builtin_nontemporal_load((const nt_u32x4 *)(x + t * 8));
      raw[k] = make_uint4(v.x, v.y, v.z, v.w);
    } else {
      raw[k] = make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int k = 0; k < kWords; ++k) {
    const int64_t t = t0 + 256 * k;
    encode_word<SBW>(raw[k], t, t < nwords, codes, scales, biases, sb_stride);
  }
}

}  // namespace

hipError_t launch_quantize_mlx4g32(const uint16_t *x, int64_t rows, int D, uint32_t *codes,
                                   uint16_t *scales, uint16_t *biases, int sb_stride,
                                   hipStream_t s) {
  const int64_t nwords = rows * (D / 8);
  if (nwords <= 0) return hipSuccess;
  if (sb_stride != 1 && sb_stride != 2) return hipErrorInvalidValue;
  const int64_t blocks = (nwords + 256 * kWords - 1) / (256 * kWords);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  // scale and bias interleaved in one 32-bit word (the slot layout): one store
  const bool sbw = sb_stride == 2 && biases == scales + 1 && ((uintptr_t)scales & 3) == 0;
  const QuantTensor q{x, codes, scales, biases};
  note_launch("quantize_mlx4g32_kernel<%d>", (int)sbw);
  if (sbw)
    hipLaunchKernelGGL(quantize_mlx4g32_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, q,
                       q, nwords, sb_stride);
  else
    hipLaunchKernelGGL(quantize_mlx4g32_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, q,
                       q, nwords, sb_stride);
  return hipGetLastError();
}

hipError_t launch_quantize_mlx4g32_pair(const uint16_t *xa, uint32_t *codes_a, uint32_t *sb_a,
                                        const uint16_t *xb, uint32_t *codes_b, uint32_t *sb_b,
                                        int64_t rows, int D, hipStream_t s) {
  const int64_t nwords = rows * (D / 8);
  if (nwords <= 0) return hipSuccess;
  const int64_t blocks = (nwords + 256 * kWords - 1) / (256 * kWords);
  if (blocks > 0x7fffffffLL || ((uintptr_t)sb_a & 3) || ((uintptr_t)sb_b & 3))
    return hipErrorInvalidValue;
  const QuantTensor qa{xa, codes_a, (uint16_t *)sb_a, (uint16_t *)sb_a + 1};
  const QuantTensor qb{xb, codes_b, (uint16_t *)sb_b, (uint16_t *)sb_b + 1};
  note_launch("quantize_mlx4g32_kernel<1>");
  hipLaunchKernelGGL(quantize_mlx4g32_kernel<true>, dim3((unsigned)blocks, 2), dim3(256), 0, s,
                     qa, qb, nwords, 2);
  return hipGetLastError();
}

}  // namespace pion
