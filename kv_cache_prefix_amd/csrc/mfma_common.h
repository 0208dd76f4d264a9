// Device helpers shared by the fp16 MFMA attention kernels (batched-Q prefill and the
// grouped-query decode): operand vector types, LDS-writing buffer loads, the LDS row
// swizzle with its transposed V reads, and cross-half lane combines.
//
// Operand layouts (v_mfma_f32_32x32x16_f16, each checked on the device): A lane l holds
// A[l % 32][8 (l / 32) + e], B holds B[8 (l / 32) + e][l % 32], and element 4 i + j of
// the 16-float result of lane l is C[8 i + 4 (l / 32) + j][l % 32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pion {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));  // builtin type
#define LDS_PTR(T, x) ((__attribute__((address_space(3))) T *)(x))

// The max / sum of lanes l and l ^ 32 in every lane, through the cross-half lane swap
// (no LDS round trip): the swap leaves lane l holding x[l % 32] in one result and
// x[l % 32 + 32] in the other.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Physical 16-byte chunk of logical chunk c in tile row r is c ^ swz(r) (found by an
// exhaustive search for conflict-free K reads and transposed V reads, 64 banks). It
// depends on r % 16 only.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 64) return ((r & 3) << 1) ^ ((r >> 1) & 7);
  else return ((r & 3) << 2) ^ ((r >> 2) & 3);
}

// Raw buffer descriptor words (0x00020000: raw 32-bit data format) for the LDS-writing
// loads.
__device__ __forceinline__ i32x4 rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), (int)bytes, 0x00020000};
}
// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane (lds uniform);
// past the buffer's end the bytes are zero. One wait state separates the M0 write from
// the load that reads it. The compiler cannot tell which LDS bytes such a load writes,
// so it is issued here, and the caller waits for it (s_waitcnt vmcnt) before reading.
// The compiler treats M0 as reserved and may ignore a clobber of it, so the statement
// saves M0 in an SGPR of its own and restores it after the load (the load reads M0 when
// it issues): whatever value the compiler keeps in M0 survives the call.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  uint32_t save;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(lds), "s"(rsrc)
      : "memory");
}

// Four such loads under one save and restore of M0: buffer ra at offsets v0, v1 into
// LDS l0, l1, then buffer rb at v0, v1 into l2, l3 (the K and V pieces of two 1 KB runs
// of a tile).
__device__ __forceinline__ void load_lds16_x4(i32x4 ra, i32x4 rb, uint32_t v0, uint32_t v1,
                                              uint32_t l0, uint32_t l1, uint32_t l2,
                                              uint32_t l3) {
  uint32_t save;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %7, 0 offen lds\n\t"
      "s_mov_b32 m0, %4\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %7, 0 offen lds\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %8, 0 offen lds\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %8, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(v0), "v"(v1), "s"(l0), "s"(l1), "s"(l2), "s"(l3), "s"(ra), "s"(rb)
      : "memory");
}

// A row max may grow by this much (log2 units, a factor 2^8) before the accumulators
// are rescaled: weights up to 2^8 stay exact enough in fp16 and the fp32 sums cannot
// overflow, and after the first tiles a rescale is rare.
constexpr float kRescaleSlack = 8.0f;

// Lane offsets of the transposed V reads of a 16-key k-step (ds_read_b64_tr_b16: in each
// 16-lane group, lane i receives element i % 4 of the 8-byte pieces addressed by lanes
// 4 j + i / 4): lane (group gq, index q) addresses row kbase + q / 4 at dims
// 32 db + 16 gq + 4 (q % 4), for kbase = 16 s + 4 hl + 8 c (c = 0, 1: the two runs of 4
// keys of the k-step), which gives it keys kbase .. kbase + 3 of one dim: the V^T
// operand in the k order of the P operand. voffs[c][db] is relative to the k-step's
// first row.
template <int D>
__device__ __forceinline__ void vt_offsets(int lane, uint32_t (&voffs)[2][D / 32]) {
  constexpr uint32_t ROWB = D * 2;
  const int hl = lane >> 5, q16 = lane & 15, gq = (lane >> 4) & 1;
  const int vch = 2 * gq + ((q16 & 3) >> 1);  // logical chunk minus 4 db
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 4 * hl + 8 * c + (q16 >> 2);  // row modulo 16
    const int vsw = swz<D>(r);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      voffs[c][db] = (uint32_t)r * ROWB + (uint32_t)(q16 & 1) * 8 +
                     (uint32_t)(((4 * db + vch) ^ vsw) << 4);
  }
}
// The V^T operand (32 dims x 16 keys) of 32-dim block db from the k-step at `base`.
template <int D>
__device__ __forceinline__ half8 vt_frag(const char *base, const uint32_t (&voffs)[2][D / 32],
                                         int db) {
  half4 part[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    part[c] = __builtin_bit_cast(
        half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(LDS_PTR(fp16x4_t, base + voffs[c][db])));
  return half8{part[0][0], part[0][1], part[0][2], part[0][3],
               part[1][0], part[1][1], part[1][2], part[1][3]};
}

}  // namespace
}  // namespace pion
