// V-store side of the prefix cache: the dequantizing range fetch (V.FETCH ... RANGE) and
// the rehydrate relayout of one layer's V-store rows into a resident slot
// (KV.PREFIX.WARM), "Shared KV Cache Serving" and the V-store page.
//
// A V-store layer holds one row per token, kv = H * D values wide: fp16 values, or the
// mlx4g32 record [kv/8 uint32 code words][kv/32 fp16 scales][kv/32 fp16 biases]
// ("The mlx4g32 tier"; 0.625 * kv bytes, a multiple of 4). Dequantized value of element
// e of group g: s_g * c_e + b_g, computed as one fp32 fma (s * c is exact, so it is the
// exact value rounded once); an fp16 slot takes it rounded to fp16.
//
// Every kernel gives one thread one "chunk" (n, k) of a token row: 8 consecutive values,
// that is one code word or 16 fp16 bytes, k in [0, kv/8). Row-major chunk order keeps
// the V-store side (the larger one) contiguous across a wave; the slot side is written
// in runs of D/8 chunks (head rows [h, n, :]). Bandwidth-bound: no LDS, no reuse.
#include "kernels.h"

namespace pion {
namespace {

struct Chunk {
  int64_t n;  // token
  int k;      // chunk within the token row
};

__device__ __forceinline__ Chunk chunk_of(int64_t i, int kc) {
  Chunk c;
  c.n = i / kc;
  c.k = (int)(i - c.n * kc);
  return c;
}

typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once16(const uint8_t *p) {  // read once: non-temporal
  const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt *)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float half_bits(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)u);
}
__device__ __forceinline__ uint16_t to_half_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
}

// Dequantize the 8 elements of code word k of a record.
__device__ __forceinline__ void dequant8(const uint8_t *rec, int kv, int k, float (&x)[8]) {
  const uint32_t w = *(const uint32_t *)(rec + 4 * k);
  const int g = k >> 2;  // 4 words per group of 32
  const float s = half_bits(*(const uint16_t *)(rec + kv / 2 + 2 * g));
  const float b = half_bits(*(const uint16_t *)(rec + kv / 2 + kv / 16 + 2 * g));
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(s, (float)((w >> (4 * e)) & 0xFu), b);
}

// V.FETCH RANGE: out[n - start][8k .. 8k + 7] in fp32.
template <int FMT>
__global__ __launch_bounds__(256) void fetch_f32_kernel(const uint8_t *__restrict__ rows, int kv,
                                                        int64_t start, int64_t count,
                                                        float *__restrict__ out) {
  const int kc = kv / 8;
  const int64_t total = count * kc;
  const int64_t rb = FMT == 0 ? 2LL * kv : (int64_t)kv * 5 / 8;  // row bytes
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const Chunk c = chunk_of(i, kc);
    const uint8_t *row = rows + (start + c.n) * rb;
    float x[8];
    if (FMT == 0) {
      const uint4 v = load_once16(row + 16 * c.k);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = half_bits(w[j] & 0xffffu);
        x[2 * j + 1] = half_bits(w[j] >> 16);
      }
    } else {
      dequant8(row, kv, c.k, x);
    }
    float4 *o = (float4 *)(out + i * 8);
    o[0] = make_float4(x[0], x[1], x[2], x[3]);
    o[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// KV.PREFIX.WARM into an fp16 slot: rows [N, H*D] -> dst [H, N, D].
template <int FMT>
__global__ __launch_bounds__(256) void rows_to_fp16_slot_kernel(const uint8_t *__restrict__ rows,
                                                                int64_t N, int H, int D,
                                                                uint16_t *__restrict__ dst) {
  const int kv = H * D, kc = kv / 8, dc = D / 8;
  const int64_t total = N * kc;
  const int64_t rb = FMT == 0 ? 2LL * kv : (int64_t)kv * 5 / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const Chunk c = chunk_of(i, kc);
    const uint8_t *row = rows + c.n * rb;
    const int h = c.k / dc, d8 = c.k - h * dc;
    uint4 v;
    if (FMT == 0) {
      v = load_once16(row + 16 * c.k);
    } else {
      float x[8];
      dequant8(row, kv, c.k, x);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)to_half_bits(x[2 * j]) | ((uint32_t)to_half_bits(x[2 * j + 1]) << 16);
      v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    *(uint4 *)(dst + (((int64_t)h * N + c.n) * D + 8 * d8)) = v;
  }
}

// KV.PREFIX.WARM into an mlx4g32 slot from mlx4g32 rows: the codes and the (scale |
// bias << 16) pairs move to the slot layout unchanged.
__global__ __launch_bounds__(256) void rows_to_mlx4_slot_kernel(const uint8_t *__restrict__ rows,
                                                                int64_t N, int H, int D,
                                                                uint32_t *__restrict__ codes,
                                                                uint32_t *__restrict__ pairs) {
  const int kv = H * D, kc = kv / 8, dc = D / 8;
  const int64_t total = N * kc;
  const int64_t rb = (int64_t)kv * 5 / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const Chunk c = chunk_of(i, kc);
    const uint8_t *row = rows + c.n * rb;
    const int h = c.k / dc, w = c.k - h * dc;
    const int64_t slot_row = (int64_t)h * N + c.n;
    codes[slot_row * dc + w] = *(const uint32_t *)(row + 4 * c.k);
    if ((w & 3) == 0) {
      const int g = c.k >> 2;
      const uint32_t s = *(const uint16_t *)(row + kv / 2 + 2 * g);
      const uint32_t b = *(const uint16_t *)(row + kv / 2 + kv / 16 + 2 * g);
      pairs[slot_row * (D / 32) + (w >> 2)] = s | (b << 16);
    }
  }
}

int grid_for(int64_t total) {
  const int64_t b = (total + 255) / 256;
  return (int)(b < 1 ? 1 : b > (1 << 20) ? (1 << 20) : b);
}

}  // namespace

hipError_t launch_vstore_fetch(const void *rows, int fmt, int kv, int64_t start, int64_t count,
                               float *out, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int g = grid_for(count * (kv / 8));
  if (fmt == 0)
    hipLaunchKernelGGL(fetch_f32_kernel<0>, dim3(g), dim3(256), 0, s, (const uint8_t *)rows, kv,
                       start, count, out);
  else
    hipLaunchKernelGGL(fetch_f32_kernel<1>, dim3(g), dim3(256), 0, s, (const uint8_t *)rows, kv,
                       start, count, out);
  return hipGetLastError();
}

hipError_t launch_rows_to_fp16_slot(const void *rows, int fmt, int64_t N, int H, int D,
                                    uint16_t *dst, hipStream_t s) {
  const int g = grid_for(N * (H * D / 8));
  if (fmt == 0)
    hipLaunchKernelGGL(rows_to_fp16_slot_kernel<0>, dim3(g), dim3(256), 0, s,
                       (const uint8_t *)rows, N, H, D, dst);
  else
    hipLaunchKernelGGL(rows_to_fp16_slot_kernel<1>, dim3(g), dim3(256), 0, s,
                       (const uint8_t *)rows, N, H, D, dst);
  return hipGetLastError();
}

hipError_t launch_rows_to_mlx4_slot(const void *rows, int64_t N, int H, int D, uint32_t *codes,
                                    uint32_t *pairs, hipStream_t s) {
  const int g = grid_for(N * (H * D / 8));
  hipLaunchKernelGGL(rows_to_mlx4_slot_kernel, dim3(g), dim3(256), 0, s, (const uint8_t *)rows,
                     N, H, D, codes, pairs);
  return hipGetLastError();
}

}  // namespace pion
