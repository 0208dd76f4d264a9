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
// Work items are small and adjacent lanes take adjacent items, so every load and store
// instruction of a wave covers one contiguous run (fully coalesced): the fetch gives a
// lane 4 output values (16 B of fp32), the rehydrate one code word / 8 values (16 B of
// fp16 out). Each lane takes 4 items a stride apart per loop trip, loads first, so 4
// loads are in flight. Row-major item order keeps the V-store side contiguous; the slot
// side is written in runs of a head row (D values). Bandwidth-bound: no LDS, no reuse;
// the fetch output is stored non-temporally.
#include "kernels.h"

namespace pion {
namespace {

constexpr int kUnroll = 1;

// Item index i -> (token, item in the row); 32-bit arithmetic when the grid allows.
struct Item {
  int64_t n;
  int k;
};
template <bool WIDE>
__device__ __forceinline__ Item item_of(int64_t i, int per_row) {
  Item c;
  if (WIDE) {
    c.n = i / per_row;
    c.k = (int)(i - c.n * per_row);
  } else {
    const uint32_t u = (uint32_t)i, n = u / (uint32_t)per_row;
    c.n = n;
    c.k = (int)(u - n * (uint32_t)per_row);
  }
  return c;
}

typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_nt __attribute__((ext_vector_type(2)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once16(const uint8_t *p) {  // read once: non-temporal
  const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt *)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float half_bits(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)u);
}
__device__ __forceinline__ uint32_t pack_half2(float a, float b) {  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// Code word k of a record with its group's scale and bias (4 words per group of 32).
struct Word {
  uint32_t w;
  uint16_t s16, b16;
};
__device__ __forceinline__ Word read_word(const uint8_t *rec, int kv, int k) {
  Word r;
  r.w = *(const uint32_t *)(rec + 4 * k);
  r.s16 = *(const uint16_t *)(rec + kv / 2 + 2 * (k >> 2));
  r.b16 = *(const uint16_t *)(rec + kv / 2 + kv / 16 + 2 * (k >> 2));
  return r;
}
// Element e of the word: s * code + b as one fp32 fma (s * code is exact).
__device__ __forceinline__ float dq(const Word &r, int e) {
  return __builtin_fmaf(half_bits(r.s16), (float)((r.w >> (4 * e)) & 0xFu), half_bits(r.b16));
}

// V.FETCH RANGE: out[n - start][4 q .. 4 q + 3] in fp32, q in [0, kv/4).
template <int FMT, bool WIDE>
__global__ __launch_bounds__(256) void fetch_f32_kernel(const uint8_t *__restrict__ rows, int kv,
                                                        int64_t start, int64_t count,
                                                        float *__restrict__ out) {
  const int qpr = kv / 4;
  const int64_t total = count * qpr, stride = (int64_t)gridDim.x * 256;
  const int64_t rb = FMT == 0 ? 2LL * kv : (int64_t)kv * 5 / 8;  // row bytes
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < total; i0 += kUnroll * stride) {
    f32x4_nt v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i >= total) break;
      const Item c = item_of<WIDE>(i, qpr);
      const uint8_t *row = rows + (start + c.n) * rb;
      if (FMT == 0) {
        const u32x2_nt h = __builtin_nontemporal_load((const u32x2_nt *)(row + 8 * c.k));
        v[u] = f32x4_nt{half_bits(h.x & 0xffffu), half_bits(h.x >> 16), half_bits(h.y & 0xffffu),
                        half_bits(h.y >> 16)};
      } else {
        Word r = read_word(row, kv, c.k >> 1);
        r.w >>= 16 * (c.k & 1);  // this lane's 4 codes
        v[u] = f32x4_nt{dq(r, 0), dq(r, 1), dq(r, 2), dq(r, 3)};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i >= total) break;
      __builtin_nontemporal_store(v[u], (f32x4_nt *)(out + 4 * i));
    }
  }
}

// KV.PREFIX.WARM into an fp16 slot: rows [N, H*D] -> dst [H, N, D], 8 values per item.
template <int FMT, bool WIDE>
__global__ __launch_bounds__(256) void rows_to_fp16_slot_kernel(const uint8_t *__restrict__ rows,
                                                                int64_t N, int H, int D,
                                                                uint16_t *__restrict__ dst) {
  const int kv = H * D, wpr = kv / 8, dc = D / 8;
  const int64_t total = N * wpr, stride = (int64_t)gridDim.x * 256;
  const int64_t rb = FMT == 0 ? 2LL * kv : (int64_t)kv * 5 / 8;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < total; i0 += kUnroll * stride) {
    uint4 v[kUnroll];
    int64_t o[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i >= total) break;
      const Item c = item_of<WIDE>(i, wpr);
      const uint8_t *row = rows + c.n * rb;
      const int h = c.k / dc, d8 = c.k - h * dc;
      o[u] = ((int64_t)h * N + c.n) * D + 8 * d8;
      if (FMT == 0) {
        v[u] = load_once16(row + 16 * c.k);
      } else {
        const Word r = read_word(row, kv, c.k);
        v[u] = make_uint4(pack_half2(dq(r, 0), dq(r, 1)), pack_half2(dq(r, 2), dq(r, 3)),
                          pack_half2(dq(r, 4), dq(r, 5)), pack_half2(dq(r, 6), dq(r, 7)));
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (i0 + u * stride >= total) break;
      *(uint4 *)(dst + o[u]) = v[u];
    }
  }
}

// KV.PREFIX.WARM into an fp32 slot: rows [N, H*D] -> dst [H, N, D], 4 values per item
// (the fetch's values, transposed).
template <int FMT, bool WIDE>
__global__ __launch_bounds__(256) void rows_to_fp32_slot_kernel(const uint8_t *__restrict__ rows,
                                                                int64_t N, int H, int D,
                                                                float *__restrict__ dst) {
  const int kv = H * D, qpr = kv / 4, dq4 = D / 4;
  const int64_t total = N * qpr, stride = (int64_t)gridDim.x * 256;
  const int64_t rb = FMT == 0 ? 2LL * kv : (int64_t)kv * 5 / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const Item c = item_of<WIDE>(i, qpr);
    const uint8_t *row = rows + c.n * rb;
    const int h = c.k / dq4, d4 = c.k - h * dq4;
    f32x4_nt v;
    if (FMT == 0) {
      const u32x2_nt x = __builtin_nontemporal_load((const u32x2_nt *)(row + 8 * c.k));
      v = f32x4_nt{half_bits(x.x & 0xffffu), half_bits(x.x >> 16), half_bits(x.y & 0xffffu),
                   half_bits(x.y >> 16)};
    } else {
      Word r = read_word(row, kv, c.k >> 1);
      r.w >>= 16 * (c.k & 1);
      v = f32x4_nt{dq(r, 0), dq(r, 1), dq(r, 2), dq(r, 3)};
    }
    *(f32x4_nt *)(dst + ((int64_t)h * N + c.n) * D + 4 * d4) = v;
  }
}

// KV.PREFIX.WARM into an mlx4g32 slot from mlx4g32 rows: the codes and the (scale |
// bias << 16) pairs move to the slot layout unchanged, one code word per item.
template <bool WIDE>
__global__ __launch_bounds__(256) void rows_to_mlx4_slot_kernel(const uint8_t *__restrict__ rows,
                                                                int64_t N, int H, int D,
                                                                uint32_t *__restrict__ codes,
                                                                uint32_t *__restrict__ pairs) {
  const int kv = H * D, wpr = kv / 8, dc = D / 8;
  const int64_t total = N * wpr, stride = (int64_t)gridDim.x * 256;
  const int64_t rb = (int64_t)kv * 5 / 8;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < total; i0 += kUnroll * stride) {
    Word r[kUnroll];
    int64_t slot_row[kUnroll];
    int w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i >= total) break;
      const Item c = item_of<WIDE>(i, wpr);
      r[u] = read_word(rows + c.n * rb, kv, c.k);
      const int h = c.k / dc;
      w[u] = c.k - h * dc;
      slot_row[u] = (int64_t)h * N + c.n;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (i0 + u * stride >= total) break;
      codes[slot_row[u] * dc + w[u]] = r[u].w;
      if ((w[u] & 3) == 0)
        pairs[slot_row[u] * (D / 32) + (w[u] >> 2)] = (uint32_t)r[u].s16 | ((uint32_t)r[u].b16 << 16);
    }
  }
}

int grid_for(int64_t total) {
  const int64_t b = (total + 256 * kUnroll - 1) / (256 * kUnroll);
  return (int)(b < 1 ? 1 : b > (1 << 20) ? (1 << 20) : b);
}

// 32-bit group indexing while every index of the grid-stride loop fits
bool narrow(int64_t total) { return total + (int64_t)kUnroll * (1 << 20) * 256 < (1LL << 31); }

}  // namespace

hipError_t launch_vstore_fetch(const void *rows, int fmt, int kv, int64_t start, int64_t count,
                               float *out, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int64_t total = count * (kv / 4);
  const dim3 g(grid_for(total)), b(256);
  const uint8_t *r = (const uint8_t *)rows;
  note_launch("fetch_f32_kernel<%d,%s>", fmt, narrow(total) ? "false" : "true");
  if (fmt == 0) {
    if (narrow(total)) hipLaunchKernelGGL((fetch_f32_kernel<0, false>), g, b, 0, s, r, kv, start, count, out);
    else hipLaunchKernelGGL((fetch_f32_kernel<0, true>), g, b, 0, s, r, kv, start, count, out);
  } else {
    if (narrow(total)) hipLaunchKernelGGL((fetch_f32_kernel<1, false>), g, b, 0, s, r, kv, start, count, out);
    else hipLaunchKernelGGL((fetch_f32_kernel<1, true>), g, b, 0, s, r, kv, start, count, out);
  }
  return hipGetLastError();
}

hipError_t launch_rows_to_fp16_slot(const void *rows, int fmt, int64_t N, int H, int D,
                                    uint16_t *dst, hipStream_t s) {
  const int64_t total = N * (H * D / 8);
  const dim3 g(grid_for(total)), b(256);
  const uint8_t *r = (const uint8_t *)rows;
  note_launch("rows_to_fp16_slot_kernel<%d,%s>", fmt, narrow(total) ? "false" : "true");
  if (fmt == 0) {
    if (narrow(total)) hipLaunchKernelGGL((rows_to_fp16_slot_kernel<0, false>), g, b, 0, s, r, N, H, D, dst);
    else hipLaunchKernelGGL((rows_to_fp16_slot_kernel<0, true>), g, b, 0, s, r, N, H, D, dst);
  } else {
    if (narrow(total)) hipLaunchKernelGGL((rows_to_fp16_slot_kernel<1, false>), g, b, 0, s, r, N, H, D, dst);
    else hipLaunchKernelGGL((rows_to_fp16_slot_kernel<1, true>), g, b, 0, s, r, N, H, D, dst);
  }
  return hipGetLastError();
}

hipError_t launch_rows_to_fp32_slot(const void *rows, int fmt, int64_t N, int H, int D,
                                    float *dst, hipStream_t s) {
  const int64_t total = N * (H * D / 4);
  const dim3 g(grid_for(total)), b(256);
  const uint8_t *r = (const uint8_t *)rows;
  note_launch("rows_to_fp32_slot_kernel<%d,%s>", fmt, narrow(total) ? "false" : "true");
  if (fmt == 0) {
    if (narrow(total)) hipLaunchKernelGGL((rows_to_fp32_slot_kernel<0, false>), g, b, 0, s, r, N, H, D, dst);
    else hipLaunchKernelGGL((rows_to_fp32_slot_kernel<0, true>), g, b, 0, s, r, N, H, D, dst);
  } else {
    if (narrow(total)) hipLaunchKernelGGL((rows_to_fp32_slot_kernel<1, false>), g, b, 0, s, r, N, H, D, dst);
    else hipLaunchKernelGGL((rows_to_fp32_slot_kernel<1, true>), g, b, 0, s, r, N, H, D, dst);
  }
  return hipGetLastError();
}

hipError_t launch_rows_to_mlx4_slot(const void *rows, int64_t N, int H, int D, uint32_t *codes,
                                    uint32_t *pairs, hipStream_t s) {
  const int64_t total = N * (H * D / 8);
  const dim3 g(grid_for(total)), b(256);
  const uint8_t *r = (const uint8_t *)rows;
  note_launch("rows_to_mlx4_slot_kernel<%s>", narrow(total) ? "false" : "true");
  if (narrow(total)) hipLaunchKernelGGL((rows_to_mlx4_slot_kernel<false>), g, b, 0, s, r, N, H, D, codes, pairs);
  else hipLaunchKernelGGL((rows_to_mlx4_slot_kernel<true>), g, b, 0, s, r, N, H, D, codes, pairs);
  return hipGetLastError();
}

}  // namespace pion
