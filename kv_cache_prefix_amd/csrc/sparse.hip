// Block-mean top-K selection for the sparse-auto query ("Shared KV Cache Serving",
// Stage 2 sparse-mask paragraph: block-mean top-K from the resident K, block size B,
// K_top blocks; ATTEND.* page, QUERY_SPARSE_AUTO rows: K_mean cached per slot).
//
//   block_mean : K_mean[g, b, d] = (sum of K[g, j, d] over the tokens j of block b) / n_b,
//                summed in token order in fp32; one thread per (g, b, d), coalesced over d.
//   block_score: score[g, b] = sum over q-heads h with head_map[h] == g of q_h . K_mean[g, b];
//                one wave per (g, b).
//   block_topk : per kv-head, the min(K_top, nb) best blocks by (score desc, index asc),
//                found as K_top successive arg-max passes over the scores (each pass
//                takes the best block ranked strictly after the previous pick), then
//                written in ascending index order, -1 past nb.
// The arithmetic of a block depends only on its own data, so identical blocks get
// identical scores and the lower index wins the tie.
#include "kernels.h"

namespace pion {
namespace {

__device__ __forceinline__ float h2f(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}

template <int FMT>
__global__ __launch_bounds__(256) void block_mean_kernel(KVView kv, int B, int nb,
                                                         float *__restrict__ kmean) {
  const int b = blockIdx.x, g = blockIdx.y;
  const int D = kv.D;
  const int j0 = b * B, j1 = min(j0 + B, kv.N);
  const float n = (float)(j1 - j0);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float sum = 0.f;
    for (int j = j0; j < j1; ++j) {
      const size_t tok = (size_t)g * kv.N + j;
      float x;
      if (FMT == 0) {
        x = h2f(kv.K[tok * D + d]);
      } else {
        const uint32_t w = kv.Kc[tok * (D / 8) + d / 8];
        const float c = (float)((w >> (4 * (d % 8))) & 0xFu);
        const uint32_t sb = kv.Ksb[tok * (D / 32) + d / 32];
        x = __builtin_fmaf(h2f((uint16_t)(sb & 0xffffu)), c, h2f((uint16_t)(sb >> 16)));
      }
      sum += x;
    }
    kmean[((size_t)g * nb + b) * D + d] = __fdiv_rn(sum, n);
  }
}

__global__ __launch_bounds__(256) void block_score_kernel(const uint16_t *__restrict__ Q,
                                                          HeadMap hm,
                                                          const float *__restrict__ kmean,
                                                          int nb, int D,
                                                          float *__restrict__ score) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x * 4 + wave, g = blockIdx.y;
  if (b >= nb) return;
  const float *km = kmean + ((size_t)g * nb + b) * D;
  float acc = 0.f;
  for (int h = 0; h < hm.H_q; ++h) {
    if (hm.m[h] != g) continue;
    float dot = 0.f;
    for (int d = lane; d < D; d += 64) dot = __builtin_fmaf(h2f(Q[(size_t)h * D + d]), km[d], dot);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) dot += __shfl_xor(dot, o);
    acc += dot;
  }
  if (lane == 0) score[(size_t)g * nb + b] = acc;
}

// (score, index) ordering: a ranks before b.
__device__ __forceinline__ bool ranks_before(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

constexpr int kMaxTop = 1024;

__global__ __launch_bounds__(256) void block_topk_kernel(const float *__restrict__ score,
                                                         int nb, int K_top,
                                                         int32_t *__restrict__ blocks) {
  __shared__ int picked[kMaxTop];
  __shared__ float red_s[4];
  __shared__ int red_i[4];
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *sc = score + (size_t)g * nb;
  const int n_sel = min(K_top, nb);
  float last_s = INFINITY;
  int last_i = -1;
  int found = 0;
  for (int k = 0; k < n_sel; ++k) {
    float bs = -INFINITY;
    int bi = 0x7fffffff;
    for (int b = tid; b < nb; b += 256) {
      const float s = sc[b];
      // candidates rank strictly after the previous pick
      if (ranks_before(last_s, last_i, s, b) && ranks_before(s, b, bs, bi)) {
        bs = s;
        bi = b;
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float os = __shfl_xor(bs, o);
      const int oi = __shfl_xor(bi, o);
      if (ranks_before(os, oi, bs, bi)) {
        bs = os;
        bi = oi;
      }
    }
    if (lane == 0) {
      red_s[wave] = bs;
      red_i[wave] = bi;
    }
    __syncthreads();
    bs = red_s[0];
    bi = red_i[0];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (ranks_before(red_s[w], red_i[w], bs, bi)) {
        bs = red_s[w];
        bi = red_i[w];
      }
    __syncthreads();
    if (bi == 0x7fffffff) break;  // nothing left (only with non-finite scores)
    if (tid == 0) picked[k] = bi;
    last_s = bs;
    last_i = bi;
    found = k + 1;
  }
  __syncthreads();
  // ascending order: the rank of a pick among distinct picks is its output slot
  int32_t *out = blocks + (size_t)g * K_top;
  for (int k = tid; k < found; k += 256) {
    const int v = picked[k];
    int rank = 0;
    for (int j = 0; j < found; ++j) rank += picked[j] < v;
    out[rank] = v;
  }
  for (int k = found + tid; k < K_top; k += 256) out[k] = -1;
}

}  // namespace

hipError_t launch_block_mean(const KVView &kv, int B, float *kmean, hipStream_t s) {
  const int nb = (kv.N + B - 1) / B;
  dim3 grid(nb, kv.H);
  const int threads = kv.D < 256 ? kv.D : 256;
  if (kv.fmt == 0)
    hipLaunchKernelGGL(block_mean_kernel<0>, grid, dim3(threads), 0, s, kv, B, nb, kmean);
  else
    hipLaunchKernelGGL(block_mean_kernel<1>, grid, dim3(threads), 0, s, kv, B, nb, kmean);
  return hipGetLastError();
}

hipError_t launch_block_score(const uint16_t *Q, const HeadMap &hm, const float *kmean,
                              int H_kv, int nb, int D, float *score, hipStream_t s) {
  dim3 grid((nb + 3) / 4, H_kv);
  hipLaunchKernelGGL(block_score_kernel, grid, dim3(256), 0, s, Q, hm, kmean, nb, D, score);
  return hipGetLastError();
}

hipError_t launch_block_topk(const float *score, int H_kv, int nb, int K_top, int32_t *blocks,
                             hipStream_t s) {
  if (K_top > kMaxTop || K_top < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_topk_kernel, dim3(H_kv), dim3(256), 0, s, score, nb, K_top, blocks);
  return hipGetLastError();
}

}  // namespace pion
