// Block-mean top-K selection for the sparse-auto query ("Shared KV Cache Serving",
// Stage 2 sparse-mask paragraph: block-mean top-K from the resident K, block size B,
// K_top blocks; ATTEND.* page, QUERY_SPARSE_AUTO rows: K_mean cached per slot).
//
//   block_mean : K_mean[g, b, d] = (sum of K[g, j, d] over the tokens j of block b) / n_b,
//                summed in fp32; threads read 16-byte chunks of the key rows (coalesced
//                rows), partial sums of row slots added through LDS.
//   block_select: score[g, b] = sum over q-heads h with head_map[h] == g of q_h . K_mean[g, b],
//                computed as (sum of those q_h) . K_mean[g, b] (equal in exact arithmetic),
//                then per kv-head the min(K_top, nb) best blocks by (score desc, index asc),
//                written in ascending index order, -1 past nb. One launch: the
//                workgroups score, the last one of each kv-head selects.
// The arithmetic of a block depends only on its own data, so identical blocks get
// identical scores and the lower index wins the tie.
#include "sparse.h"

namespace pion {
namespace {

__device__ __forceinline__ float h2f(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}

// Block means, workgroup (block b, kv-head g): thread t owns 16-byte chunk c = t % TPR of
// the key rows (E dims: 8 fp16, 4 fp32, or one 32-dim mlx4g32 group, dequantized as
// s * code + b) and rows j0 + t / TPR + k RP of the block (RP = 256 / TPR row slots);
// threads past the row's chunks idle. Each thread sums its rows in fp32 in row order, the
// row slots' sums are added in slot order through LDS, and the total is divided by the
// block's row count. The order depends only on the block's own rows.
template <int FMT>
__global__ __launch_bounds__(256) void block_mean_kernel(KVView kv, int B, int nb, int tpr,
                                                         float *__restrict__ kmean) {
  constexpr int E = FMT == 0 ? 8 : FMT == 2 ? 4 : 32;  // dims per chunk
  __shared__ float part[256 * E];
  const int b = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int D = kv.D, CH = D / E, RP = 256 / tpr;
  const int j0 = b * B, j1 = min(j0 + B, kv.N);
  const int c = t % tpr;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (c < CH) {
    const size_t row0 = (size_t)g * kv.N;
#pragma unroll 4
    for (int j = j0 + t / tpr; j < j1; j += RP) {
      if constexpr (FMT == 0) {
        const uint4 w = *((const uint4 *)((const uint16_t *)kv.K + (row0 + j) * D) + c);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += h2f((uint16_t)(u[e / 2] >> (16 * (e % 2))));
      } else if constexpr (FMT == 2) {
        const float4 w = *((const float4 *)((const float *)kv.K + (row0 + j) * D) + c);
        acc[0] += w.x;
        acc[1] += w.y;
        acc[2] += w.z;
        acc[3] += w.w;
      } else {
        const uint4 w = *((const uint4 *)(kv.Kc + (row0 + j) * (D / 8)) + c);
        const uint32_t sb = kv.Ksb[(row0 + j) * (D / 32) + c];
        const float sc = h2f((uint16_t)(sb & 0xffffu)), bi = h2f((uint16_t)(sb >> 16));
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 32; ++e)
          acc[e] += __builtin_fmaf(sc, (float)((u[e / 8] >> (4 * (e % 8))) & 0xFu), bi);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) part[t * E + e] = acc[e];
  __syncthreads();
  const float n = (float)(j1 - j0);
  for (int d = t; d < D; d += 256) {
    const int cd = d / E, e = d - cd * E;
    float sum = 0.f;
    for (int r = 0; r < RP; ++r) sum += part[(r * tpr + cd) * E + e];
    kmean[((size_t)g * nb + b) * D + d] = __fdiv_rn(sum, n);
  }
}

// Lane moves without LDS: DPP within rows of 16 lanes, swaps across rows (gfx950).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}
__device__ __forceinline__ float add_swapped(float v, bool by32) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = by32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                      : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
// Sum over each aligned group of W lanes (W = 8 .. 64), in every lane of the group:
// quad sums and row half-mirror give the 8-lane sum, row mirror the 16-lane sum; the
// row swaps pair rows 16 and 32 apart. Every group adds in the same order, so a group's result depends
// only on its own values.
template <int W>
__device__ __forceinline__ float lane_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  if constexpr (W >= 16) v += dpp_f<0x140>(v);
  if constexpr (W >= 32) v = add_swapped(v, false);
  if constexpr (W >= 64) v = add_swapped(v, true);
  return v;
}

// Order-preserving key of a score: a larger score gets a larger key, -0 counts as +0,
// and NaN gets 0, below every other score.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) return 0u;
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelBlocks = 64;  // blocks scored per workgroup
constexpr int kSelE = 16;       // keys per thread per chunk of the selection
constexpr int kSelCand = 512;   // candidate merge: at most this many candidates

// Score phase, one workgroup per kSelBlocks blocks of one kv-head g: each block's score
// is qsum . K_mean[g, b] with qsum the fp32 sum of the q-heads mapped to g (in head
// order), the dot summed by a fixed lane tree so that a score depends only on the
// block's own data. Scores are written as keys (agent-coherent stores); the last
// workgroup of g (ticket on counters[g]) selects:
//   candidate merge (K_top <= 64 and few candidates): each workgroup also ranks its own
//   blocks by (key desc, index asc) and stores its best min(K, blocks) as 64-bit
//   composites key << 32 | ~index (larger is better); the last workgroup ranks every
//   candidate among all of them (the global best K are among the candidates) and
//   writes the chosen blocks in ascending index order;
//   otherwise radix select, 8 bits a pass from the top, finds the key T of the K-th
//   best block (K = min(K_top, nb)) and how many blocks with key T are still needed;
//   then one scan in block order places each chosen block at
//     (blocks with key > T before it) + min(blocks with key T before it, need),
//   which is ascending index order with ties going to the lower index.
template <int D, bool Q32>
__global__ __launch_bounds__(256) void block_select_kernel(const void *__restrict__ Q,
                                                           HeadMap hm,
                                                           const float *__restrict__ kmean,
                                                           int nb, int K_top, uint32_t *keys,
                                                           uint64_t *cand, int *counters,
                                                           int32_t *__restrict__ blocks) {
  // lanes per block row: the largest power of two (at most 64) that divides D / 4, so
  // that each lane holds F whole float4 of the row
  constexpr int LPB = (D / 4) % 64 == 0 ? 64 : (D / 4) % 32 == 0 ? 32 : (D / 4) % 16 == 0 ? 16 : 8;
  constexpr int F = D / (4 * LPB);              // float4 per lane
  constexpr int RPL = 64 / LPB;                 // block rows per wave load
  constexpr int NL = kSelBlocks / 4 / RPL;      // wave loads
  __shared__ float qsum[D];
  __shared__ int hist[256];
  __shared__ int wsum[4][2];
  __shared__ uint32_t st_prefix;
  __shared__ int st_need, st_last;
  __shared__ uint32_t wkey[kSelBlocks];
  __shared__ int wrank[4][kSelBlocks];
  __shared__ uint64_t cx[kSelCand];
  __shared__ uint32_t sel[kSelBlocks];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.y;
  uint32_t *kg = keys + (size_t)g * nb;
  const int K = min(K_top, nb);
  const int KC = min(K_top, kSelBlocks);  // candidate slots per workgroup
  const bool fast = K_top <= kSelBlocks && (int)gridDim.x * KC <= kSelCand;
  const int w0 = blockIdx.x * kSelBlocks, nv = min(kSelBlocks, nb - w0);

  for (int d = tid; d < D; d += 256) {
    float a = 0.f;
#pragma unroll 8
    for (int h = 0; h < hm.H_q; ++h) {
      const float v = Q32 ? ((const float *)Q)[(size_t)h * D + d]
                          : h2f(((const uint16_t *)Q)[(size_t)h * D + d]);
      if (hm.m[h] == g) a += v;
    }
    qsum[d] = a;
  }
  __syncthreads();

  {
    const int sub = lane % LPB, rl = lane / LPB;
    float4 qv[F];
#pragma unroll
    for (int f = 0; f < F; ++f) qv[f] = *(const float4 *)&qsum[4 * (sub + f * LPB)];
    const int b0 = blockIdx.x * kSelBlocks + wave * (kSelBlocks / 4) + rl;
    float4 kv[NL][F];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int b = b0 + i * RPL;
#pragma unroll
      for (int f = 0; f < F; ++f)
        kv[i][f] = b < nb ? *(const float4 *)(kmean + ((size_t)g * nb + b) * D + 4 * (sub + f * LPB))
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float s = 0.f;
#pragma unroll
      for (int f = 0; f < F; ++f) {
        s = __builtin_fmaf(qv[f].x, kv[i][f].x, s);
        s = __builtin_fmaf(qv[f].y, kv[i][f].y, s);
        s = __builtin_fmaf(qv[f].z, kv[i][f].z, s);
        s = __builtin_fmaf(qv[f].w, kv[i][f].w, s);
      }
      s = lane_sum<LPB>(s);
      const int b = b0 + i * RPL;
      if (sub == 0 && b < nb) {
        __hip_atomic_store(kg + b, score_key(s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wkey[b - w0] = score_key(s);
      }
    }
  }
  if (fast) {
    // local rank of block i among this workgroup's blocks, in four quarters
    __syncthreads();
    const int i = tid & (kSelBlocks - 1), q = tid >> 6;
    if (i < nv) {
      const uint32_t ki = wkey[i];
      int cnt = 0;
      for (int j = q * 16; j < min(nv, q * 16 + 16); ++j) {
        const uint32_t kj = wkey[j];
        cnt += (kj > ki) || (kj == ki && j < i);
      }
      wrank[q][i] = cnt;
    }
    __syncthreads();
    if (tid < nv) {
      const int rank = wrank[0][tid] + wrank[1][tid] + wrank[2][tid] + wrank[3][tid];
      if (rank < min(K, nv))
        __hip_atomic_store(cand + ((size_t)g * gridDim.x + blockIdx.x) * KC + rank,
                           ((uint64_t)wkey[tid] << 32) | (uint32_t)~(uint32_t)(w0 + tid),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // this wave's key stores have completed before the barrier and the ticket
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    st_last = __hip_atomic_fetch_add(counters + g, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
  __syncthreads();
  if (!st_last) return;

  int32_t *out = blocks + (size_t)g * K_top;
  if (fast) {
    const int C = gridDim.x * KC;
    for (int x = tid; x < C; x += 256) {
      const int w = x / KC, r = x - w * KC;
      const int kc = min(K, min(kSelBlocks, nb - w * kSelBlocks));  // valid slots of w
      cx[x] = r < kc ? __hip_atomic_load(cand + (size_t)g * C + x, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : 0ull;  // below every valid composite
    }
    __syncthreads();
    for (int x = tid; x < C; x += 256) {
      const uint64_t X = cx[x];
      if (X == 0ull) continue;
      int rank = 0;
      for (int j = 0; j < C; ++j) rank += cx[j] > X;
      if (rank < K) sel[rank] = ~(uint32_t)X;
    }
    __syncthreads();
    if (tid < K) {
      const uint32_t v = sel[tid];
      int pos = 0;
      for (int j = 0; j < K; ++j) pos += sel[j] < v;
      out[pos] = (int32_t)v;
    }
    for (int k = K + tid; k < K_top; k += 256) out[k] = -1;
    if (tid == 0) __hip_atomic_store(counters + g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  constexpr int CH = 256 * kSelE;
  uint32_t kr[kSelE];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int e = 0; e < kSelE; ++e) {
      const int i = c0 + tid * kSelE + e;
      kr[e] = i < nb ? __hip_atomic_load(kg + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    }
  };
  const bool one = nb <= CH;
  if (one) load_chunk(0);

  uint32_t prefix = 0;
  int need = K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hmask = pass == 0 ? 0u : 0xFFFFFFFFu << (shift + 8);
    hist[tid] = 0;
    __syncthreads();
    for (int c0 = 0; c0 < nb; c0 += CH) {
      if (!one) load_chunk(c0);
#pragma unroll
      for (int e = 0; e < kSelE; ++e) {
        const int i = c0 + tid * kSelE + e;
        if (i < nb && (kr[e] & hmask) == prefix) atomicAdd(&hist[(kr[e] >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // digits in descending order: lane l holds 255 - 4l ... 252 - 4l
      int c[4], loc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[255 - 4 * lane - i];
        loc += c[i];
      }
      int inc = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
      }
      int before = inc - loc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (before < need && need <= before + c[i]) {
          st_prefix = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
          st_need = need - before;
        }
        before += c[i];
      }
    }
    __syncthreads();
    prefix = st_prefix;
    need = st_need;
  }

  const uint32_t T = prefix;
  int gt_run = 0, eq_run = 0;
  for (int c0 = 0; c0 < nb; c0 += CH) {
    if (!one) load_chunk(c0);
    int ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < kSelE; ++e) {
      const int i = c0 + tid * kSelE + e;
      if (i < nb) {
        ngt += kr[e] > T;
        neq += kr[e] == T;
      }
    }
    int igt = ngt, ieq = neq;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int a = __shfl_up(igt, o), b = __shfl_up(ieq, o);
      if (lane >= o) {
        igt += a;
        ieq += b;
      }
    }
    if (lane == 63) {
      wsum[wave][0] = igt;
      wsum[wave][1] = ieq;
    }
    __syncthreads();
    int gb = gt_run + igt - ngt, eb = eq_run + ieq - neq;
    for (int w = 0; w < wave; ++w) {
      gb += wsum[w][0];
      eb += wsum[w][1];
    }
#pragma unroll
    for (int e = 0; e < kSelE; ++e) {
      const int i = c0 + tid * kSelE + e;
      if (i < nb) {
        const bool gt = kr[e] > T, eq = kr[e] == T;
        if (gt || (eq && eb < need)) out[gb + min(eb, need)] = i;
        gb += gt;
        eb += eq;
      }
    }
    gt_run += wsum[0][0] + wsum[1][0] + wsum[2][0] + wsum[3][0];
    eq_run += wsum[0][1] + wsum[1][1] + wsum[2][1] + wsum[3][1];
    __syncthreads();
  }
  for (int k = K + tid; k < K_top; k += 256) out[k] = -1;
  if (tid == 0) __hip_atomic_store(counters + g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_block_mean(const KVView &kv, int B, float *kmean, hipStream_t s) {
  const int nb = (kv.N + B - 1) / B;
  const dim3 grid(nb, kv.H);
  // 16-byte chunks per key row, each handled by one thread of a power-of-two row group
  const int E = kv.fmt == 0 ? 8 : kv.fmt == 2 ? 4 : 32;
  if (B < 1 || kv.D % E) return hipErrorInvalidValue;
  int tpr = 1;
  while (tpr < kv.D / E) tpr <<= 1;
  if (tpr > 256) return hipErrorInvalidValue;
  note_launch("block_mean_kernel<%d>", kv.fmt);
  if (kv.fmt == 0)
    hipLaunchKernelGGL(block_mean_kernel<0>, grid, dim3(256), 0, s, kv, B, nb, tpr, kmean);
  else if (kv.fmt == 2)
    hipLaunchKernelGGL(block_mean_kernel<2>, grid, dim3(256), 0, s, kv, B, nb, tpr, kmean);
  else
    hipLaunchKernelGGL(block_mean_kernel<1>, grid, dim3(256), 0, s, kv, B, nb, tpr, kmean);
  return hipGetLastError();
}

hipError_t launch_block_select(const void *Q, bool q32, const HeadMap &hm, const float *kmean,
                               int H_kv, int nb, int D, int K_top, uint32_t *keys,
                               uint64_t *cand, int *counters, int32_t *blocks, hipStream_t s) {
  if (K_top < 1 || nb < 1 || H_kv < 1) return hipErrorInvalidValue;
  dim3 grid((nb + kSelBlocks - 1) / kSelBlocks, H_kv);
  note_launch("block_select_kernel<%d,%s>", D, q32 ? "true" : "false");
#define PION_SELECT_D(DD)                                                                  \
  case DD:                                                                               \
    if (q32)                                                                             \
      hipLaunchKernelGGL((block_select_kernel<DD, true>), grid, dim3(256), 0, s, Q, hm, kmean, \
                         nb, K_top, keys, cand, counters, blocks);                       \
    else                                                                                 \
      hipLaunchKernelGGL((block_select_kernel<DD, false>), grid, dim3(256), 0, s, Q, hm,     \
                         kmean, nb, K_top, keys, cand, counters, blocks);                \
    break;
  switch (D) {
    PION_SELECT_D(32)
    PION_SELECT_D(64)
    PION_SELECT_D(96)
    PION_SELECT_D(128)
    PION_SELECT_D(160)
    PION_SELECT_D(192)
    PION_SELECT_D(256)
    PION_SELECT_D(512)
    default:
      return hipErrorInvalidValue;
  }
#undef PION_SELECT_D
  return hipGetLastError();
}

}  // namespace pion
