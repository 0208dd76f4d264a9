// Batched-Q attention over a resident fp16 prefix and a causal fp16 suffix, on fp16
// MFMA (the QUERY_FUSED wire form of the ATTEND.* page and the batched-Q QUERY of the
// "Shared KV Cache Serving" page, Wire-protocol details). Row i of q-head h attends the
// N prefix keys of kv-head g = head_map[h] and the suffix keys j <= S_suf - M + i.
//
// Per workgroup: 128 query rows of one q-head (4 waves x 32 rows) against one split of
// the key index space [0, N + S_suf) (prefix then suffix), in tiles of 64 keys.
//   S^T = K Q^T   on v_mfma_f32_32x32x16_f16: A = a 32-key x 16-dim slice of the K tile
//                 (LDS, row-major), B = Q^T (registers, loaded once); the result lane l
//                 holds 16 keys x 1 query (query l % 32).
//   online softmax in fp32 (log2 units, scale folded into the exponent; the row sum
//                 uses the fp32 weights, the PV product their fp16 roundings); a lane's p
//                 values are already the B operand of the next product: result element
//                 (i, j) of the S^T block is key 8i + 4(l/32) + j, and a 16-key k-step of
//                 the PV product takes elements i = 2s, 2s+1 as its eight k slots.
//   O^T += V^T P^T  A = V^T (LDS, stored transposed at staging so each lane reads two
//                 runs of 4 keys), with the k slots in that same key order.
// K and V of the next tile are fetched into registers while the current tile is
// consumed, then written to LDS (K as rows padded by 16 bytes, V transposed with rows
// padded by 8 bytes; both conflict-free for the operand reads).
// Splits of the key range run in different workgroups; the last one of a row block
// merges their (acc, m, l) partials with the LSE rule, as in the split-KV decode kernel.
#include "kernels.h"

namespace pion {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr float kNegBig = -1.0e30f;
constexpr int BQ = 128;   // query rows per workgroup
constexpr int BK = 64;    // keys per tile
constexpr int kMaxPrefillSplits = 16;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
struct PrefillSmem {
  static constexpr int KST = D + 8;   // K tile row stride (halves)
  static constexpr int VST = BK + 4;  // V^T row stride (halves)
  _Float16 k[BK * KST];
  _Float16 vt[D * VST];
  int last;
};

template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
  constexpr int NDB = D / 32;                 // 32-dim blocks of O^T
  constexpr int NDS = D / 16;                 // 16-dim k-steps of S^T
  constexpr int KST = PrefillSmem<D>::KST, VST = PrefillSmem<D>::VST;
  constexpr int CH = D / 8;                   // 16-byte chunks per key row
  constexpr int KITEMS = BK * CH / 256;       // K chunks per thread per tile
  constexpr int VITEMS = (BK / 2) * CH / 256; // V (key-pair, chunk) items per thread
  __shared__ PrefillSmem<D> sm;

  const int tile = blockIdx.x, split = blockIdx.y;
  const int h = tile / p.n_iblk, i0 = (tile - h * p.n_iblk) * BQ;
  const int g = p.hm.m[h];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int qi = i0 + wave * 32 + col;
  const int qi_c = min(qi, p.M - 1);
  const int total = p.N + p.S_suf;
  const int k_begin = split * p.split_keys;
  const int k_end = min(k_begin + p.split_keys, total);
  const int i_last = min(i0 + BQ - 1, p.M - 1);
  const int lim_wg = p.S_suf > 0 ? p.N + p.S_suf - p.M + i_last + 1 : p.N;
  const int k_stop = min(k_end, lim_wg);
  const int lim_row = p.S_suf > 0 ? p.N + p.S_suf - p.M + qi_c + 1 : p.N;
  const int row_end = min(k_end, lim_row);

  const uint16_t *Kp = p.K + (size_t)g * p.N * D, *Vp = p.V + (size_t)g * p.N * D;
  const uint16_t *Ksp = p.Ksuf ? p.Ksuf + (size_t)g * p.S_suf * D : nullptr;
  const uint16_t *Vsp = p.Vsuf ? p.Vsuf + (size_t)g * p.S_suf * D : nullptr;

  half8 qb[NDS];
  {
    const uint16_t *qrow = p.Q + ((size_t)h * p.M + qi_c) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qb[ds] = *(const half8 *)(qrow + 16 * ds + 8 * hl);
  }
  f16v o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = kNegBig, l_run = 0.f;

  uint4 kreg[KITEMS], vreg[VITEMS][2];
  auto row_ptr = [&](const uint16_t *pre, const uint16_t *suf, int k) -> const uint16_t * {
    return k < p.N ? pre + (size_t)k * D : suf + (size_t)(k - p.N) * D;
  };
  auto gload = [&](int t0) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int item = tid + 256 * it, key = item / CH, ch = item - key * CH;
      const int k = t0 + key;
      kreg[it] = k < total ? *(const uint4 *)(row_ptr(Kp, Ksp, k) + ch * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int item = tid + 256 * it, kp = item & 31, ch = item >> 5;
      const int k = t0 + 2 * kp;
      vreg[it][0] = k < total ? *(const uint4 *)(row_ptr(Vp, Vsp, k) + ch * 8) : make_uint4(0, 0, 0, 0);
      vreg[it][1] = k + 1 < total ? *(const uint4 *)(row_ptr(Vp, Vsp, k + 1) + ch * 8)
                                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int item = tid + 256 * it, key = item / CH, ch = item - key * CH;
      *(uint4 *)&sm.k[key * KST + ch * 8] = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int item = tid + 256 * it, kp = item & 31, ch = item >> 5;
      const uint32_t a[4] = {vreg[it][0].x, vreg[it][0].y, vreg[it][0].z, vreg[it][0].w};
      const uint32_t b[4] = {vreg[it][1].x, vreg[it][1].y, vreg[it][1].z, vreg[it][1].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t lo = (a[c] & 0xffffu) | (b[c] << 16);          // dim 2c of both keys
        const uint32_t hi = (a[c] >> 16) | (b[c] & 0xffff0000u);     // dim 2c + 1
        *(uint32_t *)&sm.vt[(ch * 8 + 2 * c) * VST + 2 * kp] = lo;
        *(uint32_t *)&sm.vt[(ch * 8 + 2 * c + 1) * VST + 2 * kp] = hi;
      }
    }
  };

  int t0 = k_begin;
  if (t0 < k_stop) gload(t0);
  for (; t0 < k_stop; t0 += BK) {
    __syncthreads();  // the previous tile's operand reads are done
    swrite();
    __syncthreads();
    if (t0 + BK < k_stop) gload(t0 + BK);

    f16v s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const half8 a = *(const half8 *)&sm.k[(32 * kb + col) * KST + 16 * ds + 8 * hl];
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qb[ds], s[kb], 0, 0, 0);
      }
    }
    float mt = kNegBig;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = t0 + 32 * kb + 8 * i + 4 * hl + j;
          const float v = key < row_end ? s[kb][4 * i + j] * p.qscale : -INFINITY;
          s[kb][4 * i + j] = v;
          mt = fmaxf(mt, v);
        }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      half8 pb[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pf = fast_exp2(s[kb][e] - m_new);  // masked: 0
        l_run += pf;                                    // row sum from the fp32 weights
        pb[e >> 3][e & 7] = (_Float16)pf;
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const _Float16 *vrow = &sm.vt[(32 * db + col) * VST + 32 * kb + 16 * s2 + 4 * hl];
          const half4 lo = *(const half4 *)vrow;
          const half4 hi = *(const half4 *)(vrow + 8);
          const half8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[s2], o[db], 0, 0, 0);
        }
      }
    }
  }
  l_run += __shfl_xor(l_run, 32);

  const bool row_ok = qi < p.M;
  const size_t row = (size_t)h * p.M + qi_c;
  if (p.n_splits == 1) {
    if (row_ok) {
      const float inv = 1.f / l_run;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float4 v = make_float4(o[db][4 * i] * inv, o[db][4 * i + 1] * inv,
                                 o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
          *(float4 *)(p.out + row * D + 32 * db + 8 * i + 4 * hl) = v;
        }
      if (hl == 0 && p.lse) p.lse[row] = (m_run + __log2f(l_run)) * 0.69314718055994530942f;
    }
    return;
  }

  // split partial: acc unnormalized against m_run, in the split-KV layout
  if (row_ok) {
    const size_t o_idx = row * p.n_splits + split;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st_agent(p.part_acc + o_idx * D + 32 * db + 8 * i + 4 * hl + j, o[db][4 * i + j]);
    if (hl == 0) {
      st_agent(p.part_m + o_idx, l_run > 0.f ? m_run : -INFINITY);
      st_agent(p.part_l + o_idx, l_run);
    }
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int t = __hip_atomic_fetch_add(p.counters + tile, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    sm.last = (t == p.n_splits - 1);
  }
  __syncthreads();
  if (!sm.last) return;
  // merge: thread t handles dim t % D of rows t / D, t / D + 256 / D, ...
  constexpr int RPP = 256 / D;  // rows per pass
  const int d = tid % D;
  for (int r = tid / D; r < BQ; r += RPP) {
    const int i = i0 + r;
    if (i >= p.M) break;
    const size_t rw = (size_t)h * p.M + i;
    float mc[kMaxPrefillSplits], lc[kMaxPrefillSplits], ac[kMaxPrefillSplits];
    float M = kNegBig;
#pragma unroll
    for (int c = 0; c < kMaxPrefillSplits; ++c) {
      const bool in = c < p.n_splits;
      mc[c] = in ? ld_agent(p.part_m + rw * p.n_splits + c) : -INFINITY;
      lc[c] = in ? ld_agent(p.part_l + rw * p.n_splits + c) : 0.f;
      ac[c] = in ? ld_agent(p.part_acc + (rw * p.n_splits + c) * D + d) : 0.f;
      M = fmaxf(M, mc[c]);
    }
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxPrefillSplits; ++c) {
      const float w = fast_exp2(mc[c] - M);
      L = __builtin_fmaf(w, lc[c], L);
      A = __builtin_fmaf(w, ac[c], A);
    }
    p.out[rw * D + d] = A / L;
    if (d == 0 && p.lse) p.lse[rw] = (M + __log2f(L)) * 0.69314718055994530942f;
  }
  if (tid == 0) __hip_atomic_store(p.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, hipStream_t s) {
  if (p.n_splits < 1 || p.n_splits > kMaxPrefillSplits || p.split_keys % BK) return hipErrorInvalidValue;
  dim3 grid(p.H_q * p.n_iblk, p.n_splits);
  switch (p.D) {
    case 64: hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(256), 0, s, p); break;
    case 256: hipLaunchKernelGGL(prefill_kernel<256>, grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pion
