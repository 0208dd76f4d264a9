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
//                 uses the fp32 weights, the PV product their fp16 roundings; the
//                 accumulators are rescaled only when a row max grows by more than
//                 2^8, and only boundary tiles are masked); a lane's p
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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Note: the result of __builtin_amdgcn_raw_buffer_load_b128 is reinterpreted as a whole
// vector (bit_cast to f32x4); bit-casting its elements one by one makes this compiler
// narrow the load to a single dword.

constexpr float kNegBig = -1.0e30f;
constexpr int BQ = 128;   // query rows per workgroup
constexpr int BK = 64;    // keys per tile
constexpr int kMaxPrefillSplits = 16;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


template <int D>
struct PrefillSmem {
  static constexpr int KST = D + 8;   // K tile row stride (halves)
  static constexpr int VST = BK + 4;  // V^T row stride (halves)
  union {
    struct {
      alignas(16) _Float16 k[BK * KST];
      alignas(16) _Float16 vt[D * VST];
    };
    struct {                      // split merge: per (row, split) m then weight, and l
      float w[BQ * 16];
      float l[BQ * 16];
      float inv[BQ];
    } mg;
  };
  int last;
};

// A row max may grow by this much (log2 units, a factor 2^8) before the accumulators
// are rescaled: weights up to 2^8 stay exact enough in fp16 and the fp32 sums cannot
// overflow, and after the first tiles a rescale is rare.
constexpr float kRescaleSlack = 8.0f;

// Buffer resource over `bytes` bytes at `base`: loads past the end return zero, which
// masks the tails of the prefix and suffix without branches. 0x00020000 is the raw
// 32-bit data format of the descriptor's last word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
  constexpr int NDB = D / 32;                 // 32-dim blocks of O^T
  constexpr int NDS = D / 16;                 // 16-dim k-steps of S^T
  constexpr int KST = PrefillSmem<D>::KST, VST = PrefillSmem<D>::VST;
  constexpr int CH = D / 8;                   // 16-byte chunks per key row
  constexpr int KITEMS = BK * CH / 256;       // K chunks per thread per tile
  constexpr int VITEMS = (BK / 2) * CH / 256; // V (key-pair, chunk) items per thread
  constexpr uint32_t ROWB = D * 2;            // bytes per key row
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
  // 32-key sub-tiles ending at or below this need no mask for any row of the workgroup
  const int lim_first = p.S_suf > 0 ? p.N + p.S_suf - p.M + i0 + 1 : p.N;
  const int full_end = min(k_end, lim_first);

  const __amdgpu_buffer_rsrc_t rK = make_rsrc(p.K + (size_t)g * p.N * D, (uint32_t)p.N * ROWB);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(p.V + (size_t)g * p.N * D, (uint32_t)p.N * ROWB);
  const bool has_suf = p.S_suf > 0;  // a null suffix gets an empty range
  const __amdgpu_buffer_rsrc_t rKs =
      make_rsrc(has_suf ? p.Ksuf + (size_t)g * p.S_suf * D : p.K, (uint32_t)p.S_suf * ROWB);
  const __amdgpu_buffer_rsrc_t rVs =
      make_rsrc(has_suf ? p.Vsuf + (size_t)g * p.S_suf * D : p.V, (uint32_t)p.S_suf * ROWB);

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
  // Tiles never straddle the prefix / suffix boundary: the split's prefix part
  // [k_begin, pre_end) is tiled from k_begin, its suffix part [suf_beg, k_stop) from
  // suf_beg. Tile j < n_pre is prefix, the rest suffix.
  const int pre_end = min(k_stop, p.N);
  const int suf_beg = max(k_begin, p.N);
  const int n_pre = k_begin < pre_end ? (pre_end - k_begin + BK - 1) / BK : 0;
  const int n_suf = suf_beg < k_stop ? (k_stop - suf_beg + BK - 1) / BK : 0;
  auto gload = [&](int j) {
    const bool suf = j >= n_pre;  // workgroup-uniform
    const int r0 = suf ? suf_beg - p.N + (j - n_pre) * BK : k_begin + j * BK;  // source row
    const __amdgpu_buffer_rsrc_t rk = suf ? rKs : rK, rv = suf ? rVs : rV;
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int item = tid + 256 * it, key = item / CH, ch = item - key * CH;
      kreg[it] = bload(rk, (uint32_t)(r0 + key) * ROWB + ch * 16);
    }
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int item = tid + 256 * it, kp = item & 31, ch = item >> 5;
      vreg[it][0] = bload(rv, (uint32_t)(r0 + 2 * kp) * ROWB + ch * 16);
      vreg[it][1] = bload(rv, (uint32_t)(r0 + 2 * kp + 1) * ROWB + ch * 16);
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

  const int n_tiles = n_pre + n_suf;
  if (n_tiles > 0) gload(0);
  for (int j = 0; j < n_tiles; ++j) {
    const bool suf = j >= n_pre;
    const int t0 = suf ? suf_beg + (j - n_pre) * BK : k_begin + j * BK;  // concatenated index
    const int seg_end = suf ? k_stop : pre_end;   // keys at or past this are not in the tile
    const int lane_end = suf ? row_end : pre_end; // this row's limit inside the tile
    const int clean_end = suf ? min(k_stop, full_end) : pre_end;  // no mask below this
    __syncthreads();  // the previous tile's operand reads are done
    swrite();
    __syncthreads();
    if (j + 1 < n_tiles) gload(j + 1);

    // two 32-key sub-tiles: S^T, softmax, PV
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kt = t0 + 32 * kb;
      if (kt >= seg_end) break;  // workgroup-uniform
      f16v s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const uint4 araw = *(const uint4 *)&sm.k[(32 * kb + col) * KST + 16 * ds + 8 * hl];
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, araw), qb[ds], s,
                                                   0, 0, 0);
      }
      if (kt + 32 > clean_end) {  // boundary sub-tile: mask keys past this row's limit
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (kt + 8 * i + 4 * hl + jj >= lane_end) s[4 * i + jj] = -INFINITY;
      }
      float mt = -INFINITY;  // raw-score max; the scale is positive
#pragma unroll
      for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s[e]);
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * p.qscale;
      const bool grow = mt > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform, rare after the first tiles
        const float m_new = grow ? mt : m_run;
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      }
      half8 pb[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pf = fast_exp2(__builtin_fmaf(s[e], p.qscale, -m_run));  // masked: 0
        l_run += pf;                       // row sum from the fp32 weights
        pb[e >> 3][e & 7] = (_Float16)pf;  // at most 2^8
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const _Float16 *vrow = &sm.vt[(32 * db + col) * VST + 32 * kb + 16 * s2 + 4 * hl];
          const uint2 lo = *(const uint2 *)vrow;
          const uint2 hi = *(const uint2 *)(vrow + 8);
          const uint4 araw = make_uint4(lo.x, lo.y, hi.x, hi.y);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, araw), pb[s2],
                                                         o[db], 0, 0, 0);
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

  // Split partial (acc unnormalized against m_run; m and l in log2 units) in the
  // split-KV layout [row][split][D], written with agent-coherent (sc1) 16-byte stores
  // through a buffer range that covers only this block's valid rows.
  const int S = p.n_splits;
  const int rows_valid = min(BQ, p.M - i0);
  const size_t row0 = (size_t)h * p.M + i0;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(p.part_acc + row0 * S * D, (uint32_t)(rows_valid * S * D * 4));
  const __amdgpu_buffer_rsrc_t rM = make_rsrc(p.part_m + row0 * S, (uint32_t)(rows_valid * S * 4));
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(p.part_l + row0 * S, (uint32_t)(rows_valid * S * 4));
  constexpr int SC1 = 16;  // cache policy: system coherent
  {
    const int r = wave * 32 + col;  // local row; rows past rows_valid fall out of range
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 v = {o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, v), rA,
            (int)(((r * S + split) * D + 32 * db + 8 * i + 4 * hl) * 4), 0, SC1);
      }
    if (hl == 0) {
      const float mv = l_run > 0.f ? m_run : -INFINITY;  // empty split: weight 0
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, mv), rM,
                                            (r * S + split) * 4, 0, SC1);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l_run), rL,
                                            (r * S + split) * 4, 0, SC1);
    }
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int t = __hip_atomic_fetch_add(p.counters + tile, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    sm.last = (t == S - 1);
  }
  __syncthreads();
  if (!sm.last) return;

  // Merge, in three phases with every load of a phase in flight together:
  // (1) m and l of all (row, split) into LDS; (2) per row the weights 2^(m_c - m*) and
  // 1 / sum_c w_c l_c, and lse; (3) out = sum_c w_c acc_c / L in 16-byte pieces.
  for (int x = tid; x < rows_valid * S; x += 256) {
    sm.mg.w[x] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rM, x * 4, 0, SC1));
    sm.mg.l[x] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rL, x * 4, 0, SC1));
  }
  __syncthreads();
  if (tid < rows_valid) {
    float M = -INFINITY;
    for (int c = 0; c < S; ++c) M = fmaxf(M, sm.mg.w[tid * S + c]);
    float L = 0.f;
    for (int c = 0; c < S; ++c) {
      const float w = fast_exp2(sm.mg.w[tid * S + c] - M);  // -inf -> 0
      sm.mg.w[tid * S + c] = w;
      L = __builtin_fmaf(w, sm.mg.l[tid * S + c], L);
    }
    sm.mg.inv[tid] = 1.f / L;
    if (p.lse) p.lse[row0 + tid] = (M + __log2f(L)) * 0.69314718055994530942f;
  }
  __syncthreads();
  constexpr int Q4 = D / 4;                  // 16-byte pieces per row
  constexpr int ITER = BQ * Q4 / 256;        // pieces per thread
  float4 acc[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) acc[it] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = 0; c < S; ++c) {
    f32x4 v[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int q = tid + 256 * it, r = q / Q4, d4 = q - r * Q4;
      v[it] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, ((r * S + c) * D + 4 * d4) * 4, 0, SC1));
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int q = tid + 256 * it, r = q / Q4;
      const float w = r < rows_valid ? sm.mg.w[r * S + c] : 0.f;
      acc[it].x = __builtin_fmaf(w, v[it].x, acc[it].x);
      acc[it].y = __builtin_fmaf(w, v[it].y, acc[it].y);
      acc[it].z = __builtin_fmaf(w, v[it].z, acc[it].z);
      acc[it].w = __builtin_fmaf(w, v[it].w, acc[it].w);
    }
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int q = tid + 256 * it, r = q / Q4, d4 = q - r * Q4;
    if (r < rows_valid) {
      const float inv = sm.mg.inv[r];
      *(float4 *)(p.out + (row0 + r) * D + 4 * d4) =
          make_float4(acc[it].x * inv, acc[it].y * inv, acc[it].z * inv, acc[it].w * inv);
    }
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
