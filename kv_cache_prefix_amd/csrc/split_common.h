// Device helpers shared by the split-over-keys attention kernels (fp16 and mlx4g32
// prefix): span and problem addressing, agent-coherent hand-off of partials between
// workgroups, and the last-arriving workgroup's merge of a row group's partials.
//
// The merge is the LSE rule of the "Shared KV Cache Serving" page (Stage 2 consumer and
// Wire-protocol details): with partials (m_c, l_c, acc_c) in log2 units,
//     m* = max_c m_c,  w_c = 2^(m_c - m*),  out = sum_c w_c acc_c / sum_c w_c l_c,
//     lse = ln 2 * (m* + log2 sum_c w_c l_c).
//
// Cross-XCD visibility without L2 flushes: partials are written and read with the sc1
// cache policy (coherent at agent scope, never held dirty or stale in a per-XCD L2),
// and each wave waits for its partial stores to complete
// (s_waitcnt vmcnt(0)) before the workgroup barrier that precedes its ticket. An
// agent-scope fence here would write back and invalidate the whole L2 of the XCD for
// every workgroup.
#pragma once

#include "kernels.h"

namespace pion {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;  // running-max start: 2^(kNegBig - kNegBig) = 1
constexpr int kMaxSplits = 8192;  // spans of a row (partials per row in the workspace)

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ float h2f(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16- and 4-byte loads of K/V data that is streamed once per query: the non-temporal
// hint keeps it from displacing reused lines in the caches (worth ~14% of cold-HBM
// decode bandwidth).
typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void *p) {
  const nt_u32x4 v = __builtin_nontemporal_load((const nt_u32x4 *)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream4(const uint32_t *p) {
  return __builtin_nontemporal_load(p);
}

// Row-level lane permutation (DPP). Every control used here (quad_perm, row half-mirror,
// row mirror, row rotate) reads in-range lanes only, so bound_ctrl (zero for an
// out-of-range source) never applies; it lets the compiler fold the move into the
// consuming add or max (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// A segment is one contiguous key range: a prefix chunk of pre_chunk tokens (or, with
// `blocks`, one selected block), or a suffix chunk of suf_chunk tokens clipped to the
// causal limit of query index qi. Span x of a problem covers segments
// [x * seg_per_span, (x + 1) * seg_per_span).
struct Span {
  int j0, j1;
  bool suffix;
};

__device__ __forceinline__ Span get_segment(const PartialParams &p, int x, int pre_segs, int N,
                                            int g, int qi) {
  Span s;
  if (x < pre_segs) {
    s.suffix = false;
    if (p.blocks) {
      const int nb = (N + p.B - 1) / p.B;
      const int b = p.blocks[g * p.K_top + x];
      if (b < 0 || b >= nb) {  // device-produced index: never trust it for addressing
        s.j0 = s.j1 = 0;
      } else {
        s.j0 = b * p.B;
        s.j1 = min(s.j0 + p.B, N);
      }
    } else {  // dense chunks of the prefix, or of a caller's token list
      s.j0 = x * p.pre_chunk;
      s.j1 = min(s.j0 + p.pre_chunk, p.gidx ? p.gmax : N);
    }
  } else {
    s.suffix = true;
    const int c = x - pre_segs;
    const int lim = p.S_suf - p.M + qi + 1;  // causal, bottom-right aligned
    s.j0 = c * p.suf_chunk;
    s.j1 = min(min(s.j0 + p.suf_chunk, p.S_suf), lim);
  }
  return s;
}

// Per-problem pointers of this workgroup.
struct Prob {
  int N, pre_splits, n_seg, S_total;  // pre_splits: prefix segments
  const void *Q;
  float *out, *lse, *part_acc, *part_m, *part_l;
  int *counter;
};

__device__ __forceinline__ Prob get_prob(const PartialParams &p, int z, int y) {
  Prob b;
  b.N = p.N[z];
  b.pre_splits = p.blocks ? p.n_sel : ((p.gidx ? p.gmax : b.N) + p.pre_chunk - 1) / p.pre_chunk;
  b.n_seg = b.pre_splits + p.suf_splits;
  b.S_total = (b.n_seg + p.seg_per_span - 1) / p.seg_per_span;
  b.Q = (const char *)p.Q + z * p.q_stride * p.esz;
  b.out = p.out + z * p.out_stride;
  b.lse = p.lse ? p.lse + z * p.lse_stride : nullptr;
  b.part_acc = p.part_acc + z * p.part_stride;
  b.part_m = p.part_m + z * p.ml_stride;
  b.part_l = p.part_l + z * p.ml_stride;
  b.counter = p.counters + (size_t)z * p.y_groups + y;
  return b;
}

// Partials of one (problem, query index): rows are the q-heads h, layout
// [h][S_max][D] (acc) and [h][S_max] (m, l) inside the problem's workspace, at
// qi * H_q rows. Accessed through buffer descriptors with the agent-coherent cache
// policy (sc1), in 16-byte pieces for acc.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kSC1 = 16;  // buffer cache-policy bit sc1: coherent across the agent's XCDs

// Buffer resource over `bytes` bytes at `base` (0x00020000: raw 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Streaming (non-temporal) buffer loads: bytes past the range read zero.
constexpr int kNT = 2;  // buffer cache-policy bit nt
__device__ __forceinline__ uint4 bload_stream16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNT);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload_stream4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kNT);
}

struct PartRsrc {
  __amdgpu_buffer_rsrc_t a, m, l;
  int S_max, D;
};

__device__ __forceinline__ PartRsrc part_rsrc(const PartialParams &p, const Prob &b, int qi) {
  PartRsrc r;
  const size_t row0 = (size_t)qi * p.H_q;
  const uint32_t n = (uint32_t)p.H_q * p.S_max;
  r.a = make_rsrc(b.part_acc + row0 * p.S_max * p.D, n * p.D * 4);
  r.m = make_rsrc(b.part_m + row0 * p.S_max, n * 4);
  r.l = make_rsrc(b.part_l + row0 * p.S_max, n * 4);
  r.S_max = p.S_max;
  r.D = p.D;
  return r;
}

// Store span x's partial of q-head h: acc[4 dq .. 4 dq + 3]; with ml, also m and l.
__device__ __forceinline__ void store_part(const PartRsrc &r, int h, int x, int dq, f32x4 a) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), r.a,
                                         ((h * r.S_max + x) * r.D + 4 * dq) * 4, 0, kSC1);
}
__device__ __forceinline__ void store_ml(const PartRsrc &r, int h, int x, float m, float l) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, m), r.m,
                                        (h * r.S_max + x) * 4, 0, kSC1);
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l), r.l,
                                        (h * r.S_max + x) * 4, 0, kSC1);
}
// Note: a raw_buffer_load_b128 result is bit-cast as a whole vector; bit-casting its
// elements one by one makes this compiler narrow the load to a single dword.
__device__ __forceinline__ f32x4 load_part(const PartRsrc &r, int h, int c, int dq) {
  return __builtin_bit_cast(
      f32x4, __builtin_amdgcn_raw_buffer_load_b128(r.a, ((h * r.S_max + c) * r.D + 4 * dq) * 4, 0,
                                                   kSC1));
}
__device__ __forceinline__ float load_m(const PartRsrc &r, int h, int c) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_raw_buffer_load_b32(r.m, (h * r.S_max + c) * 4, 0, kSC1));
}
__device__ __forceinline__ float load_l(const PartRsrc &r, int h, int c) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_raw_buffer_load_b32(r.l, (h * r.S_max + c) * 4, 0, kSC1));
}

// LDS of the merge: per thread a running (m, l, acc piece); NT threads.
template <int NT>
struct MergeScratch {
  f32x4 a[NT];
  float m[NT], l[NT];
};

// Merge the S_total partials of the rows of this workgroup into out / lse, in the one
// workgroup of the row group that took the last ticket. Thread t takes (row r, dim
// quad dq) = pair t % np of the np = min(NT, cnt * D/4) pairs of a pass, and spans
// c = t / np, + P, ... (P = NT / np phases); it issues the loads of CH spans of its
// row before consuming any, so every row's partials are in flight together. The P
// phase results of a pair merge through LDS.
template <int D, int NT>
__device__ __forceinline__ void merge_rows(const PartialParams &p, const Prob &b,
                                           const PartRsrc &pr, const uint8_t *heads, int cnt,
                                           int qi, MergeScratch<NT> &ms) {
  constexpr int DQ = D / 4, CH = 16;
  const int tid = threadIdx.x;
  const int RT = cnt * DQ;
  for (int pass0 = 0; pass0 < RT; pass0 += NT) {
    const int np = min(NT, RT - pass0);
    const int P = NT / np;
    const int ph = tid / np, pair = pass0 + tid % np;
    const int r = pair / DQ, dq = pair - r * DQ;
    const int h = heads[r];
    float m = kNegBig, l = 0.f;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if (ph < P) {
      for (int c0 = ph; c0 < b.S_total; c0 += P * CH) {
        float mc[CH], lc[CH];
        f32x4 ac[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const int c = c0 + k * P;
          const bool in = c < b.S_total;
          const int cc = in ? c : 0;
          mc[k] = load_m(pr, h, cc);
          lc[k] = load_l(pr, h, cc);
          ac[k] = load_part(pr, h, cc, dq);
          if (!in) mc[k] = -INFINITY;
        }
        float mx = m;
#pragma unroll
        for (int k = 0; k < CH; ++k) mx = fmaxf(mx, mc[k]);
        const float f = fast_exp2(m - mx);
        l *= f;
        a *= f;
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const float w = fast_exp2(mc[k] - mx);  // empty or absent span: m = -inf -> 0
          l = __builtin_fmaf(w, lc[k], l);
          a.x = __builtin_fmaf(w, ac[k].x, a.x);
          a.y = __builtin_fmaf(w, ac[k].y, a.y);
          a.z = __builtin_fmaf(w, ac[k].z, a.z);
          a.w = __builtin_fmaf(w, ac[k].w, a.w);
        }
        m = mx;
      }
    }
    if (P > 1) {
      ms.m[tid] = m;
      ms.l[tid] = l;
      ms.a[tid] = a;
      __syncthreads();
      if (ph == 0) {
        float M = m;
        for (int q = 1; q < P; ++q) M = fmaxf(M, ms.m[q * np + tid]);
        float L = 0.f;
        f32x4 A = {0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < P; ++q) {
          const float f = fast_exp2(ms.m[q * np + tid] - M);
          L = __builtin_fmaf(f, ms.l[q * np + tid], L);
          A += f * ms.a[q * np + tid];
        }
        m = M;
        l = L;
        a = A;
      }
      __syncthreads();
    }
    if (ph == 0) {  // a row with no key at all (an empty token list): out 0, lse -inf
      const size_t row = (size_t)h * p.M + qi;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      *(float4 *)(b.out + row * D + 4 * dq) = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
      if (dq == 0 && b.lse) b.lse[row] = l > 0.f ? (m + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
    }
  }
}

// After this workgroup's partial stores: wait for them, take a ticket on the row
// group's counter, and if this is the last span of the row group, merge and reset the
// counter to zero for the next call. `last` is a workgroup-shared flag.
template <int D, int NT>
__device__ __forceinline__ void ticket_and_merge(const PartialParams &p, const Prob &b,
                                                 const PartRsrc &pr, const uint8_t *heads,
                                                 int cnt, int qi, MergeScratch<NT> &ms,
                                                 int &last) {
  // this wave's partial stores have completed before the barrier and the ticket
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int t = __hip_atomic_fetch_add(b.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = (t == b.S_total - 1);
  }
  __syncthreads();
  if (!last) return;
  merge_rows<D, NT>(p, b, pr, heads, cnt, qi, ms);
  if (threadIdx.x == 0)
    __hip_atomic_store(b.counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace
}  // namespace pion
