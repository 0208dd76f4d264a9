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

#include <stddef.h>

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

// Row group hg: its kv-head, row count and q-heads (row r: byte r of heads), from two
// scalar loads. The row group of workgroup row y is y / M (y itself for one query index,
// the latency-bound case, which then skips the division).
struct Group {
  int g, cnt;
  uint64_t heads;
  __device__ __forceinline__ int head(int r) const { return (int)((heads >> (8 * r)) & 0xffu); }
};
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
  const uint32_t sp = p.spans[z];  // prefix segments and spans, counted by the host
  b.pre_splits = (int)(sp & 0xffffu);
  b.n_seg = b.pre_splits + p.suf_splits;
  b.S_total = (int)(sp >> 16);
  b.Q = (const char *)p.Q + z * p.q_stride * p.esz;
  b.out = p.out + z * p.out_stride;
  float *const lse_z = p.lse + z * p.lse_stride;  // (no branch: read with the rest)
  b.lse = p.lse ? lse_z : nullptr;
  b.part_acc = p.part_acc + z * p.part_stride;
  b.part_m = p.part_m + z * p.ml_stride;
  b.part_l = p.part_l + z * p.ml_stride;
  b.counter = p.counters + (size_t)z * p.y_groups + y;
  return b;
}

// At entry: the group of workgroup row y (its index in hg) and the problem's pointers.
// Left to itself the compiler loads each kernel argument just before its use, behind the
// branches between them, and a scalar load can only be waited for together with every
// other outstanding one: a chain of round trips to L2 before the first K/V load. Here one
// batch of loads first brings every argument line the entry reads into the scalar
// cache; the compiler's loads, all made before the first branch, then hit that cache.
// The group record is read for hg = y, the group when M = 1 (the latency-bound case;
// y < kMaxHeads then), and read again after the division otherwise.
__device__ __forceinline__ Group entry_group(const PartialParams &p, int z, int y, int &hg,
                                             Prob &b) {
  const int M = p.M;
  const int hy = min(y, kMaxHeads - 1);
  {
    // One round of scalar loads that brings every kernel-argument cache line the entry
    // reads into the scalar cache: the header (its first 256 bytes) and this
    // workgroup's entries of the per-problem and per-group tables. The compiler's own
    // loads below then hit that cache instead of each waiting on L2. p is the kernel's
    // only argument, at offset 0 of the argument segment.
    const char __attribute__((address_space(4))) *ka =
        (const char __attribute__((address_space(4))) *)__builtin_amdgcn_kernarg_segment_ptr();
    // (byte offsets of the table entries, read into scalar registers)
    const auto off = [](size_t o) { return __builtin_amdgcn_readfirstlane((int)o); };
    const int o_sp = off(offsetof(PartialParams, spans) + 4 * (size_t)z);
    const int o_n = off(offsetof(PartialParams, N) + 4 * (size_t)z);
    const int o_kv = off(offsetof(PartialParams, kv_base) + 8 * (size_t)z);
    const int o_gc = off(offsetof(PartialParams, rg) + offsetof(RowGroups, gc) + 4 * (size_t)hy);
    const int o_hw = off(offsetof(PartialParams, rg) + offsetof(RowGroups, heads) + 8 * (size_t)hy);
    uint32_t t[9];
    __asm__ volatile(
        "s_load_dword %0, %9, 0x0\n\t"
        "s_load_dword %1, %9, 0x40\n\t"
        "s_load_dword %2, %9, 0x80\n\t"
        "s_load_dword %3, %9, 0xc0\n\t"
        "s_load_dword %4, %9, %10\n\t"
        "s_load_dword %5, %9, %11\n\t"
        "s_load_dword %6, %9, %12\n\t"
        "s_load_dword %7, %9, %13\n\t"
        "s_load_dword %8, %9, %14\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(t[0]), "=&s"(t[1]), "=&s"(t[2]), "=&s"(t[3]), "=&s"(t[4]), "=&s"(t[5]),
          "=&s"(t[6]), "=&s"(t[7]), "=&s"(t[8])
        : "s"(ka), "s"(o_sp), "s"(o_n), "s"(o_kv), "s"(o_gc), "s"(o_hw)
        : "memory");
  }
  uint32_t gc = p.rg.gc[hy];
  uint64_t hw = p.rg.heads[hy];
  b = get_prob(p, z, y);
  __asm__ volatile("" ::"s"(M), "s"(gc), "s"(hw), "s"(b.N), "s"(b.S_total), "s"(b.n_seg),
                   "s"(b.Q), "s"(b.out), "s"(b.lse), "s"(b.part_acc), "s"(b.part_m),
                   "s"(b.part_l), "s"(b.counter), "s"(p.kv_base[z]), "s"(p.x_begin),
                   "s"(p.pre_chunk), "s"(p.seg_per_span), "s"(p.fmt), "s"(p.H_kv), "s"(p.esz),
                   "s"(p.blocks), "s"(p.gidx), "s"(p.qscale), "s"(p.S_suf), "s"(p.suf_chunk));
  hg = y;
  if (M != 1) {
    hg = y / M;
    gc = p.rg.gc[hg];
    hw = p.rg.heads[hg];
  }
  Group gr;
  gr.g = (int)(gc & 0xffu);
  gr.cnt = (int)(gc >> 8);
  gr.heads = hw;
  return gr;
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

// Merge the S_total partials of the rows of this workgroup into out / lse, in the one
// workgroup of the row group that took the last ticket. A pass covers np = min(NT,
// cnt * D/4) (row r, dim quad dq) pairs; each pair gets P adjacent lanes of one wave (P
// a power of two, at most 64, P * np <= NT), lane ph taking spans ph, ph + P, ... and
// issuing the loads of CH of them before consuming any, so every row's partials are in
// flight together. The P lanes of a pair then combine their (m, l, acc) by lane
// exchanges, log2 P steps of the same LSE rule (no LDS, no barrier).
__device__ __forceinline__ float xor_lane(float v, int s) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ s) & 63) * 4, __builtin_bit_cast(int, v)));
}
template <int D, int NT>
__device__ __forceinline__ void merge_rows(const PartialParams &p, const Prob &b,
                                           const PartRsrc &pr, const Group &gr, int qi) {
  constexpr int DQ = D / 4, CH = 16;
  const int tid = threadIdx.x;
  const int RT = gr.cnt * DQ;
  for (int pass0 = 0; pass0 < RT; pass0 += NT) {
    const int np = min(NT, RT - pass0);
    int P = 1;  // workgroup-uniform
    while (2 * P * np <= NT && 2 * P <= 64) P *= 2;
    const int ph = tid & (P - 1), pi = tid / P;
    const bool active = pi < np;
    const int pair = pass0 + (active ? pi : 0);
    const int r = pair / DQ, dq = pair - r * DQ;
    const int h = gr.head(r);
    float m = kNegBig, l = 0.f;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      for (int c0 = ph; c0 < b.S_total; c0 += P * CH) {
        float mc[CH], lc[CH];
        f32x4 ac[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const int c = c0 + k * P;
          mc[k] = -INFINITY;  // past the last span: weight 0
          lc[k] = 0.f;
          ac[k] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (c < b.S_total) {  // (no request at all for the slots past it)
            mc[k] = load_m(pr, h, c);
            lc[k] = load_l(pr, h, c);
            ac[k] = load_part(pr, h, c, dq);
          }
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
    // every lane's m is finite (at least kNegBig), so the weights below are too
    for (int s = 1; s < P; s <<= 1) {
      const float m2 = xor_lane(m, s), l2 = xor_lane(l, s);
      const f32x4 a2 = {xor_lane(a.x, s), xor_lane(a.y, s), xor_lane(a.z, s), xor_lane(a.w, s)};
      const float mx = fmaxf(m, m2);
      const float f1 = fast_exp2(m - mx), f2 = fast_exp2(m2 - mx);
      l = __builtin_fmaf(l, f1, l2 * f2);
      a = a * f1 + a2 * f2;
      m = mx;
    }
    if (active && ph == 0) {  // a row with no key at all (an empty token list): out 0, lse -inf
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
                                                 const PartRsrc &pr, const Group &gr, int qi,
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
  merge_rows<D, NT>(p, b, pr, gr, qi);
  if (threadIdx.x == 0)
    __hip_atomic_store(b.counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace
}  // namespace pion
