// Split-over-keys attention over fp16 (or fp32) keys and values (VALU path), with the
// split merge done in-kernel. Serves an fp16 or fp32 prefix and the causal suffix of a
// fused query in the same precision (the mlx4g32 prefix has its own kernel; its suffix
// is fp16 and runs here).
//
// What is computed: for each query row (q-head h, query index i) and each key span of
// a workgroup, the online-softmax partial
//     m = max_j s_j,  l = sum_j 2^(s_j - m),  acc = sum_j 2^(s_j - m) v_j,
// with s_j = log2(e)/sqrt(D) * (q . k_j), the scaled logit in log2 units. The spans of
// a row are merged by the LSE rule (split_common.h).
//
// Layout and schedule. A key row of D values is read by LPR consecutive lanes, 8 values
// (16 bytes of fp16, 32 of fp32) each, LPR = D/8 rounded up to a power of two (for D = 96, 160, 192 the lanes past D/8
// hold no dims and load nothing); one wave-wide load covers 64/LPR whole rows, fully
// coalesced. Each group of LPR lanes is a "slot" that runs its own online softmax over
// the keys it sees, so the inner loop needs no cross-lane max: only the LPR-lane
// dot-product sum, done with DPP row operations and lane swaps. K and V of the next tile are loaded before the current tile is
// consumed. At the end the slots of a wave and the 4 waves of the workgroup merge (LDS),
// and the workgroup stores its partial. All q-heads that read the same kv-head share a
// workgroup, so K/V bytes are read once per kv-head (GQA).
//
// The merge runs in the same kernel: every workgroup stores its partial, then takes a
// ticket on its row group's counter; the workgroup that arrives last merges all spans
// and resets the counter to zero for the next call.
#include "split_common.h"

namespace pion {
namespace {

// The sum / max of lanes l and l ^ 16 (by32: l ^ 32) in every lane, by the row swaps.
__device__ __forceinline__ float swap_pair_max(float v, bool by32) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = by32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                      : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float swap_pair_sum(float v, bool by32) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = by32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                      : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
// Sum over each group of W consecutive lanes (W = 4 .. 64); every lane of a group
// receives the group sum. quad_perm [1,0,3,2] and [2,3,0,1] give quad sums, row
// half-mirror pairs the two quads of 8 lanes, row mirror the two halves of 16, a
// swizzle with xor 16 the two rows of 32, and the cross-half swap the halves of 64.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  if constexpr (W >= 8) v += dpp<0x141>(v);
  if constexpr (W >= 16) v += dpp<0x140>(v);
  if constexpr (W >= 32)
    v += __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  if constexpr (W >= 64) v = swap_pair_sum(v, true);
  return v;
}

// Combine each lane with the lanes that differ from it in the bits >= LPR of the lane
// index (the slots of a wave holding the same dims), without LDS: within a 16-lane row
// by rotations (by 4, then 8: together every lane of the same index mod LPR), lane ^ 16
// and lane ^ 32 by the row swaps. Every lane gets the result; LPR = 64 is one slot.
template <int LPR>
__device__ __forceinline__ float slots_max(float v) {
  if constexpr (LPR <= 4) v = fmaxf(v, dpp<0x124>(v));  // row rotate by 4
  if constexpr (LPR <= 8) v = fmaxf(v, dpp<0x128>(v));  // row rotate by 8: lane ^ 8
  if constexpr (LPR <= 16) v = swap_pair_max(v, false);
  if constexpr (LPR <= 32) v = swap_pair_max(v, true);
  return v;
}
template <int LPR>
__device__ __forceinline__ float slots_sum(float v) {
  if constexpr (LPR <= 4) v += dpp<0x124>(v);
  if constexpr (LPR <= 8) v += dpp<0x128>(v);
  if constexpr (LPR <= 16) v = swap_pair_sum(v, false);
  if constexpr (LPR <= 32) v = swap_pair_sum(v, true);
  return v;
}

template <int D, int R, int NW>
struct WaveState {
  float m[NW][R];
  float l[NW][R];
  alignas(16) float acc[NW][R][D];
};

template <int D, int R, int NW>
struct Scratch {
  union {
    WaveState<D, R, NW> ws;
  };
  int last;
};

// Wave-level slot merge, workgroup merge, partial store, ticket, and (last) merge.
template <int D, int R, int LPR, int NW>
__device__ __forceinline__ void finish(const PartialParams &p, const Prob &b, Scratch<D, R, NW> &sm,
                                       float (&m)[R], float (&l)[R], float (&acc)[R][8],
                                       const Group &gr, int qi, int x) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int sub = lane % LPR, kk = lane / LPR;
  WaveState<D, R, NW> &ws = sm.ws;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float M = slots_max<LPR>(m[r]);
    const float f = fast_exp2(m[r] - M);
    const float lr = slots_sum<LPR>(l[r] * f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = slots_sum<LPR>(acc[r][e] * f);
    if (kk == 0 && sub < D / 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ws.acc[wave][r][sub * 8 + e] = acc[r][e];
    }
    if (lane == 0) {
      ws.m[wave][r] = M;
      ws.l[wave][r] = lr;
    }
  }
  __syncthreads();
  const PartRsrc pr = part_rsrc(p, b, qi);
  constexpr int DQ = D / 4;
  for (int t = threadIdx.x; t < gr.cnt * DQ; t += 64 * NW) {
    const int r = t / DQ, dq = t - r * DQ;
    float mm = ws.m[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) mm = fmaxf(mm, ws.m[w][r]);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    float lw = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(ws.m[w][r] - mm);
      a += f * *(const f32x4 *)&ws.acc[w][r][4 * dq];
      lw = __builtin_fmaf(f, ws.l[w][r], lw);
    }
    if (b.S_total == 1) {  // the only span of its rows: final output, no merge
      const size_t row = (size_t)gr.head(r) * p.M + qi;
      const float inv = lw > 0.f ? 1.f / lw : 0.f;  // no key at all: out 0, lse -inf
      *(float4 *)(b.out + row * D + 4 * dq) = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
      if (dq == 0 && b.lse)
        b.lse[row] = lw > 0.f ? (mm + __log2f(lw)) * 0.69314718055994530942f : -INFINITY;
    } else {
      store_part(pr, gr.head(r), x, dq, a);
      if (dq == 0) store_ml(pr, gr.head(r), x, lw > 0.f ? mm : -INFINITY, lw);  // empty: weight 0
    }
  }
  if (b.S_total > 1) ticket_and_merge<D, 64 * NW>(p, b, pr, gr, qi, sm.last);
}

// One tile: U keys per lane (keys base + u*KPI + kk), NV 16-byte pieces per key and side.
template <int U, int NV>
struct Tile {
  uint4 k[U][NV], v[U][NV];
  bool ok[U];
};

// A lane's 8 q values of each row: fp16 pairs, or fp32.
template <bool F32, int R>
struct QRegs {
  h2_t q[R][4];
};
template <int R>
struct QRegs<true, R> {
  float q[R][8];
};

__device__ __forceinline__ float f32_bits(uint32_t u) { return __builtin_bit_cast(float, u); }

template <int D, int R, int U, bool GATHER, bool F32, int NW = 4>
__global__ __launch_bounds__(64 * NW) void attn_split_kernel(PartialParams p) {
  constexpr int LPR = fp16_row_lanes(D), KPI = 64 / LPR, STEP = KPI * U;
  constexpr int ESZ = F32 ? 4 : 2, NV = F32 ? 2 : 1;  // bytes per value, pieces per 8 values
  __shared__ Scratch<D, R, NW> sm;
  __shared__ int gsp[GATHER ? kGatherChunk : 1];  // the span's token indices
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int sub = lane % LPR, kk = lane / LPR;
  const bool dims = sub < D / 8;  // this lane holds 8 dims of a row
  const int z = blockIdx.z, y = blockIdx.y;
  int hg;
  Prob b;
  const Group gr = entry_group(p, z, y, hg, b);
  const int x = blockIdx.x + p.x_begin;
  if (x >= b.S_total) return;  // this problem has fewer spans than the grid
  const int qi = y - hg * p.M;
  const int g = gr.g, cnt = gr.cnt;
  // q of each row: this lane's 8 values
  QRegs<F32, R> qr;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = gr.head(r < cnt ? r : 0);
    const uint4 *qp =
        (const uint4 *)((const char *)b.Q + (((size_t)h * p.M + qi) * D + sub * 8) * ESZ);
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const uint4 qq = dims ? qp[t] : make_uint4(0, 0, 0, 0);
      if constexpr (F32) {
        qr.q[r][4 * t] = f32_bits(qq.x);
        qr.q[r][4 * t + 1] = f32_bits(qq.y);
        qr.q[r][4 * t + 2] = f32_bits(qq.z);
        qr.q[r][4 * t + 3] = f32_bits(qq.w);
      } else {
        qr.q[r][0] = as_h2(qq.x);
        qr.q[r][1] = as_h2(qq.y);
        qr.q[r][2] = as_h2(qq.z);
        qr.q[r][3] = as_h2(qq.w);
      }
    }
  }

  float m[R], l[R], acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegBig;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  // the segments of this span, one after another (wave-uniform loop)
  const int seg0 = x * p.seg_per_span, seg1 = min(seg0 + p.seg_per_span, b.n_seg);
  for (int sgi = seg0; sgi < seg1; ++sgi) {
    Span sp = get_segment(p, sgi, b.pre_splits, b.N, g, qi);
    if (!sp.suffix && p.fmt == 1) continue;  // an mlx4g32 prefix has its own kernel
    if constexpr (GATHER) {  // list positions [j0, j1) of q-head heads[0]'s token list
      const int h = gr.head(0);
      sp.j1 = min(sp.j1, max(sp.j0, min(p.gcount[h], p.gmax)));
      __syncthreads();  // the previous segment is done with gsp
      for (int t = threadIdx.x; t < sp.j1 - sp.j0; t += 64 * NW)
        gsp[t] = p.gidx[(size_t)h * p.gmax + sp.j0 + t];
      __syncthreads();
    }
    const char *Kf, *Vf;  // kv-head g's rows of this segment's keys
    if (sp.suffix) {
      Kf = (const char *)p.Ksuf + (size_t)g * p.S_suf * D * ESZ;
      Vf = (const char *)p.Vsuf + (size_t)g * p.S_suf * D * ESZ;
    } else {
      const KVView kv = make_view(p.kv_base[z], p.fmt, p.H_kv, b.N, D);
      Kf = (const char *)kv.K + (size_t)g * b.N * D * ESZ;
      Vf = (const char *)kv.V + (size_t)g * b.N * D * ESZ;
    }

    auto load = [&](Tile<U, NV> &t, int base) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int j = base + u * KPI + kk;
        t.ok[u] = j < sp.j1;
        if constexpr (GATHER) {  // the listed token; one outside [0, N) is skipped
          const int tok = t.ok[u] ? gsp[j - sp.j0] : 0;
          t.ok[u] = t.ok[u] && tok >= 0 && tok < b.N;
          j = tok;
        }
        const size_t off = ((size_t)j * D + sub * 8) * ESZ;
#pragma unroll
        for (int w = 0; w < NV; ++w) {
          if (t.ok[u] && dims) {
            t.k[u][w] = ld_stream16(Kf + off + 16 * w);
            t.v[u][w] = ld_stream16(Vf + off + 16 * w);
          } else {
            t.k[u][w] = make_uint4(0, 0, 0, 0);
            t.v[u][w] = make_uint4(0, 0, 0, 0);
          }
        }
      }
    };

    auto consume = [&](const Tile<U, NV> &t) {
      float vals[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if constexpr (F32) {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            vals[u][4 * w] = f32_bits(t.v[u][w].x);
            vals[u][4 * w + 1] = f32_bits(t.v[u][w].y);
            vals[u][4 * w + 2] = f32_bits(t.v[u][w].z);
            vals[u][4 * w + 3] = f32_bits(t.v[u][w].w);
          }
        } else {
          const uint32_t w4[4] = {t.v[u][0].x, t.v[u][0].y, t.v[u][0].z, t.v[u][0].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            vals[u][2 * c] = h2f((uint16_t)(w4[c] & 0xffffu));
            vals[u][2 * c + 1] = h2f((uint16_t)(w4[c] >> 16));
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float dsum;
          if constexpr (F32) {
            dsum = 0.f;
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              dsum = __builtin_fmaf(qr.q[r][4 * w], f32_bits(t.k[u][w].x), dsum);
              dsum = __builtin_fmaf(qr.q[r][4 * w + 1], f32_bits(t.k[u][w].y), dsum);
              dsum = __builtin_fmaf(qr.q[r][4 * w + 2], f32_bits(t.k[u][w].z), dsum);
              dsum = __builtin_fmaf(qr.q[r][4 * w + 3], f32_bits(t.k[u][w].w), dsum);
            }
          } else {
            dsum = __builtin_amdgcn_fdot2(qr.q[r][0], as_h2(t.k[u][0].x), 0.f, false);
            dsum = __builtin_amdgcn_fdot2(qr.q[r][1], as_h2(t.k[u][0].y), dsum, false);
            dsum = __builtin_amdgcn_fdot2(qr.q[r][2], as_h2(t.k[u][0].z), dsum, false);
            dsum = __builtin_amdgcn_fdot2(qr.q[r][3], as_h2(t.k[u][0].w), dsum, false);
          }
          dsum = group_sum<LPR>(dsum);
          s[u] = t.ok[u] ? dsum * p.qscale : -INFINITY;
        }
        float mx = m[r];
#pragma unroll
        for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u]);
        const float alpha = fast_exp2(m[r] - mx);
        l[r] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
        m[r] = mx;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float pe = fast_exp2(s[u] - mx);  // masked: 2^-inf = 0
          l[r] += pe;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] = __builtin_fmaf(pe, vals[u][e], acc[r][e]);
        }
      }
    };

    int base = sp.j0 + wave * STEP;
    Tile<U, NV> cur;
    if (base < sp.j1) load(cur, base);
    while (base < sp.j1) {
      const int next = base + NW * STEP;
      Tile<U, NV> nxt;
      if (next < sp.j1) load(nxt, next);
      consume(cur);
      cur = nxt;
      base = next;
    }
  }
  finish<D, R, LPR, NW>(p, b, sm, m, l, acc, gr, qi, x);
}

// fp32 (slot format 2) tiles hold twice the bytes per key, so half the keys per lane
template <int D, int R>
hipError_t launch_partial_d(const PartialParams &p, int x_count, hipStream_t s) {
  dim3 grid(x_count, p.y_groups, p.n_prob);
  const bool f32 = p.fmt == 2;
  if (p.gidx)
    note_launch("attn_split_kernel<%d,1,%d,true,%s>", D, f32 ? 2 : 4, f32 ? "true" : "false");
  else if (f32)
    note_launch("attn_split_kernel<%d,%d,2,false,true>", D, R);
  else if (p.waves == 8 && R <= 4)
    note_launch("attn_split_kernel<%d,%d,4,false,false,8>", D, R);
  else
    note_launch("attn_split_kernel<%d,%d,4,false,false>", D, R);
  if (p.gidx && f32)
    hipLaunchKernelGGL((attn_split_kernel<D, 1, 2, true, true>), grid, dim3(256), 0, s, p);
  else if (p.gidx)
    hipLaunchKernelGGL((attn_split_kernel<D, 1, 4, true, false>), grid, dim3(256), 0, s, p);
  else if (f32)
    hipLaunchKernelGGL((attn_split_kernel<D, R, 2, false, true>), grid, dim3(256), 0, s, p);
  else if (p.waves == 8 && R <= 4)  // 8-wave workgroups (twice the keys per workgroup)
    hipLaunchKernelGGL((attn_split_kernel<D, R <= 4 ? R : 1, 4, false, false, 8>), grid, dim3(512),
                       0, s, p);
  else
    hipLaunchKernelGGL((attn_split_kernel<D, R, 4, false, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_partial_r(const PartialParams &p, int R, int xc, hipStream_t s) {
  switch (R) {
    case 1: return launch_partial_d<D, 1>(p, xc, s);
    case 2: return launch_partial_d<D, 2>(p, xc, s);
    case 4: return launch_partial_d<D, 4>(p, xc, s);
    default: return launch_partial_d<D, 8>(p, xc, s);
  }
}

__global__ void fill_zero_kernel(int *p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_counters(int *counters, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, counters, n);
  return hipGetLastError();
}

hipError_t launch_partial(const PartialParams &p, int rows_per_group, int x_count,
                          hipStream_t s) {
  if (x_count < 1 || p.y_groups < 1 || p.n_prob < 1) return hipSuccess;
  if (p.S_max > kMaxSplits || p.n_prob > kMaxBatch) return hipErrorInvalidValue;
  // a token list: one q-head per row group, one segment per span of at most kGatherChunk
  if (p.gidx && (rows_per_group != 1 || p.seg_per_span != 1 || p.pre_chunk > kGatherChunk ||
                 p.n_prob != 1 || p.fmt == 1))
    return hipErrorInvalidValue;
  if (p.esz != (p.fmt == 2 ? 4 : 2)) return hipErrorInvalidValue;
  if (p.waves != 4 && !(p.waves == 8 && !p.gidx && p.fmt == 0 && rows_per_group <= 4))
    return hipErrorInvalidValue;
  switch (p.D) {
    case 32: return launch_partial_r<32>(p, rows_per_group, x_count, s);
    case 64: return launch_partial_r<64>(p, rows_per_group, x_count, s);
    case 96: return launch_partial_r<96>(p, rows_per_group, x_count, s);
    case 128: return launch_partial_r<128>(p, rows_per_group, x_count, s);
    case 160: return launch_partial_r<160>(p, rows_per_group, x_count, s);
    case 192: return launch_partial_r<192>(p, rows_per_group, x_count, s);
    case 256: return launch_partial_r<256>(p, rows_per_group, x_count, s);
    case 512: return launch_partial_r<512>(p, rows_per_group, x_count, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pion
