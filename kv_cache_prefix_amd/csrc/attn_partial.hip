// Split-over-keys attention (VALU path) with the split merge done in-kernel.
//
// What is computed: for each query row (q-head h, query index i) and each key span of
// a workgroup, the online-softmax partial
//     m = max_j s_j,  l = sum_j 2^(s_j - m),  acc = sum_j 2^(s_j - m) v_j,
// with s_j = log2(e)/sqrt(D) * (q . k_j), the scaled logit in log2 units. The spans of
// a row are merged by the LSE rule (the online-softmax merge of the "Shared KV Cache
// Serving" page, Stage 2 consumer and Wire-protocol details):
//     m* = max_c m_c,  w_c = 2^(m_c - m*),  out = sum_c w_c acc_c / sum_c w_c l_c,
//     lse = ln 2 * (m* + log2 sum_c w_c l_c).
//
// Layout and schedule. A key row of D halves is read by D/8 consecutive lanes, 16 bytes
// each (one wave-wide load covers 64/(D/8) whole rows, fully coalesced). Each group of
// D/8 lanes is a "slot" that runs its own online softmax over the keys it sees, so the
// inner loop needs no cross-lane max: only the D/8-lane dot-product sum, done with DPP
// row operations. K and V of the next tile are loaded before the current tile is
// consumed. At the end the slots of a wave and the 4 waves of the workgroup merge (LDS),
// and the workgroup stores its partial. All q-heads that read the same kv-head share a
// workgroup, so K/V bytes are read once per kv-head (GQA).
//
// The mlx4g32 variant reads, per lane and key, one uint32 of codes (8 elements) and the
// fp16 scale and bias of that word's group, and dequantizes in registers:
// q . k = s * (q . c) + b * sum(q) per word, v = s * c + b (the bias term is
// accumulated once per key as p * b).
//
// The merge runs in the same kernel: every workgroup stores its partial, then takes a
// ticket on its row group's counter; the workgroup that arrives last merges all spans
// and resets the counter to zero for the next call. Cross-XCD visibility without L2
// flushes: partials are written and read with agent-scope relaxed atomic accesses
// (coherent at agent scope, never held dirty or stale in a per-XCD L2), and each wave
// waits for its partial stores to complete (s_waitcnt vmcnt(0)) before the workgroup
// barrier that precedes its ticket. An agent-scope fence here would write back and
// invalidate the whole L2 of the XCD for every workgroup.
#include "kernels.h"

namespace pion {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;  // running-max start: 2^(kNegBig - kNegBig) = 1
constexpr int kMaxSplits = 1024;

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ float h2f(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each group of W consecutive lanes (W = 8, 16 or 32); every lane of a group
// receives the group sum. quad_perm [1,0,3,2] and [2,3,0,1] give quad sums, row
// half-mirror pairs the two quads of 8 lanes, row mirror the two halves of 16, and a
// swizzle with xor 16 the two rows of 32.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  if constexpr (W >= 16) v += dpp<0x140>(v);
  if constexpr (W >= 32)
    v += __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  return v;
}

// Agent-coherent accesses for data handed between workgroups (see the header).
__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Span {
  int j0, j1;
  bool suffix;
};

__device__ __forceinline__ Span get_span(const PartialParams &p, int x, int pre_splits, int N,
                                         int g, int qi) {
  Span s;
  if (x < pre_splits) {
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
    } else {
      s.j0 = x * p.pre_chunk;
      s.j1 = min(s.j0 + p.pre_chunk, N);
    }
  } else {
    s.suffix = true;
    const int c = x - pre_splits;
    const int lim = p.S_suf - p.M + qi + 1;  // causal, bottom-right aligned
    s.j0 = c * p.suf_chunk;
    s.j1 = min(min(s.j0 + p.suf_chunk, p.S_suf), lim);
  }
  return s;
}

template <int D, int R>
struct WaveState {
  float m[4][R];
  float l[4][R];
  float acc[4][R][D];
};

template <int D, int R>
struct Scratch {
  union {
    WaveState<D, R> ws;
    float red[3][256];
  };
  int last;
};

// Per-problem pointers of this workgroup.
struct Prob {
  int N, pre_splits, S_total;
  const uint16_t *Q;
  float *out, *lse, *part_acc, *part_m, *part_l;
  int *counter;
};

__device__ __forceinline__ Prob get_prob(const PartialParams &p, int z, int y) {
  Prob b;
  b.N = p.N[z];
  b.pre_splits = p.blocks ? p.n_sel : (b.N + p.pre_chunk - 1) / p.pre_chunk;
  b.S_total = b.pre_splits + p.suf_splits;
  b.Q = p.Q + z * p.q_stride;
  b.out = p.out + z * p.out_stride;
  b.lse = p.lse ? p.lse + z * p.lse_stride : nullptr;
  b.part_acc = p.part_acc + z * p.part_stride;
  b.part_m = p.part_m + z * p.ml_stride;
  b.part_l = p.part_l + z * p.ml_stride;
  b.counter = p.counters + (size_t)z * p.y_groups + y;
  return b;
}

// Merge the S_total partials of the rows of this workgroup into out / lse, in the one
// workgroup of the row group that took the last ticket. Loads of a row are issued in
// batches before any is consumed: thread t owns dim d = t % D and the spans
// c = t / D mod P (P = 256 / D), keeps a running (m, l, acc) over them, and the P
// partial results merge through LDS.
template <int D, int R>
__device__ __forceinline__ void merge_rows(const PartialParams &p, const Prob &b,
                                           const uint8_t *heads, int cnt, int qi,
                                           Scratch<D, R> &sm) {
  constexpr int P = 256 / D;
  constexpr int CH = 16;  // spans loaded per batch per thread
  const int tid = threadIdx.x, d = tid % D, ph = tid / D;
  for (int r = 0; r < cnt; ++r) {
    const int row = heads[r] * p.M + qi;
    const float *pm = b.part_m + (size_t)row * p.S_max;
    const float *pl = b.part_l + (size_t)row * p.S_max;
    const float *pa = b.part_acc + (size_t)row * p.S_max * D;
    float m = kNegBig, l = 0.f, a = 0.f;
    for (int c0 = ph; c0 < b.S_total; c0 += P * CH) {
      float mc[CH], lc[CH], ac[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int c = c0 + k * P;
        const bool in = c < b.S_total;
        mc[k] = in ? ld_agent(pm + c) : -INFINITY;
        lc[k] = in ? ld_agent(pl + c) : 0.f;
        ac[k] = in ? ld_agent(pa + (size_t)c * D + d) : 0.f;
      }
      float mx = m;
#pragma unroll
      for (int k = 0; k < CH; ++k) mx = fmaxf(mx, mc[k]);
      const float f = fast_exp2(m - mx);
      l *= f;
      a *= f;
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const float w = fast_exp2(mc[k] - mx);  // empty span: m = -inf -> 0
        l = __builtin_fmaf(w, lc[k], l);
        a = __builtin_fmaf(w, ac[k], a);
      }
      m = mx;
    }
    if constexpr (P > 1) {
      sm.red[0][tid] = m;
      sm.red[1][tid] = l;
      sm.red[2][tid] = a;
      __syncthreads();
      if (ph == 0) {
        float M = m;
#pragma unroll
        for (int q = 1; q < P; ++q) M = fmaxf(M, sm.red[0][q * D + d]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int q = 0; q < P; ++q) {
          const float f = fast_exp2(sm.red[0][q * D + d] - M);
          L = __builtin_fmaf(f, sm.red[1][q * D + d], L);
          A = __builtin_fmaf(f, sm.red[2][q * D + d], A);
        }
        m = M;
        l = L;
        a = A;
      }
      __syncthreads();
    }
    if (ph == 0) {
      b.out[(size_t)row * D + d] = a / l;
      if (d == 0 && b.lse) b.lse[row] = (m + __log2f(l)) * 0.69314718055994530942f;
    }
  }
}

// Wave-level slot merge, workgroup merge, partial store, ticket, and (last) merge.
template <int D, int R, int LPR>
__device__ __forceinline__ void finish(const PartialParams &p, const Prob &b, Scratch<D, R> &sm,
                                       float (&m)[R], float (&l)[R], float (&acc)[R][8],
                                       const uint8_t *heads, int cnt, int qi, int x) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, kk = lane / LPR;
  WaveState<D, R> &ws = sm.ws;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float M = m[r];
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = fast_exp2(m[r] - M);
    float lr = l[r] * f;
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) lr += __shfl_xor(lr, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[r][e] * f;
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o);
      acc[r][e] = v;
    }
    if (kk == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ws.acc[wave][r][sub * 8 + e] = acc[r][e];
    }
    if (lane == 0) {
      ws.m[wave][r] = M;
      ws.l[wave][r] = lr;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < cnt * D; t += 256) {
    const int r = t / D, d = t - r * D;
    const float mm = fmaxf(fmaxf(ws.m[0][r], ws.m[1][r]), fmaxf(ws.m[2][r], ws.m[3][r]));
    float a = 0.f, lw = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = fast_exp2(ws.m[w][r] - mm);
      a = __builtin_fmaf(f, ws.acc[w][r][d], a);
      lw = __builtin_fmaf(f, ws.l[w][r], lw);
    }
    const int row = heads[r] * p.M + qi;
    const size_t o = (size_t)row * p.S_max + x;
    st_agent(b.part_acc + o * D + d, a);
    if (d == 0) {
      st_agent(b.part_m + o, lw > 0.f ? mm : -INFINITY);  // empty span: weight 0
      st_agent(b.part_l + o, lw);
    }
  }
  // this wave's partial stores have completed before the barrier and the ticket
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int t = __hip_atomic_fetch_add(b.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = (t == b.S_total - 1);
  }
  __syncthreads();
  if (!sm.last) return;
  merge_rows<D, R>(p, b, heads, cnt, qi, sm);
  if (threadIdx.x == 0)
    __hip_atomic_store(b.counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One tile: U key slots per lane (keys base + u*KPI + kk). FMT 0 holds fp16 rows,
// FMT 1 mlx4g32 code words with their group scale and bias.
template <int U, int FMT>
struct Tile {
  uint4 k[U], v[U];
  uint32_t kw[U], vw[U];
  float ks[U], kb[U], vs[U], vb[U];
  bool ok[U];
};

template <int D, int R, int U, int FMT>
__global__ __launch_bounds__(256) void attn_split_kernel(PartialParams p) {
  constexpr int LPR = D / 8, KPI = 64 / LPR, STEP = KPI * U, NG = D / 32;
  __shared__ Scratch<D, R> sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, kk = lane / LPR;
  const int grp = sub >> 2;  // the group of this lane's 8 elements
  const int z = blockIdx.z, y = blockIdx.y;
  const Prob b = get_prob(p, z, y);
  const int x = blockIdx.x + p.x_begin;
  if (x >= b.S_total) return;  // this problem has fewer spans than the grid
  const int hg = y / p.M, qi = y - hg * p.M;
  const int g = p.rg.g[hg], cnt = p.rg.cnt[hg];
  const uint8_t *heads = p.rg.heads[hg];
  Span sp = get_span(p, x, b.pre_splits, b.N, g, qi);
  if (FMT == 1 && sp.suffix) sp.j1 = sp.j0;                 // prefix-only kernel
  if (FMT == 0 && !sp.suffix && p.fmt != 0) sp.j1 = sp.j0;  // fp16-only kernel

  const KVView kv = make_view(p.kv_base[z], p.fmt, p.H_kv, b.N, D);
  const uint16_t *Kf = nullptr, *Vf = nullptr;
  const uint32_t *Kc = nullptr, *Vc = nullptr;
  const uint16_t *Ks = nullptr, *Kb = nullptr, *Vs = nullptr, *Vb = nullptr;
  if (sp.suffix) {
    Kf = p.Ksuf + (size_t)g * p.S_suf * D;
    Vf = p.Vsuf + (size_t)g * p.S_suf * D;
  } else if (FMT == 0) {
    Kf = kv.K + (size_t)g * b.N * D;
    Vf = kv.V + (size_t)g * b.N * D;
  } else {
    const size_t t0 = (size_t)g * b.N;
    Kc = kv.Kc + t0 * (D / 8);
    Vc = kv.Vc + t0 * (D / 8);
    Ks = kv.Ks + t0 * NG;
    Kb = kv.Kb + t0 * NG;
    Vs = kv.Vs + t0 * NG;
    Vb = kv.Vb + t0 * NG;
  }

  // q of each row: this lane's 8 halves. For mlx4g32 they are paired (k, k+4), the
  // order in which (word >> 4k) & 0x000F000F yields two codes, and summed for the
  // bias term.
  h2_t q[R][4];
  float qsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = heads[r < cnt ? r : 0];
    const uint4 qq = *(const uint4 *)(b.Q + ((size_t)h * p.M + qi) * D + sub * 8);
    if (FMT == 0) {
      q[r][0] = as_h2(qq.x);
      q[r][1] = as_h2(qq.y);
      q[r][2] = as_h2(qq.z);
      q[r][3] = as_h2(qq.w);
      qsum[r] = 0.f;
    } else {
      const uint32_t w4[4] = {qq.x, qq.y, qq.z, qq.w};
      uint16_t e[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        e[2 * c] = (uint16_t)(w4[c] & 0xffffu);
        e[2 * c + 1] = (uint16_t)(w4[c] >> 16);
      }
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h2_t t;
        t.x = __builtin_bit_cast(_Float16, e[k]);
        t.y = __builtin_bit_cast(_Float16, e[k + 4]);
        q[r][k] = t;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) s += h2f(e[k]);
      qsum[r] = s;
    }
  }

  float m[R], l[R], acc[R][8], bsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegBig;
    l[r] = 0.f;
    bsum[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  auto load = [&](Tile<U, FMT> &t, int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * KPI + kk;
      t.ok[u] = j < sp.j1;
      if (FMT == 0) {
        if (t.ok[u]) {
          t.k[u] = *(const uint4 *)(Kf + (size_t)j * D + sub * 8);
          t.v[u] = *(const uint4 *)(Vf + (size_t)j * D + sub * 8);
        } else {
          t.k[u] = make_uint4(0, 0, 0, 0);
          t.v[u] = make_uint4(0, 0, 0, 0);
        }
      } else {
        const int jj = t.ok[u] ? j : sp.j0;  // in-bounds stand-in, masked below
        t.kw[u] = Kc[(size_t)jj * (D / 8) + sub];
        t.vw[u] = Vc[(size_t)jj * (D / 8) + sub];
        t.ks[u] = h2f(Ks[(size_t)jj * NG + grp]);
        t.kb[u] = h2f(Kb[(size_t)jj * NG + grp]);
        t.vs[u] = h2f(Vs[(size_t)jj * NG + grp]);
        t.vb[u] = h2f(Vb[(size_t)jj * NG + grp]);
      }
    }
  };

  auto consume = [&](const Tile<U, FMT> &t) {
    float vals[U][8];
    h2_t kc[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (FMT == 0) {
        const uint32_t w4[4] = {t.v[u].x, t.v[u].y, t.v[u].z, t.v[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          vals[u][2 * c] = h2f((uint16_t)(w4[c] & 0xffffu));
          vals[u][2 * c + 1] = h2f((uint16_t)(w4[c] >> 16));
        }
      } else {
        const h2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[u][e] = (float)((t.vw[u] >> (4 * e)) & 0xFu) * t.vs[u];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          kc[u][k] = as_h2(((t.kw[u] >> (4 * k)) & 0x000F000Fu) | 0x64006400u) - k1024;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float dsum;
        if (FMT == 0) {
          dsum = __builtin_amdgcn_fdot2(q[r][0], as_h2(t.k[u].x), 0.f, false);
          dsum = __builtin_amdgcn_fdot2(q[r][1], as_h2(t.k[u].y), dsum, false);
          dsum = __builtin_amdgcn_fdot2(q[r][2], as_h2(t.k[u].z), dsum, false);
          dsum = __builtin_amdgcn_fdot2(q[r][3], as_h2(t.k[u].w), dsum, false);
        } else {
          dsum = __builtin_amdgcn_fdot2(q[r][0], kc[u][0], 0.f, false);
          dsum = __builtin_amdgcn_fdot2(q[r][1], kc[u][1], dsum, false);
          dsum = __builtin_amdgcn_fdot2(q[r][2], kc[u][2], dsum, false);
          dsum = __builtin_amdgcn_fdot2(q[r][3], kc[u][3], dsum, false);
          dsum = __builtin_fmaf(t.ks[u], dsum, t.kb[u] * qsum[r]);
        }
        dsum = group_sum<LPR>(dsum);
        s[u] = t.ok[u] ? dsum * p.qscale : -INFINITY;
      }
      float mx = m[r];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u]);
      const float alpha = fast_exp2(m[r] - mx);
      l[r] *= alpha;
      bsum[r] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
      m[r] = mx;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pe = fast_exp2(s[u] - mx);  // masked: 2^-inf = 0
        l[r] += pe;
        if (FMT == 1) bsum[r] = __builtin_fmaf(pe, t.vb[u], bsum[r]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = __builtin_fmaf(pe, vals[u][e], acc[r][e]);
      }
    }
  };

  int base = sp.j0 + wave * STEP;
  Tile<U, FMT> cur;
  if (base < sp.j1) load(cur, base);
  while (base < sp.j1) {
    const int next = base + 4 * STEP;
    Tile<U, FMT> nxt;
    if (next < sp.j1) load(nxt, next);
    consume(cur);
    cur = nxt;
    base = next;
  }
  if (FMT == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] += bsum[r];
  }
  finish<D, R, LPR>(p, b, sm, m, l, acc, heads, cnt, qi, x);
}

template <int D, int R>
hipError_t launch_partial_d(const PartialParams &p, int x_count, bool mlx4, hipStream_t s) {
  dim3 grid(x_count, p.y_groups, p.n_prob);
  if (mlx4) {
    constexpr int U = (D == 256) ? 2 : 4;
    hipLaunchKernelGGL((attn_split_kernel<D, R, U, 1>), grid, dim3(256), 0, s, p);
  } else {
    constexpr int U = 4;
    hipLaunchKernelGGL((attn_split_kernel<D, R, U, 0>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_partial_r(const PartialParams &p, int R, int xc, bool mlx4, hipStream_t s) {
  switch (R) {
    case 1: return launch_partial_d<D, 1>(p, xc, mlx4, s);
    case 2: return launch_partial_d<D, 2>(p, xc, mlx4, s);
    case 4: return launch_partial_d<D, 4>(p, xc, mlx4, s);
    default: return launch_partial_d<D, 8>(p, xc, mlx4, s);
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
                          bool mlx4_prefix, hipStream_t s) {
  if (x_count < 1 || p.y_groups < 1 || p.n_prob < 1) return hipSuccess;
  if (p.S_max > kMaxSplits || p.n_prob > kMaxBatch) return hipErrorInvalidValue;
  switch (p.D) {
    case 64: return launch_partial_r<64>(p, rows_per_group, x_count, mlx4_prefix, s);
    case 128: return launch_partial_r<128>(p, rows_per_group, x_count, mlx4_prefix, s);
    case 256: return launch_partial_r<256>(p, rows_per_group, x_count, mlx4_prefix, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pion
