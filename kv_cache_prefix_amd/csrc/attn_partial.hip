// Split-over-keys attention (VALU path) with the split merge done in-kernel.
//
// What is computed: for each query row (q-head h, query index i) and each key span of
// the workgroup, the unnormalized online-softmax partial
//     m = max_j s_j,  l = sum_j 2^(s_j - m),  acc = sum_j 2^(s_j - m) v_j,
// with s_j = log2(e)/sqrt(D) * (q . k_j), i.e. the scaled logit in log2 units. The
// spans of a row are then merged by the LSE rule (the online-softmax merge of the
// "Shared KV Cache Serving" page, Stage 2 consumer and Wire-protocol details):
//     m* = max_c m_c,  w_c = 2^(m_c - m*),  out = sum_c w_c acc_c / sum_c w_c l_c,
//     lse = ln 2 * (m* + log2 sum_c w_c l_c).
// The merge runs in the same kernel: every workgroup stores its partial, then takes a
// ticket on its row group's counter; the workgroup that arrives last (all spans of
// the group are stored) merges them and resets the counter to zero for the next call.
// Cross-XCD visibility without L2 flushes: partials are written and read with
// agent-scope relaxed atomic accesses (coherent at agent scope, never held dirty or
// stale in a per-XCD L2), and each wave waits for its partial stores to complete
// (s_waitcnt vmcnt(0)) before the workgroup barrier that precedes its ticket. An
// agent-scope fence here would write back and invalidate the whole L2 of the XCD for
// every workgroup.
//
// Layout: a key row of D halves is read by D/8 consecutive lanes, 16 bytes each, so one
// wave-wide load instruction covers 64/(D/8) whole key rows (fully coalesced). The
// q . k partial of each lane is summed across its D/8 lanes; every lane then holds the
// key's score, weights its own 8 V elements, and keeps 8 fp32 accumulators per row.
// All q-heads that read the same kv-head share one workgroup, so K/V bytes are read
// once per kv-head (GQA). The mlx4g32 variant reads 4 bytes of codes per lane (8
// elements, one uint32 word) plus that word's group scale and bias, and dequantizes
// in registers: q . k = s * (q . c) + b * sum(q) per word, v = s * c + b.
#include "kernels.h"

namespace pion {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }

__device__ __forceinline__ float h2f(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}

// Butterfly sum over W consecutive lanes (W a power of two).
template <int W>
__device__ __forceinline__ float sum_lanes(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v += __shfl_xor(v, o);
  return v;
}
// Sum / max over the lanes that share `lane % LPR` (one per key slot of the wave).
template <int LPR>
__device__ __forceinline__ float sum_slots(float v) {
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}
template <int LPR>
__device__ __forceinline__ float max_slots(float v) {
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

__device__ __forceinline__ Span get_span(const PartialParams &p, int x, int g, int qi) {
  Span s;
  if (x < p.pre_splits) {
    s.suffix = false;
    if (p.blocks) {
      const int nb = (p.kv.N + p.B - 1) / p.B;
      const int b = p.blocks[g * p.K_top + x];
      if (b < 0 || b >= nb) {  // device-produced index: never trust it for addressing
        s.j0 = s.j1 = 0;
      } else {
        s.j0 = b * p.B;
        s.j1 = min(s.j0 + p.B, p.kv.N);
      }
    } else {
      s.j0 = x * p.pre_chunk;
      s.j1 = min(s.j0 + p.pre_chunk, p.kv.N);
    }
  } else {
    s.suffix = true;
    const int c = x - p.pre_splits;
    const int lim = p.S_suf - p.M + qi + 1;  // causal, bottom-right aligned
    s.j0 = c * p.suf_chunk;
    s.j1 = min(min(s.j0 + p.suf_chunk, p.S_suf), lim);
  }
  return s;
}

// Workgroup-level merge of the 4 waves' (m, l, acc) and the partial store.
template <int D, int R>
struct WaveState {
  float m[4][R];
  float l[4][R];
  float acc[4][R][D];
};

constexpr int kMaxSplits = 1024;

template <int D, int R>
struct WaveScratch {
  union {
    WaveState<D, R> ws;
    float w[kMaxSplits];
  };
  float red[8];
  int last;
};

template <int D, int R>
__device__ __forceinline__ void store_partial(const PartialParams &p, WaveState<D, R> &ws,
                                              const uint8_t *heads, int cnt, int qi, int x) {
  for (int t = threadIdx.x; t < cnt * D; t += 256) {
    const int r = t / D, d = t - r * D;
    float mm = fmaxf(fmaxf(ws.m[0][r], ws.m[1][r]), fmaxf(ws.m[2][r], ws.m[3][r]));
    const int row = heads[r] * p.M + qi;
    const size_t o = (size_t)row * p.S_total + x;
    if (mm == -INFINITY) {  // empty span
      st_agent(p.part_acc + o * D + d, 0.f);
      if (d == 0) {
        st_agent(p.part_m + o, -INFINITY);
        st_agent(p.part_l + o, 0.f);
      }
      continue;
    }
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = fast_exp2(ws.m[w][r] - mm);  // empty wave: exp2(-inf) = 0
      a += f * ws.acc[w][r][d];
      l += f * ws.l[w][r];
    }
    st_agent(p.part_acc + o * D + d, a);
    if (d == 0) {
      st_agent(p.part_m + o, mm);
      st_agent(p.part_l + o, l);
    }
  }
}

// One online-softmax step for U key slots of one row: s[u] scores (-inf = masked),
// vals[u][8] this lane's 8 V elements of each slot.
template <int LPR, int U>
__device__ __forceinline__ void online_step(float (&s)[U], const float (&vals)[U][8], float &m,
                                            float &l, float (&acc)[8]) {
  float tmax = s[0];
#pragma unroll
  for (int u = 1; u < U; ++u) tmax = fmaxf(tmax, s[u]);
  tmax = max_slots<LPR>(tmax);
  const float mnew = fmaxf(m, tmax);
  const float alpha = fast_exp2(m - mnew);
  l *= alpha;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= alpha;
  m = mnew;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float pe = fast_exp2(s[u] - mnew);
    l += pe;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(pe, vals[u][e], acc[e]);
  }
}

template <int D, int R, int U>
__global__ __launch_bounds__(256) void partial_fp16_kernel(PartialParams p) {
  constexpr int LPR = D / 8, KPI = 64 / LPR, STEP = KPI * U;
  __shared__ WaveScratch<D, R> sm;
  WaveState<D, R> &ws = sm.ws;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, kk = lane / LPR;
  const int x = blockIdx.x + p.x_begin, y = blockIdx.y;
  const int hg = y / p.M, qi = y - hg * p.M;
  const int g = p.rg.g[hg], cnt = p.rg.cnt[hg];
  const uint8_t *heads = p.rg.heads[hg];
  Span sp = get_span(p, x, g, qi);
  if (!sp.suffix && p.kv.fmt != 0) sp.j1 = sp.j0;  // this kernel reads fp16 only
  const uint16_t *Kbase, *Vbase;
  if (sp.suffix) {
    Kbase = p.Ksuf + (size_t)g * p.S_suf * D;
    Vbase = p.Vsuf + (size_t)g * p.S_suf * D;
  } else {
    Kbase = p.kv.K + (size_t)g * p.kv.N * D;
    Vbase = p.kv.V + (size_t)g * p.kv.N * D;
  }

  h2_t q[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = heads[r < cnt ? r : 0];
    const uint4 qq = *(const uint4 *)(p.Q + ((size_t)h * p.M + qi) * D + sub * 8);
    q[r][0] = as_h2(qq.x);
    q[r][1] = as_h2(qq.y);
    q[r][2] = as_h2(qq.z);
    q[r][3] = as_h2(qq.w);
  }
  float m[R], l[R], acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  for (int base = sp.j0 + wave * STEP; base < sp.j1; base += 4 * STEP) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * KPI + kk;
      ok[u] = j < sp.j1;
      if (ok[u]) {
        kr[u] = *(const uint4 *)(Kbase + (size_t)j * D + sub * 8);
        vr[u] = *(const uint4 *)(Vbase + (size_t)j * D + sub * 8);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float vals[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w4[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        vals[u][2 * c] = h2f((uint16_t)(w4[c] & 0xffff));
        vals[u][2 * c + 1] = h2f((uint16_t)(w4[c] >> 16));
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float d = __builtin_amdgcn_fdot2(q[r][0], as_h2(kr[u].x), 0.f, false);
        d = __builtin_amdgcn_fdot2(q[r][1], as_h2(kr[u].y), d, false);
        d = __builtin_amdgcn_fdot2(q[r][2], as_h2(kr[u].z), d, false);
        d = __builtin_amdgcn_fdot2(q[r][3], as_h2(kr[u].w), d, false);
        d = sum_lanes<LPR>(d);
        s[u] = ok[u] ? d * p.qscale : -INFINITY;
      }
      online_step<LPR, U>(s, vals, m[r], l[r], acc[r]);
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    l[r] = sum_slots<LPR>(l[r]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = sum_slots<LPR>(acc[r][e]);
    if (kk == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ws.acc[wave][r][sub * 8 + e] = acc[r][e];
    }
    if (lane == 0) {
      ws.m[wave][r] = m[r];
      ws.l[wave][r] = l[r];
    }
  }
  __syncthreads();
  finish<D, R>(p, sm, heads, cnt, qi, x, y);
}

// mlx4g32 prefix (the suffix, when present, is fp16 and handled by the fp16 kernel
// launched for the suffix spans only).
template <int D, int R, int U>
__global__ __launch_bounds__(256) void partial_mlx4_kernel(PartialParams p) {
  constexpr int LPR = D / 8, KPI = 64 / LPR, STEP = KPI * U, NG = D / 32;
  __shared__ WaveScratch<D, R> sm;
  WaveState<D, R> &ws = sm.ws;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, kk = lane / LPR;
  const int grp = sub >> 2;  // this lane's 8 elements lie in group sub/4
  const int x = blockIdx.x + p.x_begin, y = blockIdx.y;
  const int hg = y / p.M, qi = y - hg * p.M;
  const int g = p.rg.g[hg], cnt = p.rg.cnt[hg];
  const uint8_t *heads = p.rg.heads[hg];
  Span sp = get_span(p, x, g, qi);
  if (sp.suffix) sp.j1 = sp.j0;  // this kernel reads the mlx4g32 prefix only

  const size_t tok0 = (size_t)g * p.kv.N;
  const uint32_t *Kc = p.kv.Kc + tok0 * (D / 8);
  const uint32_t *Vc = p.kv.Vc + tok0 * (D / 8);
  const uint16_t *Ks = p.kv.Ks + tok0 * NG, *Kb = p.kv.Kb + tok0 * NG;
  const uint16_t *Vs = p.kv.Vs + tok0 * NG, *Vb = p.kv.Vb + tok0 * NG;

  // q pairs in nibble order: word element k sits at bits 4k, so (w >> 4k) & 0x000F000F
  // yields elements (k, k+4) as two 16-bit integers.
  h2_t q[R][4];
  float qsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = heads[r < cnt ? r : 0];
    const uint4 qq = *(const uint4 *)(p.Q + ((size_t)h * p.M + qi) * D + sub * 8);
    const uint16_t *qe = (const uint16_t *)&qq;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h2_t t;
      t.x = __builtin_bit_cast(_Float16, qe[k]);
      t.y = __builtin_bit_cast(_Float16, qe[k + 4]);
      q[r][k] = t;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s += h2f(qe[e]);
    qsum[r] = s;
  }
  float m[R], l[R], acc[R][8], bsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
    bsum[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }
  const h2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};

  for (int base = sp.j0 + wave * STEP; base < sp.j1; base += 4 * STEP) {
    uint32_t kw[U], vw[U];
    float ks[U], kb[U], vs[U], vb[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * KPI + kk;
      ok[u] = j < sp.j1;
      const int jj = ok[u] ? j : sp.j0;  // in-bounds stand-in, masked below
      kw[u] = Kc[(size_t)jj * (D / 8) + sub];
      vw[u] = Vc[(size_t)jj * (D / 8) + sub];
      ks[u] = h2f(Ks[(size_t)jj * NG + grp]);
      kb[u] = h2f(Kb[(size_t)jj * NG + grp]);
      vs[u] = h2f(Vs[(size_t)jj * NG + grp]);
      vb[u] = h2f(Vb[(size_t)jj * NG + grp]);
    }
    // dequantized V elements of this lane (without the bias; the bias is accumulated
    // separately per row as p * b)
    float vals[U][8];
    h2_t kc[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) vals[u][e] = (float)((vw[u] >> (4 * e)) & 0xFu) * vs[u];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        kc[u][k] = as_h2(((kw[u] >> (4 * k)) & 0x000F000Fu) | 0x64006400u) - k1024;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float d = __builtin_amdgcn_fdot2(q[r][0], kc[u][0], 0.f, false);
        d = __builtin_amdgcn_fdot2(q[r][1], kc[u][1], d, false);
        d = __builtin_amdgcn_fdot2(q[r][2], kc[u][2], d, false);
        d = __builtin_amdgcn_fdot2(q[r][3], kc[u][3], d, false);
        d = __builtin_fmaf(ks[u], d, kb[u] * qsum[r]);
        d = sum_lanes<LPR>(d);
        s[u] = ok[u] ? d * p.qscale : -INFINITY;
      }
      // online step with the bias term carried in bsum
      float tmax = s[0];
#pragma unroll
      for (int u = 1; u < U; ++u) tmax = fmaxf(tmax, s[u]);
      tmax = max_slots<LPR>(tmax);
      const float mnew = fmaxf(m[r], tmax);
      const float alpha = fast_exp2(m[r] - mnew);
      l[r] *= alpha;
      bsum[r] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
      m[r] = mnew;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pe = fast_exp2(s[u] - mnew);
        l[r] += pe;
        bsum[r] = __builtin_fmaf(pe, vb[u], bsum[r]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = __builtin_fmaf(pe, vals[u][e], acc[r][e]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    l[r] = sum_slots<LPR>(l[r]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = sum_slots<LPR>(acc[r][e] + bsum[r]);
    if (kk == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ws.acc[wave][r][sub * 8 + e] = acc[r][e];
    }
    if (lane == 0) {
      ws.m[wave][r] = m[r];
      ws.l[wave][r] = l[r];
    }
  }
  __syncthreads();
  finish<D, R>(p, sm, heads, cnt, qi, x, y);
}

// Merge the S_total partials of this workgroup's rows into out / lse. Runs in the one
// workgroup of the row group that took the last ticket. `w` is LDS scratch of
// kMaxSplits floats, `red` of 8 floats.
__device__ __forceinline__ void merge_rows(const PartialParams &p, const uint8_t *heads, int cnt,
                                           int qi, int D, float *w, float *red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r = 0; r < cnt; ++r) {
    const int row = heads[r] * p.M + qi;
    const float *pm = p.part_m + (size_t)row * p.S_total;
    const float *pl = p.part_l + (size_t)row * p.S_total;
    float mx = -INFINITY;
    for (int c = tid; c < p.S_total; c += 256) mx = fmaxf(mx, ld_agent(pm + c));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float L = 0.f;
    for (int c = tid; c < p.S_total; c += 256) {
      const float mc = ld_agent(pm + c);
      const float f = (mc == -INFINITY) ? 0.f : fast_exp2(mc - mx);
      w[c] = f;
      L += f * ld_agent(pl + c);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o);
    if (lane == 0) red[4 + wave] = L;
    __syncthreads();
    L = red[4] + red[5] + red[6] + red[7];
    const float *pa = p.part_acc + (size_t)row * p.S_total * D;
    for (int d = tid; d < D; d += 256) {
      float o = 0.f;
      for (int c = 0; c < p.S_total; ++c) o = __builtin_fmaf(w[c], ld_agent(pa + (size_t)c * D + d), o);
      p.out[(size_t)row * D + d] = o / L;
    }
    if (tid == 0 && p.lse) p.lse[row] = (mx + __log2f(L)) * 0.69314718055994530942f;
    __syncthreads();
  }
}

// Store this workgroup's partial, take a ticket, and merge if it is the last span.
template <int D, int R>
__device__ __forceinline__ void finish(const PartialParams &p, WaveScratch<D, R> &sm,
                                       const uint8_t *heads, int cnt, int qi, int x, int y) {
  store_partial<D, R>(p, sm.ws, heads, cnt, qi, x);
  // this wave's partial stores have completed before the barrier and the ticket
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int t = __hip_atomic_fetch_add(p.counters + y, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    sm.last = (t == p.S_total - 1);
  }
  __syncthreads();
  if (!sm.last) return;
  merge_rows(p, heads, cnt, qi, D, sm.w, sm.red);
  if (threadIdx.x == 0)
    __hip_atomic_store(p.counters + y, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int R>
hipError_t launch_partial_d(const PartialParams &p, int y_groups, int x_count, bool mlx4,
                            hipStream_t s) {
  dim3 grid(x_count, y_groups);
  if (mlx4) {
    constexpr int U = (D == 256) ? 2 : 4;
    hipLaunchKernelGGL((partial_mlx4_kernel<D, R, U>), grid, dim3(256), 0, s, p);
  } else {
    constexpr int U = 4;
    hipLaunchKernelGGL((partial_fp16_kernel<D, R, U>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_partial_r(const PartialParams &p, int R, int y, int xc, bool mlx4,
                            hipStream_t s) {
  switch (R) {
    case 1: return launch_partial_d<D, 1>(p, y, xc, mlx4, s);
    case 2: return launch_partial_d<D, 2>(p, y, xc, mlx4, s);
    case 4: return launch_partial_d<D, 4>(p, y, xc, mlx4, s);
    default: return launch_partial_d<D, 8>(p, y, xc, mlx4, s);
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

hipError_t launch_partial(const PartialParams &p, int rows_per_group, int y_groups,
                          int x_count, bool mlx4_prefix, hipStream_t s) {
  if (x_count < 1 || y_groups < 1) return hipSuccess;
  switch (p.kv.D) {
    case 64: return launch_partial_r<64>(p, rows_per_group, y_groups, x_count, mlx4_prefix, s);
    case 128: return launch_partial_r<128>(p, rows_per_group, y_groups, x_count, mlx4_prefix, s);
    case 256: return launch_partial_r<256>(p, rows_per_group, y_groups, x_count, mlx4_prefix, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pion
