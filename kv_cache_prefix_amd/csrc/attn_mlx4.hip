// Split-over-keys attention over an mlx4g32 prefix (VALU path), with the split merge
// done in-kernel as for the fp16 kernel (split_common.h). The dequantized keys and
// values are those of the mlx4g32 tier ("Shared KV Cache Serving", Quantized tier -
// mlx4g32): element e of group g of token j is s_jg * c_je + b_jg, with fp16 scale s
// and bias b, integer code c in [0, 15].
//
// Layout. A key row of D elements is NG = D/32 groups, read by NGP lanes (NG rounded up
// to a power of two; for D = 96, 160, 192 the lanes past NG hold no group and load
// nothing); lane (slot kk, group g) owns group g of its keys. It reads the group's 16
// code bytes and its 4-byte (scale, bias) pair per key and side, so dequantization
// needs no other lane's data. A wave covers KPW = 64/NGP keys per load instruction;
// each lane takes U keys per tile (keys base + u*KPW + kk), and the next tile is loaded
// before the current one is consumed.
//
// Arithmetic, per row (q-head) and key j:
//   q . k_j = sum_g  s_jg (q_g . c_jg) + b_jg sum(q_g)
//   sum_j p_j v_j = sum_j (p_j s_jg) c_jg + sum_j p_j b_jg       (per group g)
// Codes become fp16 operands with a mask only: a nibble in bits 0..3 of an fp16 is the
// subnormal c * 2^-24, a nibble in bits 4..7 the subnormal c * 2^-20 (both exact).
// Of a code word, the masks 0x000F000F / 0x00F000F0 on the word and on the word >> 8
// give the element pairs (0,4), (1,5), (2,6), (3,7). q . c runs on v_dot2_f32_f16 with
// fp16 q and fp32 sums; the q pairs meeting high nibbles are scaled by 1/16 so that one
// sum holds every product in units of 2^-24 (exact unless |q| < 2^-10, where the scaled
// value is rounded to the fp16 subnormal grid: an error below 2^-25 |c|). The value side
// pairs two keys per v_dot2_f32_f16: byte k of the code words of keys a, b goes to the
// low bytes of the two halves by one byte permute, and the masks give elements 2k and
// 2k + 1 of both keys; the weights are fp16 (p_a s_a, p_b s_b), rounded to nearest. Odd
// elements accumulate in units of 2^-20, even ones in 2^-24; the scale back is exact.
//
// Online softmax per key slot with a lazy rescale: the running reference m moves only
// when a tile's max exceeds it by more than kSlack (log2 units), so p <= 2^kSlack and
// p * s stays within fp16 range for any fp16 scale (s <= 131008 / 15).
//
// End of span: the slots of each 16-lane row merge with DPP row rotations (for D = 512
// also the 4 rows of a wave, by the lane swaps, so that the LDS partials fit), the row
// (or wave) partials of the workgroup merge through LDS, and the workgroup stores its
// partial, takes its ticket, and the last one merges the row group.
#include "split_common.h"

namespace pion {
namespace {

constexpr float kSlack = 2.0f;
constexpr uint32_t kLo4 = 0x000F000Fu;  // nibble 0 of each half
constexpr uint32_t kHi4 = 0x00F000F0u;  // nibble 1 of each half

// Sum over each group of W consecutive lanes (W = 1 .. 16): quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row half-mirror (which pairs the two quads of 8 lanes), row
// mirror (the two halves of 16).
template <int W>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (W >= 2) v += dpp<0xB1>(v);
  if constexpr (W >= 4) v += dpp<0x4E>(v);
  if constexpr (W >= 8) v += dpp<0x141>(v);
  if constexpr (W >= 16) v += dpp<0x140>(v);
  return v;
}

// The max / sum of lanes l and l ^ 16 (by32: l ^ 32) in every lane, by the row swaps.
__device__ __forceinline__ float swap_max(float v, bool by32) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = by32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                      : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float swap_sum(float v, bool by32) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = by32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                      : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Combine the lanes that are NGP apart (the slots holding the same group): row
// rotations by NGP, 2 NGP, ..., 8 inside each 16-lane row; with WAVE also the two row
// swaps, so that every lane of the wave holds the wave's result.
template <int NGP, bool WAVE>
__device__ __forceinline__ float slots_max(float v) {
  if constexpr (NGP <= 1) v = fmaxf(v, dpp<0x121>(v));
  if constexpr (NGP <= 2) v = fmaxf(v, dpp<0x122>(v));
  if constexpr (NGP <= 4) v = fmaxf(v, dpp<0x124>(v));
  if constexpr (NGP <= 8) v = fmaxf(v, dpp<0x128>(v));
  if constexpr (WAVE) v = swap_max(swap_max(v, false), true);
  return v;
}
template <int NGP, bool WAVE>
__device__ __forceinline__ float slots_sum(float v) {
  if constexpr (NGP <= 1) v += dpp<0x121>(v);
  if constexpr (NGP <= 2) v += dpp<0x122>(v);
  if constexpr (NGP <= 4) v += dpp<0x124>(v);
  if constexpr (NGP <= 8) v += dpp<0x128>(v);
  if constexpr (WAVE) v = swap_sum(swap_sum(v, false), true);
  return v;
}

// Row (16-lane) partials of a workgroup of NW waves, or wave partials for D = 512.
template <int D, int R, int NW>
struct Mlx4Scratch {
  static constexpr bool kWave = D >= 512;
  static constexpr int kParts = kWave ? NW : 4 * NW;
  float m[kParts][R], l[kParts][R];
  union {
    alignas(16) float acc[kParts][R][D];
  };
  int last;
};

template <int U>
struct Mlx4Tile {
  uint4 kc[U], vc[U];
  uint32_t ksb[U], vsb[U];
};

// a.x*b.x + a.y*b.y with a zero accumulator operand (the three-operand encoding; the
// accumulating two-operand form the compiler prefers needs a zeroed register first)
__device__ __forceinline__ float dot2_first(h2_t a, h2_t b) {
  float d;
  __asm__("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

__device__ __forceinline__ float lo_f(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float hi_f(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

template <int D, int R, int U, int NW>
__global__ __launch_bounds__(64 * NW) void mlx4_split_kernel(PartialParams p) {
  constexpr int NG = D / 32, NGP = pow2_ceil(NG), KPW = 64 / NGP, STEP = KPW * U, NT = 64 * NW;
  static_assert(U % 2 == 0, "keys are consumed in pairs");
  __shared__ Mlx4Scratch<D, R, NW> sm;
  constexpr int kParts = Mlx4Scratch<D, R, NW>::kParts;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane % NGP, kk = lane / NGP;
  const bool grp = g < NG;  // this lane owns a group of its keys
  const int z = blockIdx.z, y = blockIdx.y;
  int hg;
  Prob b;
  const Group gr = entry_group(p, z, y, hg, b);
  const int x = blockIdx.x + p.x_begin;
  if (x >= b.S_total) return;  // this problem has fewer spans than the grid
  const int qi = y - hg * p.M;
  const int gk = gr.g, cnt = gr.cnt;
  Span sp = get_segment(p, x, b.pre_splits, b.N, gk, qi);  // one segment per span here
  if (sp.suffix) sp.j1 = sp.j0;  // suffix spans belong to the fp16 kernel

  // this kv-head's codes and (scale, bias) pairs as buffer ranges: keys past the span
  // are masked in consume, keys past N read zero
  const KVView kv = make_view(p.kv_base[z], p.fmt, p.H_kv, b.N, D);
  const size_t t0 = (size_t)gk * b.N;
  const __amdgpu_buffer_rsrc_t rKc = make_rsrc(kv.Kc + t0 * (D / 8), (uint32_t)b.N * (D / 2));
  const __amdgpu_buffer_rsrc_t rVc = make_rsrc(kv.Vc + t0 * (D / 8), (uint32_t)b.N * (D / 2));
  const __amdgpu_buffer_rsrc_t rKsb = make_rsrc(kv.Ksb + t0 * NG, (uint32_t)b.N * NG * 4);
  const __amdgpu_buffer_rsrc_t rVsb = make_rsrc(kv.Vsb + t0 * NG, (uint32_t)b.N * NG * 4);

  auto load = [&](Mlx4Tile<U> &t, int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t e = (uint32_t)(base + u * KPW + kk) * NG + g;  // (key, group) index
      if (grp) {
        t.kc[u] = bload_stream16(rKc, e * 16);
        t.vc[u] = bload_stream16(rVc, e * 16);
        t.ksb[u] = bload_stream4(rKsb, e * 4);
        t.vsb[u] = bload_stream4(rVsb, e * 4);
      } else {  // no group: zero codes, scale and bias
        t.kc[u] = t.vc[u] = make_uint4(0, 0, 0, 0);
        t.ksb[u] = t.vsb[u] = 0;
      }
    }
  };

  // the first tile is in flight while q is read
  int base = sp.j0 + wave * STEP;
  Mlx4Tile<U> cur;
  if (base < sp.j1) load(cur, base);

  // q of each row: group g's 32 halves as the pairs (8w+k, 8w+k+4) that the code masks
  // produce, and qsum * qscale for the bias term
  h2_t q[R][16];
  float qsq[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = gr.head(r < cnt ? r : 0);
    const uint4 *qp =
        (const uint4 *)((const uint16_t *)b.Q + ((size_t)h * p.M + qi) * D + 32 * (grp ? g : 0));
    float qs = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint4 qq = grp ? qp[w] : make_uint4(0, 0, 0, 0);
      const uint32_t u4[4] = {qq.x, qq.y, qq.z, qq.w};
      uint16_t e[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        e[2 * c] = (uint16_t)(u4[c] & 0xffffu);
        e[2 * c + 1] = (uint16_t)(u4[c] >> 16);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // pairs k = 1, 3 meet the high nibbles (codes in units of 2^-20): scaled by 1/16
        // so that every product lands in units of 2^-24 and one sum takes them all
        const _Float16 f = (k & 1) ? (_Float16)0.0625f : (_Float16)1.0f;
        h2_t t;
        t.x = __builtin_bit_cast(_Float16, e[k]) * f;
        t.y = __builtin_bit_cast(_Float16, e[k + 4]) * f;
        q[r][4 * w + k] = t;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) qs += h2f(e[k]);
    }
    qsq[r] = qs * p.qscale;
  }
  const float kq = 16777216.0f * p.qscale;  // 2^24: code units of the even pairs

  float m[R], l[R], bs[R], acc[R][32];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegBig;
    l[r] = 0.f;
    bs[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[r][e] = 0.f;
  }

  // keys past the span end (in its last tile) get -inf
  auto consume = [&](const Mlx4Tile<U> &t, int base) {
    float s[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float ks = lo_f(t.ksb[u]) * kq, kb = hi_f(t.ksb[u]);
      const uint32_t w4[4] = {t.kc[u].x, t.kc[u].y, t.kc[u].z, t.kc[u].w};
      float dot[R];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x0 = w4[w], x8 = w4[w] >> 8;
        const h2_t c0 = as_h2(x0 & kLo4), c1 = as_h2(x0 & kHi4);
        const h2_t c2 = as_h2(x8 & kLo4), c3 = as_h2(x8 & kHi4);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          dot[r] = w == 0 ? dot2_first(q[r][0], c0)
                          : __builtin_amdgcn_fdot2(q[r][4 * w + 0], c0, dot[r], false);
          dot[r] = __builtin_amdgcn_fdot2(q[r][4 * w + 1], c1, dot[r], false);
          dot[r] = __builtin_amdgcn_fdot2(q[r][4 * w + 2], c2, dot[r], false);
          dot[r] = __builtin_amdgcn_fdot2(q[r][4 * w + 3], c3, dot[r], false);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
        s[u][r] = lane_group_sum<NGP>(__builtin_fmaf(ks, dot[r], kb * qsq[r]));
    }
    // keys past the span end (its last tile only: a wave-uniform test) get -inf
    if (base + U * KPW > sp.j1) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = base + u * KPW + kk < sp.j1;
#pragma unroll
        for (int r = 0; r < R; ++r) s[u][r] = ok ? s[u][r] : -INFINITY;
      }
    }

    h2_t P[R][U / 2];
    float mx[R];
    bool grow = false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      mx[r] = s[0][r];
#pragma unroll
      for (int u = 1; u < U; ++u) mx[r] = fmaxf(mx[r], s[u][r]);
      grow |= mx[r] > m[r] + kSlack;
    }
    if (grow) {  // rare after a slot's first tile: rescale the rows whose max moved
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool gr = mx[r] > m[r] + kSlack;
        const float nm = gr ? mx[r] : m[r];
        const float a = fast_exp2(m[r] - nm);
        l[r] *= a;
        bs[r] *= a;
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[r][e] *= a;
        m[r] = nm;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float pw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pe = fast_exp2(s[u][r] - m[r]);  // masked: 2^-inf = 0
        l[r] += pe;
        bs[r] = __builtin_fmaf(pe, hi_f(t.vsb[u]), bs[r]);
        pw[u] = pe * lo_f(t.vsb[u]);
      }
#pragma unroll
      for (int i = 0; i < U / 2; ++i) {
        h2_t ph;
        ph.x = (_Float16)pw[2 * i];
        ph.y = (_Float16)pw[2 * i + 1];
        P[r][i] = ph;
      }
    }

#pragma unroll
    for (int i = 0; i < U / 2; ++i) {
      const uint32_t a4[4] = {t.vc[2 * i].x, t.vc[2 * i].y, t.vc[2 * i].z, t.vc[2 * i].w};
      const uint32_t b4[4] = {t.vc[2 * i + 1].x, t.vc[2 * i + 1].y, t.vc[2 * i + 1].z,
                              t.vc[2 * i + 1].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // byte k of both keys' words (elements 2k, 2k+1) into the low bytes of the two
        // halves: v_perm_b32 takes bytes 0-3 from its second operand, 4-7 from its
        // first, and 0x0C is a zero byte
        h2_t c[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t xk =
              __builtin_amdgcn_perm(b4[w], a4[w], 0x0C000C00u | ((4u + k) << 16) | (uint32_t)k);
          c[2 * k] = as_h2(xk & kLo4);
          c[2 * k + 1] = as_h2(xk & kHi4);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[r][8 * w + e] = __builtin_amdgcn_fdot2(P[r][i], c[e], acc[r][8 * w + e], false);
      }
    }
  };

  // two tiles alternate roles (no copy of the prefetched tile)
  Mlx4Tile<U> nxt;
  while (base < sp.j1) {
    int next = base + NW * STEP;
    if (next < sp.j1) load(nxt, next);
    consume(cur, base);
    base = next;
    if (base >= sp.j1) break;
    next = base + NW * STEP;
    if (next < sp.j1) load(cur, next);
    consume(nxt, base);
    base = next;
  }

  // back to value units, bias added; slots of the row (D = 512: of the wave) merged
  constexpr bool WAVE = Mlx4Scratch<D, R, NW>::kWave;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float M = slots_max<NGP, WAVE>(m[r]);
    const float f = fast_exp2(m[r] - M);
    l[r] = slots_sum<NGP, WAVE>(l[r] * f);
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float v = __builtin_fmaf(acc[r][e], (e & 1) ? 1048576.0f : 16777216.0f, bs[r]);
      acc[r][e] = slots_sum<NGP, WAVE>(v * f);
    }
    m[r] = M;
  }
  const int part = WAVE ? wave : wave * 4 + (lane >> 4);
  if ((WAVE ? lane : (lane & 15)) < NG) {  // slot 0's groups of the row (lane % 16 = g)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float4 *dst = (float4 *)&sm.acc[part][r][32 * g];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dst[e] = make_float4(acc[r][4 * e], acc[r][4 * e + 1], acc[r][4 * e + 2], acc[r][4 * e + 3]);
      if (g == 0) {
        sm.m[part][r] = m[r];
        sm.l[part][r] = l[r];
      }
    }
  }
  __syncthreads();
  const PartRsrc pr = part_rsrc(p, b, qi);
  constexpr int DQ = D / 4;
  for (int t = threadIdx.x; t < cnt * DQ; t += NT) {
    const int r = t / DQ, dq = t - r * DQ;
    float mm = sm.m[0][r];
#pragma unroll
    for (int q2 = 1; q2 < kParts; ++q2) mm = fmaxf(mm, sm.m[q2][r]);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    float lw = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < kParts; ++q2) {
      const float f = fast_exp2(sm.m[q2][r] - mm);
      lw = __builtin_fmaf(f, sm.l[q2][r], lw);
      a += f * *(const f32x4 *)&sm.acc[q2][r][4 * dq];
    }
    store_part(pr, gr.head(r), x, dq, a);
    if (dq == 0) store_ml(pr, gr.head(r), x, lw > 0.f ? mm : -INFINITY, lw);  // empty: weight 0
  }
  // (ticket_and_merge's barrier precedes any reuse of acc as merge scratch)
  ticket_and_merge<D, NT>(p, b, pr, gr, qi, sm.last);
}

// 8 waves per workgroup (two per SIMD: one wave alone issues VALU work at about half
// the SIMD's rate) where the registers allow it; 4 rows need 4 waves.
template <int D, int R>
hipError_t launch_mlx4_d(const PartialParams &p, int x_count, hipStream_t s) {
  constexpr int NW = R <= 3 ? 8 : 4;
  dim3 grid(x_count, p.y_groups, p.n_prob);
  note_launch("mlx4_split_kernel<%d,%d,2,%d>", D, R, NW);
  hipLaunchKernelGGL((mlx4_split_kernel<D, R, 2, NW>), grid, dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mlx4_r(const PartialParams &p, int R, int xc, hipStream_t s) {
  switch (R) {
    case 1: return launch_mlx4_d<D, 1>(p, xc, s);
    case 2: return launch_mlx4_d<D, 2>(p, xc, s);
    case 3: return launch_mlx4_d<D, 3>(p, xc, s);
    case 4: return launch_mlx4_d<D, 4>(p, xc, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_partial_mlx4(const PartialParams &p, int rows_per_group, int x_count,
                               hipStream_t s) {
  if (x_count < 1 || p.y_groups < 1 || p.n_prob < 1) return hipSuccess;
  if (p.S_max > kMaxSplits || p.n_prob > kMaxBatch) return hipErrorInvalidValue;
  if (rows_per_group < 1 || rows_per_group > kMlx4Rows) return hipErrorInvalidValue;
  switch (p.D) {
    case 32: return launch_mlx4_r<32>(p, rows_per_group, x_count, s);
    case 64: return launch_mlx4_r<64>(p, rows_per_group, x_count, s);
    case 96: return launch_mlx4_r<96>(p, rows_per_group, x_count, s);
    case 128: return launch_mlx4_r<128>(p, rows_per_group, x_count, s);
    case 160: return launch_mlx4_r<160>(p, rows_per_group, x_count, s);
    case 192: return launch_mlx4_r<192>(p, rows_per_group, x_count, s);
    case 256: return launch_mlx4_r<256>(p, rows_per_group, x_count, s);
    case 512: return launch_mlx4_r<512>(p, rows_per_group, x_count, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pion
