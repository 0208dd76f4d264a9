// Grouped-query M = 1 attention over an fp16 prefix (dense chunks or selected blocks)
// and an fp16 suffix on fp16 MFMA: the q-heads that share a kv-head are the rows of the
// products, so one read of a key feeds all of them (the QUERY and QUERY_SPARSE_AUTO
// forms of the ATTEND.* page with a GQA head map; "Shared KV Cache Serving", Stage 2).
// It computes what the split-KV VALU kernel computes (attn_partial.hip) and shares its
// problem, span and merge machinery (split_common.h); it serves row groups of 4 to 8
// q-heads, where the per-key VALU work of that kernel grows with the rows.
//
// Per workgroup: one span (a list of key segments) of one row group. The segments are
// cut into 32-key sub-tiles, dealt round-robin to the NW waves (4, or 2 at D = 256 for
// the LDS budget). Each wave stages its sub-tiles' K and V rows in its own LDS region
// (buffer loads that write LDS, rows XOR-swizzled by 16-byte chunk, two stages; the
// next sub-tile's loads are issued before the current one is consumed). Per sub-tile:
//   S^T = K Q^T   on v_mfma_f32_32x32x16_f16, A = 32 keys x 16 dims of K from LDS, B =
//                 Q^T (registers; the group's rows, zero past the group), lane l gets
//                 16 keys of row l % 32;
//   softmax       online, in log2 units, fp32, with a lazy rescale (kRescaleSlack);
//   O^T += V^T P^T  A = V^T read transposed from LDS (ds_read_b64_tr_b16), B = the fp16
//                 weights, already in the B layout.
// At the end the waves merge through LDS; a single-span problem writes out and lse, else
// the span stores its partial and the last span of the row group merges (ticket).
#include "attn_gqa.h"
#include "mfma_common.h"
#include "split_common.h"

namespace pion {
namespace {

constexpr int kSub = 32;  // keys per sub-tile

template <int D>
struct GqaSmem {
  static constexpr int NW = D == 256 ? 2 : 4;  // waves
  static constexpr int VB = kSub * 2 * D;      // bytes of one K or V sub-tile
  union {
    alignas(16) char kv[NW][2][2][VB];  // per wave: [stage][0: K, 1: V]
    struct {
      float m[NW][kGqaMaxRows], l[NW][kGqaMaxRows];
      alignas(16) float acc[NW][kGqaMaxRows][D];
    } wm;
  };
  int seg_j0[kGqaMaxSegs], seg_j1[kGqaMaxSegs], seg_cum[kGqaMaxSegs + 1];
  unsigned char seg_suf[kGqaMaxSegs];
  int last;
};

template <int D>
__global__ __launch_bounds__(64 * GqaSmem<D>::NW) void gqa_mfma_kernel(PartialParams p) {
  constexpr int NDB = D / 32, NDS = D / 16;
  constexpr uint32_t ROWB = D * 2;
  constexpr int NW = GqaSmem<D>::NW, NT = 64 * NW;
  constexpr int VB = GqaSmem<D>::VB;
  constexpr int NLV = VB / 1024;  // 1 KB LDS loads per K or V sub-tile
  constexpr int CH = D / 8;       // 16-byte chunks per row
  __shared__ GqaSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, col = lane & 31;
  const int z = blockIdx.z, y = blockIdx.y;
  int hg;
  Prob b;
  const Group gr = entry_group(p, z, y, hg, b);
  const int x = blockIdx.x + p.x_begin;
  if (x >= b.S_total) return;  // this problem has fewer spans than the grid
  const int qi = y - hg * p.M;
  const int g = gr.g, cnt = gr.cnt;

  // the span's segments: start key, suffix flag and cumulative sub-tile counts
  const int seg0 = x * p.seg_per_span, nseg = min(seg0 + p.seg_per_span, b.n_seg) - seg0;
  if (tid == 0) {
    int cum = 0;
    for (int s = 0; s < nseg; ++s) {
      const Span sp = get_segment(p, seg0 + s, b.pre_splits, b.N, g, qi);
      sm.seg_j0[s] = sp.j0;
      sm.seg_j1[s] = sp.j1;
      sm.seg_suf[s] = sp.suffix;
      sm.seg_cum[s] = cum;
      cum += sp.j1 > sp.j0 ? (sp.j1 - sp.j0 + kSub - 1) / kSub : 0;
    }
    sm.seg_cum[nseg] = cum;
  }
  __syncthreads();  // tid 0 wrote the table; every wave reads it
  const int n_sub = sm.seg_cum[nseg];

  const KVView kv = make_view(p.kv_base[z], 0, p.H_kv, b.N, D);
  const uint16_t *Kp = (const uint16_t *)kv.K + (size_t)g * b.N * D;
  const uint16_t *Vp = (const uint16_t *)kv.V + (size_t)g * b.N * D;
  const bool has_suf = p.S_suf > 0;
  const uint16_t *Ks = has_suf ? (const uint16_t *)p.Ksuf + (size_t)g * p.S_suf * D : Kp;
  const uint16_t *Vs = has_suf ? (const uint16_t *)p.Vsuf + (size_t)g * p.S_suf * D : Vp;
  const i32x4 wKp = rsrc_words(Kp, (uint32_t)b.N * ROWB), wVp = rsrc_words(Vp, (uint32_t)b.N * ROWB);
  const uint32_t suf_bytes = (uint32_t)(has_suf ? p.S_suf : 0) * ROWB;
  const i32x4 wKs = rsrc_words(Ks, suf_bytes), wVs = rsrc_words(Vs, suf_bytes);

  // LDS lane offsets: sub-tile loads (row r, physical chunk lane % CH holding logical
  // chunk (lane % CH) ^ swz(r)), K operand reads (row col, logical chunk 2 ds + hl) and
  // the transposed V reads
  uint32_t dv[NLV];
#pragma unroll
  for (int t = 0; t < NLV; ++t) {
    const int r = (1024 * t + 16 * lane) / (int)ROWB;
    dv[t] = (uint32_t)r * ROWB + (uint32_t)(((lane % CH) ^ swz<D>(r)) << 4);
  }
  uint32_t koff[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds)
    koff[ds] = (uint32_t)col * ROWB + (uint32_t)(((2 * ds + hl) ^ swz<D>(col)) << 4);
  uint32_t voffs[2][NDB];
  vt_offsets<D>(lane, voffs);
  const char *wbase = &sm.kv[wave][0][0][0];
  const uint32_t lds_w = (uint32_t)(uintptr_t)LDS_PTR(char, wbase);

  // sub-tile k of the span: its first key, valid keys and source
  struct Sub {
    int j, len;
    bool suf;
  };
  auto locate = [&](int k) {
    int s = 0;
    while (sm.seg_cum[s + 1] <= k) ++s;
    Sub u;
    u.j = sm.seg_j0[s] + kSub * (k - sm.seg_cum[s]);
    u.len = min(kSub, sm.seg_j1[s] - u.j);
    u.suf = sm.seg_suf[s];
    return u;
  };
  auto issue = [&](const Sub &u, int stage) {
    const i32x4 wk = u.suf ? wKs : wKp, wv = u.suf ? wVs : wVp;
    const uint32_t st = lds_w + (uint32_t)(stage * 2 * VB);
#pragma unroll
    for (int t = 0; t < NLV; ++t) {
      load_lds16(wk, (uint32_t)u.j * ROWB + dv[t], st + 1024 * t);
      load_lds16(wv, (uint32_t)u.j * ROWB + dv[t], st + VB + 1024 * t);
    }
  };

  f16v o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = kNegBig, l_run = 0.f;

  int k = wave, stage = 0;
  Sub cur;
  if (k < n_sub) {  // the first sub-tile's loads overlap the Q loads
    cur = locate(k);
    issue(cur, 0);
  }
  // Q^T operand: row col is q-head gr.head(col) (zero past the group)
  half8 qb[NDS];
  {
    const bool live = col < cnt;
    const uint16_t *qrow = (const uint16_t *)b.Q + ((size_t)gr.head(live ? col : 0) * p.M + qi) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const half8 v = *(const half8 *)(qrow + 16 * ds + 8 * hl);
      qb[ds] = live ? v : half8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // Q and the first sub-tile have arrived: no load of the compiler's own is outstanding
  // in the loop, where a vmcnt wait it added would also drain the next sub-tile's loads
  __builtin_amdgcn_s_waitcnt(0);
  while (k < n_sub) {
    const int kn = k + NW;
    Sub nxt;
    if (kn < n_sub) {
      nxt = locate(kn);
      issue(nxt, stage ^ 1);
      // this sub-tile's loads are done; the next one's (2 NLV) may stay in flight
      __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NLV) : "memory");
    } else {
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const char *kst = wbase + stage * 2 * VB, *vst = kst + VB;
    // S^T: 32 keys x 32 rows; lane l holds keys 8 i + 4 hl + jj of row l % 32
    f16v s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      s = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          __builtin_bit_cast(half8, *(const uint4 *)(kst + koff[ds])), qb[ds], s, 0, 0, 0);
    if (cur.len < kSub) {  // wave-uniform: keys past the segment end
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (8 * i + 4 * hl + jj >= cur.len) s[4 * i + jj] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s[e]);
    mt = max_xor32(mt) * p.qscale;
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
      pb[e >> 3][e & 7] = (_Float16)pf;  // at most 2^kRescaleSlack
    }
    // O^T += V^T P^T over the two 16-key k-steps
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      half8 vf[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) vf[db] = vt_frag<D>(vst + 16 * s2 * (int)ROWB, voffs, db);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[db], pb[s2], o[db], 0, 0, 0);
    }
    if (kn >= n_sub) break;
    cur = nxt;
    k = kn;
    stage ^= 1;
  }
  l_run = sum_xor32(l_run);

  // merge the waves' rows through LDS (the stages are done with)
  __syncthreads();
  if (col < cnt) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(f32x4 *)&sm.wm.acc[wave][col][32 * db + 8 * i + 4 * hl] =
            f32x4{o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]};
    if (hl == 0) {
      sm.wm.m[wave][col] = m_run;
      sm.wm.l[wave][col] = l_run;
    }
  }
  __syncthreads();
  const PartRsrc pr = part_rsrc(p, b, qi);
  constexpr int DQ = D / 4;
  for (int t = tid; t < cnt * DQ; t += NT) {
    const int r = t / DQ, dq = t - r * DQ;
    float mm = sm.wm.m[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) mm = fmaxf(mm, sm.wm.m[w][r]);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    float lw = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm.wm.m[w][r] - mm);
      a += f * *(const f32x4 *)&sm.wm.acc[w][r][4 * dq];
      lw = __builtin_fmaf(f, sm.wm.l[w][r], lw);
    }
    if (b.S_total == 1) {  // the only span of its rows: final output, no merge
      const size_t row = (size_t)gr.head(r) * p.M + qi;
      const float inv = 1.f / lw;
      *(float4 *)(b.out + row * D + 4 * dq) = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
      if (dq == 0 && b.lse) b.lse[row] = (mm + __log2f(lw)) * 0.69314718055994530942f;
    } else {
      store_part(pr, gr.head(r), x, dq, a);
      if (dq == 0) store_ml(pr, gr.head(r), x, lw > 0.f ? mm : -INFINITY, lw);  // empty: weight 0
    }
  }
  if (b.S_total > 1) ticket_and_merge<D, NT>(p, b, pr, gr, qi, sm.last);
}

template <int D>
hipError_t launch_d(const PartialParams &p, int x_count, hipStream_t s) {
  dim3 grid(x_count, p.y_groups, p.n_prob);
  note_launch("gqa_mfma_kernel<%d>", D);
  hipLaunchKernelGGL(gqa_mfma_kernel<D>, grid, dim3(64 * GqaSmem<D>::NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gqa_mfma(const PartialParams &p, int x_count, hipStream_t s) {
  if (x_count < 1 || p.y_groups < 1 || p.n_prob < 1) return hipSuccess;
  if (p.S_max > kMaxSplits || p.n_prob > kMaxBatch || p.fmt != 0 || p.M != 1 ||
      p.seg_per_span > kGqaMaxSegs)
    return hipErrorInvalidValue;
  switch (p.D) {
    case 64: return launch_d<64>(p, x_count, s);
    case 128: return launch_d<128>(p, x_count, s);
    case 256: return launch_d<256>(p, x_count, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pion
