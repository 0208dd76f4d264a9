// Split-over-keys attention over an mlx4g32 prefix at head dim 128 on fp16 MFMA (the
// QUERY forms of the ATTEND.* page over the Quantized tier - mlx4g32 of "Shared KV
// Cache Serving": element e of group g of token j is s_jg * c_je + b_jg, fp16 scale s
// and bias b, integer code c in [0, 15]). It computes what mlx4_split_kernel computes
// (attn_mlx4.hip) and shares its problem, span and merge machinery (split_common.h);
// the products run on the matrix cores, so the per-key vector work no longer bounds
// the pass over the resident codes.
//
// Codes become fp16 operands by masking alone: a nibble in bits 0..3 of an fp16 is the
// subnormal c * 2^-24, one in bits 4..7 the subnormal c * 2^-20 (both exact). Of a
// 32-bit word of 8 nibbles, the masks 0x000F000F / 0x00F000F0 on the word and on the
// word >> 8 give nibble pairs (0,4), (1,5), (2,6), (3,7). Products of the 2^-24 and
// the 2^-20 operands accumulate apart and are scaled back exactly at the end.
//
// Per wave, tiles of 64 keys (a workgroup's waves take the span's tiles round-robin).
// Rows of the group (up to 4 q-heads) are r, lanes l = 16 kb + n.
//   S: for each 16-key sub-tile, v_mfma_f32_16x16x32_f16 with B = codes (lane (n, kb)
//      holds one 16-byte load: group kb of key n, whose four words feed four products)
//      and A = q, where product row 4 g + r holds q-row r on group g's k-slots and zero
//      elsewhere. Result lane (n, g) holds the four rows' partial dots of group g,
//      which it scales by s_g and offsets by b_g * sum(q_g) (exact nibble units), and
//      a reduce-scatter over the four lane rows (two cross-half swaps, one cross-row
//      swap) leaves lane (n, h) the score of key n for row h.
//   softmax: online per row, log2 units, fp32, a lazy rescale (the reference moves only
//      when a score exceeds it by more than kSlack); lane (n, h) forms the fp16 weights
//      p s_g of its key for the four groups g and accumulates p b_g.
//   O^T += V^T P'^T: A = V^T read from LDS with the 4-bit transpose read
//      (ds_read_b64_tr_b4: in each 16-lane group, lane i receives nibble i of the
//      8-byte pieces addressed by lanes 0..15, lane j's at bits 4j .. 4j+3), 16 keys of
//      one dim per lane; B = the weights, columns (h, g) = 4 h + g, written to LDS in
//      the k-slot order of the A operand and read back with ds_read_b64_tr_b16. Column
//      (h, g) of a 16-dim block is kept where the block lies in group g.
// Staging: a tile's V codes and both sides' (scale, bias) words go from HBM straight
// into the wave's LDS (buffer loads that write LDS, two stages), its K codes into
// registers (two sets); the next tile's loads are issued before the current tile is
// consumed, and the wave waits for all of them at the top of the next tile (no load
// the compiler issued is outstanding inside the loop body, so its own waits are
// satisfied). No barrier in the loop: each wave owns its LDS region.
// The wave partials (m, l, the weighted code sums and the bias sums) merge through LDS;
// the workgroup stores its partial and takes its ticket as the other split kernels do.
#include "mfma_common.h"
#include "split_common.h"

namespace pion {
namespace {

constexpr int kTile = 64;            // keys per wave tile
constexpr float kSlack = 2.0f;       // p <= 4, so p * s stays in fp16 range (s <= 131008 / 15)
constexpr uint32_t kLoNib = 0x000F000Fu, kHiNib = 0x00F000F0u;
constexpr int kVcBytes = kTile * 64;              // V codes of a tile (128 dims / 2)
constexpr int kSbBytes = kTile * 16;              // (scale, bias) words of a tile, 4 groups
constexpr int kStage = kVcBytes + 2 * kSbBytes;   // V codes, K words, V words
// fp16 weights [slot row][16 columns]: row r at 32 r + 128 (r / 8), so that the four
// 8-row groups one transposed read covers start on alternating bank halves
constexpr int kPwBytes = kTile * 32 + 8 * 128;
constexpr int kWaveBytes = 2 * kStage + kPwBytes;

template <int NW>
struct Mlx4MfmaSmem {
  union {
    alignas(16) char w[NW][kWaveBytes];
    struct {
      float m[NW][4], l[NW][4], bs[NW][4][4];
      alignas(16) float acc[NW][4][128];
    } wm;
  };
  int last;
};

__device__ __forceinline__ float swap_add32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float swap_add16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
// Max / sum over the 16 lanes of each row (row rotations by 1, 2, 4, 8).
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<0x121>(v));
  v = fmaxf(v, dpp<0x122>(v));
  v = fmaxf(v, dpp<0x124>(v));
  return fmaxf(v, dpp<0x128>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0x121>(v);
  v += dpp<0x122>(v);
  v += dpp<0x124>(v);
  return v + dpp<0x128>(v);
}
__device__ __forceinline__ float lo_h(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float hi_h(uint32_t w) { return h2f((uint16_t)(w >> 16)); }
// fp16(p * s) into the low (high) half of the result, s the fp16 in the low half of w:
// one v_fma_mix instruction (fp32 p, fp16 s, the product rounded once to fp16). mix_lo
// leaves the high half undefined, for a mix_hi to fill.
__device__ __forceinline__ uint32_t mix_lo(float p, uint32_t w) {
  uint32_t r;
  __asm__("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p), "v"(w));
  return r;
}
__device__ __forceinline__ uint32_t mix_hi(uint32_t r, float p, uint32_t w) {
  __asm__("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(r) : "v"(p), "v"(w));
  return r;
}
__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8, u32x4{a, b, c, d});
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void mlx4_mfma_kernel(PartialParams p) {
  constexpr int D = 128, NT = 64 * NW, STEP = NW * kTile;
  __shared__ Mlx4MfmaSmem<NW> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int n = lane & 15, hb = lane >> 4;
  const int z = blockIdx.z, y = blockIdx.y;
  int hg;
  Prob b;
  const Group gr = entry_group(p, z, y, hg, b);
  const int x = blockIdx.x + p.x_begin;
  if (x >= b.S_total) return;  // this problem has fewer spans than the grid
  const int qi = y - hg * p.M;
  const int gk = gr.g, cnt = gr.cnt;
  Span sp = get_segment(p, x, b.pre_splits, b.N, gk, qi);
  if (sp.suffix) sp.j1 = sp.j0;  // suffix spans belong to the fp16 kernel

  // this kv-head's codes and (scale, bias) words as buffer ranges: keys past N read zero
  const KVView kv = make_view(p.kv_base[z], p.fmt, p.H_kv, b.N, D);
  const size_t t0 = (size_t)gk * b.N;
  const uint32_t cbytes = (uint32_t)b.N * 64, sbytes = (uint32_t)b.N * 16;
  const __amdgpu_buffer_rsrc_t rKc = make_rsrc(kv.Kc + t0 * 16, cbytes);
  const i32x4 wVc = rsrc_words(kv.Vc + t0 * 16, cbytes);
  const i32x4 wKsb = rsrc_words(kv.Ksb + t0 * 4, sbytes);
  const i32x4 wVsb = rsrc_words(kv.Vsb + t0 * 4, sbytes);

  char *wl = &sm.w[wave][0];
  const uint32_t lds_w = (uint32_t)(uintptr_t)LDS_PTR(char, wl);
  // V-code staging: byte 16 lane of load i is tile row 16 i + lane / 4, physical 16-byte
  // chunk lane % 4, which holds logical chunk (lane % 4) ^ swizzle(row), swizzle(r) =
  // (r / 4) % 4 (the transposed reads of 16 rows then spread over all 16 bank quads)
  const uint32_t vdm =
      (uint32_t)(lane >> 2) * 64 + (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  auto issue = [&](int key0, int stage, uint4(&kc)[4]) {
    const uint32_t st = lds_w + (uint32_t)(stage * kStage);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      load_lds16(wVc, (uint32_t)key0 * 64 + 1024 * i + vdm, st + 1024 * i);
    load_lds16(wKsb, (uint32_t)(key0 + lane) * 16, st + kVcBytes);
    load_lds16(wVsb, (uint32_t)(key0 + lane) * 16, st + kVcBytes + kSbBytes);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      kc[q] = bload_stream16(rKc, (uint32_t)(key0 + 16 * q + n) * 64 + (uint32_t)hb * 16);
  };

  // the first tile is in flight while q is read
  int base = sp.j0 + wave * kTile;
  uint4 kc0[4], kc1[4];
  if (base < sp.j1) issue(base, 0, kc0);

  // A operands of S: lane (m, kb) holds product row m = 4 g + r on k-block kb, which is
  // q-row r on group kb's dims when g = kb (and zero otherwise), in the k-slot order
  // of the code operand: elements {0,4,2,6,8,12,10,14} (+16) of the low nibbles and
  // the same + 1 of the high nibbles
  half8 qa[4];
  {
    const int gq = n >> 2, rq = n & 3;
    const bool live = gq == hb && rq < cnt;
    const uint4 *qp = (const uint4 *)((const uint16_t *)b.Q +
                                      ((size_t)gr.head(live ? rq : 0) * p.M + qi) * D + 32 * hb);
    uint16_t e[32];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint4 v = live ? qp[w] : make_uint4(0, 0, 0, 0);
      const uint32_t u4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        e[8 * w + 2 * c] = (uint16_t)(u4[c] & 0xffffu);
        e[8 * w + 2 * c + 1] = (uint16_t)(u4[c] >> 16);
      }
    }
    constexpr int ord[8] = {0, 4, 2, 6, 8, 12, 10, 14};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      qa[0][t] = __builtin_bit_cast(_Float16, e[ord[t]]);
      qa[1][t] = __builtin_bit_cast(_Float16, e[16 + ord[t]]);
      qa[2][t] = __builtin_bit_cast(_Float16, e[ord[t] + 1]);
      qa[3][t] = __builtin_bit_cast(_Float16, e[17 + ord[t]]);
    }
  }
  // lane (n, g): qscale * sum(q_r) over group g, the bias term's factor
  float qsq[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool lr = r < cnt;
    const uint4 *qp = (const uint4 *)((const uint16_t *)b.Q +
                                      ((size_t)gr.head(lr ? r : 0) * p.M + qi) * D + 32 * hb);
    float qs = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint4 v = qp[w];
      const uint32_t u4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) qs += lo_h(u4[c]) + hi_h(u4[c]);
    }
    qsq[r] = lr ? qs * p.qscale : 0.f;
  }
  const float kq = 1048576.0f * p.qscale;  // 2^20: q . c = 2^20 (16 C_lo + C_hi)

  // per-lane LDS offsets: the weight slot of this lane's key in each sub-tile (key
  // 16 q + n goes to slot row (n & 1) * 32 + 8 q + t, t its place in 0,4,2,6,8,12,10,14),
  // the weight operand reads (rows (ks * 32 + 8 kb + 4 c + n / 4), column quad n % 4) and
  // the transposed V reads (tile row 16 kb + n, dims of block db)
  const int ev = n & 14;
  const int slot = ((ev >> 3) << 2) | (((ev >> 1) & 1) << 1) | ((ev >> 2) & 1);
  const uint32_t pw_w = (uint32_t)((n & 1) * 32 + slot) * 32 + (uint32_t)(n & 1) * 512 +
                        (uint32_t)hb * 8;  // + 8 q rows (and their pad)
  uint32_t pw_r[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      pw_r[ks][c] = (uint32_t)(ks * 32 + 8 * hb + 4 * c + (n >> 2)) * 32 +
                    (uint32_t)(4 * ks + hb) * 128 + (uint32_t)(n & 3) * 8;
  uint32_t vrd[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    vrd[c] = (uint32_t)(16 * hb + n) * 64 + (uint32_t)((c ^ ((n >> 2) & 3)) << 4);
  char *pwt = wl + 2 * kStage;

  f32x4 acc_lo[8], acc_hi[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc_lo[db] = acc_hi[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegBig, mlim = kNegBig, l = 0.f, bs[4] = {0.f, 0.f, 0.f, 0.f};

  auto consume = [&](int key0, int stage, const uint4(&kc)[4]) {
    const char *st = wl + stage * kStage;
    const char *ksb = st + kVcBytes, *vsb = ksb + kSbBytes;
    // scores: lane (n, hb) gets key key0 + 16 q + n of row hb
    float s[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t W[4] = {kc[q].x, kc[q].y, kc[q].z, kc[q].w};
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t w8 = W[t] >> 8;
        lo[2 * t] = W[t] & kLoNib;
        lo[2 * t + 1] = w8 & kLoNib;
        hi[2 * t] = W[t] & kHiNib;
        hi[2 * t + 1] = w8 & kHiNib;
      }
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      f32x4 cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[0], as_half8(lo[0], lo[1], lo[2], lo[3]), zero, 0, 0, 0);
      cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[1], as_half8(lo[4], lo[5], lo[6], lo[7]), cl, 0, 0, 0);
      f32x4 ch = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[2], as_half8(hi[0], hi[1], hi[2], hi[3]), zero, 0, 0, 0);
      ch = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[3], as_half8(hi[4], hi[5], hi[6], hi[7]), ch, 0, 0, 0);
      const uint32_t kw = *(const uint32_t *)(ksb + (16 * q + n) * 16 + hb * 4);
      const float ks = lo_h(kw) * kq, kb = hi_h(kw);
      float t4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) t4[r] = __builtin_fmaf(ks, __builtin_fmaf(cl[r], 16.f, ch[r]), kb * qsq[r]);
      s[q] = swap_add16(swap_add32(t4[0], t4[2]), swap_add32(t4[1], t4[3]));
    }
    if (key0 + kTile > sp.j1) {  // wave-uniform: keys past the span end get -inf
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (key0 + 16 * q + n >= sp.j1) s[q] = -INFINITY;
    }
    const float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (__builtin_amdgcn_ballot_w64(mx > mlim)) {  // wave-uniform, rare after a first tile
      const float rm = row_max16(mx);
      const float nm = rm > mlim ? rm : m;  // uniform in each row
      const float a = fast_exp2(m - nm);
      m = nm;
      mlim = nm + kSlack;
      l *= a;
#pragma unroll
      for (int g = 0; g < 4; ++g) bs[g] *= a;
      // accumulator column (h, g) = lane n: row h's factor, from lane 16 h
      const int ai = __builtin_bit_cast(int, a), hc = n >> 2;
      const int r0 = __builtin_amdgcn_readlane(ai, 0), r1 = __builtin_amdgcn_readlane(ai, 16);
      const int r2 = __builtin_amdgcn_readlane(ai, 32), r3 = __builtin_amdgcn_readlane(ai, 48);
      const float f = __builtin_bit_cast(float, hc == 0 ? r0 : hc == 1 ? r1 : hc == 2 ? r2 : r3);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        acc_lo[db] *= f;
        acc_hi[db] *= f;
      }
    }
    // weights p s_g (fp16) to the slot rows, p b_g to the bias sums
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float pe = fast_exp2(s[q] - m);  // masked: 2^-inf = 0
      l += pe;
      const uint4 vw = *(const uint4 *)(vsb + (16 * q + n) * 16);
      const uint32_t v4[4] = {vw.x, vw.y, vw.z, vw.w};
      const uint32_t w01 = mix_hi(mix_lo(pe, v4[0]), pe, v4[1]);
      const uint32_t w23 = mix_hi(mix_lo(pe, v4[2]), pe, v4[3]);
#pragma unroll
      for (int g = 0; g < 4; ++g) bs[g] = __builtin_fmaf(pe, hi_h(v4[g]), bs[g]);
      *(uint2 *)(pwt + pw_w + 384 * q) = make_uint2(w01, w23);
    }
    // weight operands of the two k-steps (low-nibble keys, high-nibble keys)
    half8 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const half4 p0 = __builtin_bit_cast(
          half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(LDS_PTR(fp16x4_t, pwt + pw_r[ks][0])));
      const half4 p1 = __builtin_bit_cast(
          half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(LDS_PTR(fp16x4_t, pwt + pw_r[ks][1])));
      pb[ks] = half8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
    }
    // O^T += V^T P'^T per 16-dim block
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      typedef int v2i __attribute__((ext_vector_type(2)));
      const v2i w = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
          LDS_PTR(v2i, st + vrd[db >> 1] + (db & 1) * 8));
      const uint32_t w0 = (uint32_t)w.x, w1 = (uint32_t)w.y;
      const uint32_t w08 = w0 >> 8, w18 = w1 >> 8;
      acc_lo[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          as_half8(w0 & kLoNib, w08 & kLoNib, w1 & kLoNib, w18 & kLoNib), pb[0], acc_lo[db], 0, 0, 0);
      acc_hi[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          as_half8(w0 & kHiNib, w08 & kHiNib, w1 & kHiNib, w18 & kHiNib), pb[1], acc_hi[db], 0, 0, 0);
    }
  };

  // Q and the first tile have arrived: nothing the compiler issued is outstanding
  __builtin_amdgcn_s_waitcnt(0);
  // (each consume is followed by a full wait on every path, the exit included: the next
  // tile has arrived, and the compiler sees no load of its own in flight at the top)
  while (base < sp.j1) {
    int next = base + STEP;
    if (next < sp.j1) issue(next, 1, kc1);
    consume(base, 0, kc0);
    __builtin_amdgcn_s_waitcnt(0);
    base = next;
    if (base >= sp.j1) break;
    next = base + STEP;
    if (next < sp.j1) issue(next, 0, kc0);
    consume(base, 1, kc1);
    __builtin_amdgcn_s_waitcnt(0);
    base = next;
  }

  // row sums of the wave
  l = row_sum16(l);
#pragma unroll
  for (int g = 0; g < 4; ++g) bs[g] = row_sum16(bs[g]);
  __syncthreads();  // every wave is done with its stages (the partials reuse the LDS)
  if (n == 0 && hb < cnt) {
    sm.wm.m[wave][hb] = m;
    sm.wm.l[wave][hb] = l;
#pragma unroll
    for (int g = 0; g < 4; ++g) sm.wm.bs[wave][hb][g] = bs[g];
  }
  {
    // accumulator lane (column n = 4 h + g, row block hb): dims 16 db + 4 hb + i of
    // row h, kept for the blocks db = 2 g, 2 g + 1 of group g
    const int hc = n >> 2, gc = n & 3;
    if (hc < cnt) {
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        if ((db >> 1) == gc) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = __builtin_fmaf(acc_lo[db][i], 16777216.f, acc_hi[db][i] * 1048576.f);
          *(f32x4 *)&sm.wm.acc[wave][hc][16 * db + 4 * hb] = v;
        }
      }
    }
  }
  __syncthreads();
  const PartRsrc pr = part_rsrc(p, b, qi);
  constexpr int DQ = D / 4;
  for (int t = tid; t < cnt * DQ; t += NT) {
    const int r = t / DQ, dq = t - r * DQ, g = dq >> 3;
    float mm = sm.wm.m[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) mm = fmaxf(mm, sm.wm.m[w][r]);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    float lw = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm.wm.m[w][r] - mm);
      a += f * (*(const f32x4 *)&sm.wm.acc[w][r][4 * dq] + sm.wm.bs[w][r][g]);
      lw = __builtin_fmaf(f, sm.wm.l[w][r], lw);
    }
    if (b.S_total == 1) {  // the only span of its rows: final output, no merge
      const size_t row = (size_t)gr.head(r) * p.M + qi;
      const float inv = lw > 0.f ? 1.f / lw : 0.f;
      *(float4 *)(b.out + row * D + 4 * dq) = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
      if (dq == 0 && b.lse) b.lse[row] = lw > 0.f ? (mm + __log2f(lw)) * 0.69314718055994530942f : -INFINITY;
    } else {
      store_part(pr, gr.head(r), x, dq, a);
      if (dq == 0) store_ml(pr, gr.head(r), x, lw > 0.f ? mm : -INFINITY, lw);  // empty: weight 0
    }
  }
  if (b.S_total > 1) ticket_and_merge<D, NT>(p, b, pr, gr, qi, sm.last);
}

}  // namespace

hipError_t launch_mlx4_mfma(const PartialParams &p, int rows_per_group, int x_count,
                            hipStream_t s) {
  if (x_count < 1 || p.y_groups < 1 || p.n_prob < 1) return hipSuccess;
  if (p.S_max > kMaxSplits || p.n_prob > kMaxBatch || p.fmt != 1 || p.D != 128)
    return hipErrorInvalidValue;
  if (rows_per_group < 1 || rows_per_group > 4) return hipErrorInvalidValue;
  constexpr int NW = 8;
  dim3 grid(x_count, p.y_groups, p.n_prob);
  note_launch("mlx4_mfma_kernel<%d>", NW);
  hipLaunchKernelGGL(mlx4_mfma_kernel<NW>, grid, dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace pion
