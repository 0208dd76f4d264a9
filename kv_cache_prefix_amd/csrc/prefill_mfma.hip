// Batched-Q attention over a resident fp16 prefix and a causal fp16 suffix, on fp16
// MFMA (the QUERY_FUSED wire form of the ATTEND.* page and the batched-Q QUERY of the
// "Shared KV Cache Serving" page, Wire-protocol details). Row i of q-head h attends the
// N prefix keys of kv-head g = head_map[h] and the suffix keys j <= S_suf - M + i.
//
// Per workgroup: 128 query rows of one q-head (4 waves x 32 rows) against one split of
// the key index space [0, N + S_suf) (prefix then suffix), in tiles of 32 keys. For
// D <= 128 the tiles run as a three-deep software pipeline: one iteration issues the
// PV product of tile j - 1, the softmax weights of tile j and the S^T product of tile
// j + 1, so the matrix work of one tile covers the vector work of the next; larger head
// dims (whose accumulators leave no registers for a second tile) run tiles in sequence.
//   S^T = K Q^T   on v_mfma_f32_32x32x16_f16: A = a 32-key x 16-dim slice of the K tile
//                 (LDS, row-major), B = Q^T (registers, loaded once); the result lane l
//                 holds 16 keys x 1 query (query l % 32).
//   online softmax in fp32 (log2 units, scale folded into the exponent; the row sum
//                 uses the fp32 weights, the PV product their fp16 roundings; a tile's
//                 weights are taken against the running max as it stands, and only
//                 when they overflow (a lane's sum past 2^15) is the tile's row max
//                 taken and the accumulators rescaled; only boundary tiles are
//                 masked); a lane's p
//                 values are already the B operand of the next product: result element
//                 (i, j) of the S^T block is key 8i + 4(l/32) + j, and a 16-key k-step of
//                 the PV product takes elements i = 2s, 2s+1 as its eight k slots.
//   O^T += V^T P^T  A = V^T (LDS, stored transposed at staging so each lane reads two
//                 runs of 4 keys), with the k slots in that same key order.
// Staging: K and V tiles go from HBM straight into LDS with buffer loads that write LDS
// (no register staging), NSTAGE tiles deep: the loads of tile j + NSTAGE - 1 are issued
// when tile j starts. Both tiles are stored row-major with the 16-byte chunks of a row
// XOR-swizzled by a function of the row (swz), which makes the K operand reads and the
// transposed V reads bank-conflict free. An LDS row holds DP = D rounded up to a power of
// two (at least 64) dims, the layout the swizzle was searched for: for D = 32, 96, 160,
// 192 the chunks past D are padding (their loads fetch a chunk of the same row again,
// already in flight, and nothing reads them). V^T operands come from row-major V through the
// LDS transpose read (ds_read_b64_tr_b16): in each 16-lane group, lane i receives
// element i % 4 of the 8-byte pieces addressed by lanes 4j + i/4 (j = 0..3), so lanes
// addressing (row kbase + q/4, dims dbase + 4(q%4)) receive 4 consecutive keys of dim
// dbase + i.
// The compiler cannot tell which LDS bytes an asynchronous LDS load writes, so it
// would wait for every outstanding one before any LDS read; the loads are issued
// through inline assembly instead and the kernel waits for them itself (s_waitcnt
// vmcnt, then a barrier) before a stage is read.
// Splits of the key range run in different workgroups, which store their partials (the
// split's normalized output in fp16 and its log-sum-exp in fp32); a second kernel merges
// them with the LSE rule (no workgroup waits on another).
#include "kernels.h"
#include "mfma_common.h"

#include <type_traits>

namespace pion {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Note: the result of __builtin_amdgcn_raw_buffer_load_b128 is reinterpreted as a whole
// vector (bit_cast to f32x4); bit-casting its elements one by one makes this compiler
// narrow the load to a single dword.

constexpr float kNegBig = -1.0e30f;
constexpr int BQ = 128;   // query rows per workgroup
constexpr int BK = 32;    // keys per tile
constexpr int kMaxPrefillSplits = 16;
constexpr int kMergeChunk = 8;  // splits whose partials the merge loads per round
// A lane's weights of one tile may sum to this much before the running max moves (each
// weight then stays below 2^15, inside fp16's range with its full relative precision)
constexpr float kGrowLimit = 32768.f;

// Byte offset of the 16-byte piece (split c, wave w, 32-dim block db, pair of quads i2,
// lane) in a row block's fp16 partials
template <int NDB>
__device__ __forceinline__ uint32_t part_off(int c, int w, int db, int i2, int lane) {
  return (uint32_t)(((((c * 4 + w) * NDB + db) * 2 + i2) * 64 + lane) * 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


constexpr int NSTAGE = 4;  // LDS tile stages (tile t + 3 loads while tile t is in use)

// LDS dims per key row: D rounded up to a power of two, at least 64
template <int D>
constexpr int lds_dims() {
  int p = 64;
  while (p < D) p *= 2;
  return p;
}

template <int D>
struct PrefillSmem {
  static constexpr int TB = BK * 2 * lds_dims<D>();  // bytes of one K or V tile
  alignas(16) char kv[NSTAGE][2][TB];  // [stage][0: K, 1: V]
};

// Buffer resource over `bytes` bytes at `base`: loads past the end return zero, which
// masks the tails of the prefix and suffix without branches. 0x00020000 is the raw
// 32-bit data format of the descriptor's last word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The rows of a 128-row block (q-head h, block ib) that wave `wave` (0..3) holds:
// normalized out and lse when the keys are not split; else the split partial: the
// split's own normalized output acc / l rounded to fp16, in the register layout of o
// (tile, split, wave, 32-dim block db, quads 2 i2 and 2 i2 + 1, lane: one 16-byte piece
// per lane, so every store instruction moves 1 KB of consecutive bytes), and its
// log-sum-exp m + log2 l (log2 units; -inf for a split with no key of the row) per
// [row][split]. A normalized partial is a convex combination of fp16 V rows, so it lies
// in fp16's range and its rounding costs at most 2^-11 of its magnitude (half the bytes
// of fp32 partials). prefill_merge_kernel, next on the stream, combines the splits.
template <int D>
__device__ __forceinline__ void store_rows(const PrefillParams &p, const f16v (&o)[D / 32],
                                           float m_run, float l_run, int h, int ib, int split,
                                           int wave, int lane) {
  constexpr int NDB = D / 32;
  const int hl = lane >> 5, col = lane & 31;
  const int i0 = ib * BQ;
  const int qi = i0 + wave * 32 + col;
  const int tile = h * p.n_iblk + ib;
  if (p.n_splits == 1) {
    if (qi < p.M) {
      const size_t row = (size_t)h * p.M + qi;
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
  const int S = p.n_splits;
  const int rows_valid = min(BQ, p.M - i0);
  const size_t row0 = (size_t)h * p.M + i0;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(p.part_acc + (size_t)tile * BQ * S * D, (uint32_t)(BQ * S * D * 2));
  const __amdgpu_buffer_rsrc_t rM = make_rsrc(p.part_lse + row0 * S, (uint32_t)(rows_valid * S * 4));
  const int r = wave * 32 + col;  // local row; rows past rows_valid fall out of range
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;  // an empty split stores zeros
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      half8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (_Float16)(o[db][8 * i2 + e] * inv);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rA,
                                             part_off<NDB>(split, wave, db, i2, lane), 0, 0);
    }
  if (hl == 0) {
    const float lv = l_run > 0.f ? m_run + __log2f(l_run) : -INFINITY;  // empty: weight 0
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lv), rM, (r * S + split) * 4, 0, 0);
  }
}

// Instruction-group hints for the scheduler (masks of the AMDGPU backend's
// sched_group_barrier: MFMA, VALU, DS read).
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100;

template <int D>
__global__ __launch_bounds__(256, (D <= 128) ? 2 : 1) void prefill_kernel(PrefillParams p) {
  constexpr int NDB = D / 32;                 // 32-dim blocks of O^T
  constexpr int NDS = D / 16;                 // 16-dim k-steps of S^T
  constexpr int CH = D / 8;                   // 16-byte chunks per key row
  constexpr int DP = lds_dims<D>();           // dims per LDS row (swizzle layout)
  constexpr int CHP = DP / 8;                 // 16-byte chunks per LDS row
  constexpr uint32_t ROWG = D * 2;            // bytes per key row in HBM
  constexpr uint32_t ROWB = DP * 2;           // bytes per key row in LDS
  constexpr int TB = PrefillSmem<D>::TB;
  constexpr int NLD = TB / 1024 / 4;          // 1 KB LDS loads per wave, tile and side
  __shared__ PrefillSmem<D> sm;

  // Workgroups are dispatched to the 8 XCDs round-robin by block index; block b runs
  // logical workgroup xcd * C + b / 8 (C = blocks per XCD), and logical workgroups are
  // ordered by (q-head in kv-head order, row block, split). The workgroups that read one
  // kv-head's K and V then share an XCD and its L2. Blocks past the end exit.
  const int W = p.H_q * p.n_iblk * p.n_splits, C = (W + 7) >> 3;
  const int L = (blockIdx.x & 7) * C + (blockIdx.x >> 3);
  if (L >= W) return;
  const int split = L % p.n_splits, ts = L / p.n_splits;
  const int hs = ts / p.n_iblk, ib = ts - hs * p.n_iblk;
  const int h = p.order[hs], i0 = ib * BQ;
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
  // key tiles ending at or below this need no mask for any row of the workgroup
  const int lim_first = p.S_suf > 0 ? p.N + p.S_suf - p.M + i0 + 1 : p.N;
  const int full_end = min(k_end, lim_first);

  const i32x4 rK = rsrc_words(p.K + (size_t)g * p.N * D, (uint32_t)p.N * ROWG);
  const i32x4 rV = rsrc_words(p.V + (size_t)g * p.N * D, (uint32_t)p.N * ROWG);
  const bool has_suf = p.S_suf > 0;  // a null suffix gets an empty range
  const i32x4 rKs =
      rsrc_words(has_suf ? p.Ksuf + (size_t)g * p.S_suf * D : p.K, (uint32_t)p.S_suf * ROWG);
  const i32x4 rVs =
      rsrc_words(has_suf ? p.Vsuf + (size_t)g * p.S_suf * D : p.V, (uint32_t)p.S_suf * ROWG);

  // Tiles of BK keys never straddle the prefix / suffix boundary: the split's prefix part
  // [k_begin, pre_end) is tiled from k_begin, its suffix part [suf_beg, k_stop) from
  // suf_beg. Tile j < n_pre is prefix, the rest suffix.
  const int pre_end = min(k_stop, p.N);
  const int suf_beg = max(k_begin, p.N);
  const int n_pre = k_begin < pre_end ? (pre_end - k_begin + BK - 1) / BK : 0;
  const int n_suf = suf_beg < k_stop ? (k_stop - suf_beg + BK - 1) / BK : 0;
  const int n_tiles = n_pre + n_suf;

  // LDS loads of a tile: wave w's load t fills tile bytes [1 KB (NLD w + t), +1 KB),
  // lane l the 16 bytes at 16 l there: tile row r, physical chunk l % CHP, which holds
  // logical chunk (l % CHP) ^ swz(r) of source row r0 + r (a padding chunk, logical
  // chunk >= CH, loads chunk 0 of the row again).
  const uint32_t lds0 = (uint32_t)(uintptr_t)LDS_PTR(char, &sm.kv[0][0][0]);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t voff[NLD];
#pragma unroll
  for (int t = 0; t < NLD; ++t) {
    const int r = (1024 * (NLD * wave_u + t) + 16 * lane) / (int)ROWB;
    const int lc = (lane % CHP) ^ swz<DP>(r);
    voff[t] = (uint32_t)r * ROWG + (uint32_t)((lc < CH ? lc : 0) * 16);
  }
  // Tiles load in order; the next one's index, source byte offset and descriptors (the
  // suffix ones from tile n_pre on)
  int dma_j = 0;
  uint32_t dma_src = (uint32_t)k_begin * ROWG;
  i32x4 dk = rK, dv = rV;
  auto issue_next = [&]() {
    if (dma_j == n_pre) {  // workgroup-uniform
      dk = rKs;
      dv = rVs;
      dma_src = (uint32_t)(suf_beg - p.N) * ROWG;
    }
    const uint32_t st = lds0 + (uint32_t)((dma_j % NSTAGE) * 2 * TB + 1024 * NLD * wave_u);
#pragma unroll
    for (int t = 0; t + 1 < NLD; t += 2)
      load_lds16_x4(dk, dv, dma_src + voff[t], dma_src + voff[t + 1], st + 1024 * t,
                    st + 1024 * (t + 1), st + TB + 1024 * t, st + TB + 1024 * (t + 1));
    if (NLD & 1) {
      load_lds16(dk, dma_src + voff[NLD - 1], st + 1024 * (NLD - 1));
      load_lds16(dv, dma_src + voff[NLD - 1], st + TB + 1024 * (NLD - 1));
    }
    dma_src += BK * ROWG;
    ++dma_j;
  };
  // Tile j's first key in the concatenated index and this row's limit inside it. Tiles
  // that need the per-key mask: the last prefix tile when the prefix part ends inside it,
  // and the suffix tiles from j_suf_mask on (keys past the first row's causal limit).
  auto tile_t0 = [&](int j) { return j >= n_pre ? suf_beg + (j - n_pre) * BK : k_begin + j * BK; };
  auto tile_lane_end = [&](int j) { return j >= n_pre ? row_end : pre_end; };
  const int j_pre_mask = (n_pre > 0 && ((pre_end - k_begin) & (BK - 1))) ? n_pre - 1 : -1;
  const int lim_s = min(k_stop, full_end);
  const int j_suf_mask = n_pre + (lim_s > suf_beg ? (lim_s - suf_beg) / BK : 0);
  auto tile_clean = [&](int j) { return j != j_pre_mask && j < j_suf_mask; };

  while (dma_j < NSTAGE - 1 && dma_j < n_tiles) issue_next();
  half8 qb[NDS];
  {
    const uint16_t *qrow = p.Q + ((size_t)h * p.M + qi_c) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qb[ds] = *(const half8 *)(qrow + 16 * ds + 8 * hl);
  }
  // Q (and the first tiles) have arrived: the compiler then knows no load of its own is
  // outstanding in the loop, where any vmcnt wait it added would also drain the loads
  // of the next tiles
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f16v o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = kNegBig, l_run = 0.f;

  // Operand addresses inside a stage, as loop-invariant lane offsets (the stage part is
  // an immediate): K row col at logical chunk 2 ds + hl; V^T via transposed reads: lane
  // (group gq, index q) addresses row kbase + q/4 at dims 32 db + 16 gq + 4 (q%4), for
  // kbase = 16 s2 + 4 hl + 8 c (c = 0, 1: the two runs of 4 keys of a 16-key k-step);
  // the swizzle of those rows depends on q, hl, c.
  const char *smb = &sm.kv[0][0][0];
  uint32_t koff[NDS];
  {
    const int swk = swz<DP>(col);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      koff[ds] = (uint32_t)col * ROWB + (uint32_t)(((2 * ds + hl) ^ swk) << 4);
  }
  uint32_t voffs[2][NDB];
  {
    const int q16 = lane & 15, gq = (lane >> 4) & 1;
    const int vch = 2 * gq + ((q16 & 3) >> 1);  // logical chunk minus 4 db
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r = 4 * hl + 8 * c + (q16 >> 2);  // row modulo 16
      const int vsw = swz<DP>(r);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        voffs[c][db] = (uint32_t)r * ROWB + (uint32_t)(q16 & 1) * 8 +
                       (uint32_t)(((4 * db + vch) ^ vsw) << 4);
    }
  }
  auto kfrag = [&](int base, int ds) {  // base: byte offset of the K tile in LDS
    return __builtin_bit_cast(half8, *(const uint4 *)(smb + base + koff[ds]));
  };
  auto vfrag = [&](int base, int db) {  // base: byte offset of the 16-key k-step in LDS
    half4 part[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
      part[c] = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                              LDS_PTR(fp16x4_t, smb + base + voffs[c][db])));
    return half8{part[0][0], part[0][1], part[0][2], part[0][3],
                 part[1][0], part[1][1], part[1][2], part[1][3]};
  };

  // S^T of tile j from stage STG: result element (i, jj) of lane l is key 8 i + 4 (l / 32)
  // + jj of the tile, query row l % 32
  auto s_product = [&](auto stg) {
    constexpr int KB = decltype(stg)::value * 2 * TB;
    half8 kf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) kf[ds] = kfrag(KB, ds);
    f16v s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ds], qb[ds], s, 0, 0, 0);
    return s;
  };
  // Two workgroups on a CU share its SIMDs; the arbiter favours the older waves, so one
  // would run ahead and the other finish alone at the end. Priority falls with the tiles
  // left, so the one behind catches up and both end together.
  auto set_prio = [&](int rem) {
    if (rem > 16) __builtin_amdgcn_s_setprio(3);
    else if (rem > 8) __builtin_amdgcn_s_setprio(2);
    else if (rem > 4) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  };

  // The weights of a tile against the running max m (log2 units): fp16 into pb (masked
  // scores give 0), and this lane's part of the row sum from the fp32 values.
  auto tile_weights = [&](const f16v &sc, float m, half8 (&pb)[2]) {
    float lsum[4];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pf = fast_exp2(__builtin_fmaf(sc[e], p.qscale, -m));
      lsum[e & 3] = e < 4 ? pf : lsum[e & 3] + pf;
      pb[e >> 3][e & 7] = (_Float16)pf;
    }
    return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
  };
  // Lazy rescale without a per-tile row max: a lane's weights sum to at most kGrowLimit
  // (so each fits fp16 with room to spare) unless some score of its row exceeds the
  // running max by more than log2 of that (and always on a row's first keys, when m_run
  // is still kNegBig). Only then (wave-uniform branch, rare after the first tile) is the
  // tile's row max taken: m_run moves up to it, O and l are scaled by 2^(m_old - m_new)
  // and the weights recomputed. Rows whose max has not grown keep m_run.
  auto regrow = [&](const f16v &sc, float &lt, half8 (&pb)[2]) {
    if (__builtin_amdgcn_ballot_w64(!(lt <= kGrowLimit))) {
      float mt = fmaxf(sc[0], sc[1]);  // raw-score max; the scale is positive
#pragma unroll
      for (int e = 2; e < 16; ++e) mt = fmaxf(mt, sc[e]);
      mt = max_xor32(mt) * p.qscale;
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      lt = tile_weights(sc, m_run, pb);
    }
  };

  // Software pipeline over key tiles, three tiles deep: iteration j runs the PV product of
  // tile j - 1, the softmax weights of tile j and the S^T product of tile j + 1 - three
  // independent pieces of work, so the exponentials of one tile overlap the matrix
  // products of two others. Carried between iterations: S^T of tile j (s_cur), and the
  // fp16 weights and V^T operands of tile j - 1 (pb_prev, vf). Tile j sits in stage
  // j % NSTAGE (a compile-time constant in each unrolled copy of the body).
  f16v s_cur;
  half8 pb_prev[2];
  half8 vf[2][NDB];
  if (D <= 128 && n_tiles > 0) s_cur = s_product(std::integral_constant<int, 0>());
  // stg: the stage of tile j, an integral_constant in the unrolled main loop (every LDS
  // offset an immediate) or an int for the few tiles after it; has_prev / has_next: bool
  // constants (tile j - 1's product pending; tile j + 1 exists)
  auto step = [&](auto stg, int j, auto has_prev_c, auto has_next_c) {
    constexpr bool has_prev = decltype(has_prev_c)::value;
    constexpr bool has_next = decltype(has_next_c)::value;
    const int STG = stg;
    const int VB = STG * 2 * TB + TB;
    const int KBN = ((STG + 1) & (NSTAGE - 1)) * 2 * TB;
    if (has_next) {
      // this wave's loads of tile j + 1 are done (tile j + 2's may stay in flight) ...
      if (j + 2 < n_tiles)
        __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NLD) : "memory");
      else
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      // ... and every wave's; every wave is also done with tile j - 1 (its V^T operands
      // are in registers), whose stage tile j + 3 fills
      __syncthreads();
      if (dma_j < n_tiles) issue_next();  // tile j + NSTAGE - 1
    }
    // Tile j: mask (boundary tiles only); its weights are taken against the running max
    // m_run as it stands, and the tile's own row max only when they overflow (below)
    if (!tile_clean(j)) {
      const int kt0 = tile_t0(j), lane_end = tile_lane_end(j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (kt0 + 8 * i + 4 * hl + jj >= lane_end) s_cur[4 * i + jj] = -INFINITY;
    }
    // The three products and the weights, as one straight-line block: reads of K (tile
    // j + 1) start first, the PV product of tile j - 1 and the weights of tile j run
    // while they are in flight, then the V^T reads of tile j and the S^T product of tile
    // j + 1; the scheduling groups space the matrix products by vector ops and reads.
    constexpr int KR = NDS < 4 ? NDS : 4;  // K fragments in flight ahead of their product
    half8 kf[KR];
    if (has_next) {
#pragma unroll
      for (int ds = 0; ds < KR; ++ds) kf[ds] = kfrag(KBN, ds);
    }
    if (has_prev) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[k][db], pb_prev[k], o[db], 0, 0, 0);
    }
    half8 pb[2];
    float lt = tile_weights(s_cur, m_run, pb);
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int db = 0; db < NDB; ++db) vf[k][db] = vfrag(VB + 16 * k * (int)ROWB, db);
    f16v s_nxt;
    if (has_next) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s_nxt[e] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ds % KR], qb[ds], s_nxt, 0, 0, 0);
        if (ds + KR < NDS) kf[ds % KR] = kfrag(KBN, ds + KR);
      }
    }
    // the weights and row sum of tile j are due in this block (left alone, the compiler
    // sinks them to the next iteration, after the matrix products, serializing the two)
    __asm__ volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(lt));
    if (has_prev && has_next) {
      constexpr int NRD = NDS - KR + 4 * NDB;  // reads after the first K fragments
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, KR, 0);
#pragma unroll
      for (int i = 0; i < NDS + 2 * NDB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgValu, 4, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, (NRD + NDS + 2 * NDB - 1) / (NDS + 2 * NDB), 0);
      }
    }
    regrow(s_cur, lt, pb);
    l_run += lt;
    pb_prev[0] = pb[0];
    pb_prev[1] = pb[1];
    if (has_next) s_cur = s_nxt;
  };
  // Head dims above 128 hold twice the accumulators and operands: there the tiles run one
  // after the other (S^T, softmax and PV of tile j in iteration j), which fits the
  // registers without spilling.
  auto step_seq = [&](auto stg, int j) {
    constexpr int STG = decltype(stg)::value;
    constexpr int KB = STG * 2 * TB, VB = KB + TB;
    if (j > 0) {
      // this wave's loads of tile j are done (those of the up to two tiles issued after
      // it may stay in flight), then every wave's
      static_assert(NSTAGE - 2 == 2, "two tiles load ahead of the one in use");
      if (j + 2 < n_tiles)
        __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * NLD) : "memory");
      else if (j + 1 < n_tiles)
        __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NLD) : "memory");
      else
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if (dma_j < n_tiles) issue_next();  // tile j + NSTAGE - 1
    set_prio(n_tiles - j);
    f16v s = s_product(stg);
    if (!tile_clean(j)) {
      const int kt0 = tile_t0(j), lane_end = tile_lane_end(j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (kt0 + 8 * i + 4 * hl + jj >= lane_end) s[4 * i + jj] = -INFINITY;
    }
    half8 vv[2][NDB];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int db = 0; db < NDB; ++db) vv[k][db] = vfrag(VB + 16 * k * (int)ROWB, db);
    half8 pb[2];
    float lt = tile_weights(s, m_run, pb);
    regrow(s, lt, pb);
    l_run += lt;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv[k][db], pb[k], o[db], 0, 0, 0);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  using T = std::true_type;
  using F = std::false_type;
  static_assert(NSTAGE == 4, "the main loop is unrolled over the four stages");
  int j = 0;
  if constexpr (D > 128) {
    for (; j + NSTAGE <= n_tiles; j += NSTAGE) {
      step_seq(C0(), j);
      step_seq(C1(), j + 1);
      step_seq(C2(), j + 2);
      step_seq(C3(), j + 3);
    }
    if (j < n_tiles) step_seq(C0(), j);
    if (j + 1 < n_tiles) step_seq(C1(), j + 1);
    if (j + 2 < n_tiles) step_seq(C2(), j + 2);
  } else if (n_tiles > 1) {
    set_prio(n_tiles);
    step(C0(), 0, F(), T());
    j = 1;
    for (; j + NSTAGE < n_tiles; j += NSTAGE) {
      set_prio(n_tiles - j);  // once per four tiles
      step(C1(), j, T(), T());
      step(C2(), j + 1, T(), T());
      step(C3(), j + 2, T(), T());
      step(C0(), j + 3, T(), T());
    }
    set_prio(n_tiles - j);
    for (; j + 1 < n_tiles; ++j) step(j & (NSTAGE - 1), j, T(), T());
    step(j & (NSTAGE - 1), j, T(), F());
  } else if (n_tiles == 1) {
    step(C0(), 0, F(), F());
  }
  if (D <= 128 && n_tiles > 0) {  // the PV product of the last tile
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[k][db], pb_prev[k], o[db], 0, 0, 0);
  }
  __builtin_amdgcn_s_setprio(0);
  l_run = sum_xor32(l_run);

  store_rows<D>(p, o, m_run, l_run, h, ib, split, wave, lane);
}

// Combine the split partials of prefill_kernel. One workgroup per (row block, 32-dim
// block db): thread (wave w, lane l) takes the place of the split kernel's lane, row
// 32 w + l % 32 and dims 32 db + 8 i + 4 (l / 32) + 0..3, and reads that piece of every
// split (up to kMergeChunk splits per round of loads) with the row's per-split
// log-sum-exp s_c, then applies the LSE rule to the normalized partials o_c:
// out = sum_c 2^(s_c - s*) o_c / sum_c 2^(s_c - s*), lse = s* + log2 sum_c 2^(s_c - s*).
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams p) {
  constexpr int NDB = D / 32, CH = kMergeChunk;
  const int S = p.n_splits;
  // Logical workgroups (row block in the split kernel's q-head order, then db) spread
  // over the XCDs as the split kernel's are: XCD x takes the same share of row blocks
  // whose splits it ran, so the partials are read from its own L2 while they are there.
  const int T = p.H_q * p.n_iblk, W = T * NDB, C = (W + 7) >> 3;
  const int Lm = (blockIdx.x & 7) * C + (blockIdx.x >> 3);
  if (Lm >= W) return;
  const int ts = Lm / NDB, db = Lm - ts * NDB;
  const int hs = ts / p.n_iblk, ib = ts - hs * p.n_iblk;
  const int h = p.order[hs], tile = h * p.n_iblk + ib;
  const int i0 = ib * BQ, rows_valid = min(BQ, p.M - i0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5;
  const int r = wave * 32 + (lane & 31);
  const int rr = min(r, rows_valid - 1);  // rows past the end repeat the last row, unstored
  const size_t row0 = (size_t)h * p.M + i0;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(p.part_acc + (size_t)tile * BQ * S * D, (uint32_t)(BQ * S * D * 2));
  const __amdgpu_buffer_rsrc_t rM = make_rsrc(p.part_lse + row0 * S, (uint32_t)(rows_valid * S * 4));
  float wv[kMaxPrefillSplits];
#pragma unroll
  for (int c = 0; c < kMaxPrefillSplits; ++c)
    wv[c] = c < S ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rM, (rr * S + c) * 4, 0, 0))
                  : -INFINITY;
  f32x4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float M = -INFINITY, L = 0.f;
  for (int c0 = 0; c0 < S; c0 += CH) {
    u32x4 v[CH][2];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc)
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2)
        v[cc][i2] = c0 + cc < S ? __builtin_amdgcn_raw_buffer_load_b128(
                                      rA, part_off<NDB>(c0 + cc, wave, db, i2, lane), 0, 0)
                                : u32x4{0u, 0u, 0u, 0u};
    if (c0 == 0) {
#pragma unroll
      for (int c = 0; c < kMaxPrefillSplits; ++c) M = fmaxf(M, wv[c]);
#pragma unroll
      for (int c = 0; c < kMaxPrefillSplits; ++c) {
        wv[c] = fast_exp2(wv[c] - M);  // the split's weight; -inf (empty or absent) -> 0
        L += wv[c];
      }
    }
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      float w = 0.f;
#pragma unroll
      for (int c = 0; c < kMaxPrefillSplits; ++c) w = c == c0 + cc ? wv[c] : w;
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const half8 hv = __builtin_bit_cast(half8, v[cc][i2]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[2 * i2 + e / 4][e % 4] += w * (float)hv[e];
      }
    }
  }
  if (r < rows_valid) {
    const float inv = 1.f / L;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(f32x4 *)(p.out + (row0 + r) * D + 32 * db + 8 * i + 4 * hl) = acc[i] * inv;
    if (db == 0 && hl == 0 && p.lse) p.lse[row0 + r] = (M + __log2f(L)) * 0.69314718055994530942f;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, hipStream_t s) {
  if (p.n_splits < 1 || p.n_splits > kMaxPrefillSplits || p.split_keys % BK) return hipErrorInvalidValue;
  const int tiles = p.H_q * p.n_iblk, W = tiles * p.n_splits;
  const dim3 grid(8 * ((W + 7) / 8)), mgrid(8 * ((tiles * (p.D / 32) + 7) / 8));
  const bool merge = p.n_splits > 1;
  note_launch("prefill_kernel<%d>", p.D);
  if (merge) note_launch("prefill_merge_kernel<%d>", p.D);
#define PION_PREFILL_D(DD)                                                              \
  case DD:                                                                              \
    hipLaunchKernelGGL(prefill_kernel<DD>, grid, dim3(256), 0, s, p);                   \
    if (merge) hipLaunchKernelGGL(prefill_merge_kernel<DD>, mgrid, dim3(256), 0, s, p); \
    break;
  switch (p.D) {
    PION_PREFILL_D(32)
    PION_PREFILL_D(64)
    PION_PREFILL_D(96)
    PION_PREFILL_D(128)
    PION_PREFILL_D(160)
    PION_PREFILL_D(192)
    PION_PREFILL_D(256)
    default: return hipErrorInvalidValue;
  }
#undef PION_PREFILL_D
  return hipGetLastError();
}

}  // namespace pion
