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
// Splits of the key range run in different workgroups, which store their (acc, m, l)
// partials; a second kernel merges them with the LSE rule (no workgroup waits on
// another).
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
constexpr int BK = 64;    // keys per tile
constexpr int kMaxPrefillSplits = 16;
constexpr int kMergeChunk = 8;  // splits whose partials the merge loads per round

// Byte offset of the 16-byte piece (split c, wave w, 32-dim block db, quad i, lane) in a
// row block's partials
template <int NDB>
__device__ __forceinline__ uint32_t part_off(int c, int w, int db, int i, int lane) {
  return (uint32_t)(((((c * 4 + w) * NDB + db) * 4 + i) * 64 + lane) * 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


constexpr int NSTAGE = 2;  // LDS tile stages (loads run NSTAGE - 1 tiles ahead)

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
  const int tile = h * p.n_iblk + ib;
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

  const i32x4 rK = rsrc_words(p.K + (size_t)g * p.N * D, (uint32_t)p.N * ROWG);
  const i32x4 rV = rsrc_words(p.V + (size_t)g * p.N * D, (uint32_t)p.N * ROWG);
  const bool has_suf = p.S_suf > 0;  // a null suffix gets an empty range
  const i32x4 rKs =
      rsrc_words(has_suf ? p.Ksuf + (size_t)g * p.S_suf * D : p.K, (uint32_t)p.S_suf * ROWG);
  const i32x4 rVs =
      rsrc_words(has_suf ? p.Vsuf + (size_t)g * p.S_suf * D : p.V, (uint32_t)p.S_suf * ROWG);

  // Tiles never straddle the prefix / suffix boundary: the split's prefix part
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
  auto issue = [&](int j) {
    const bool suf = j >= n_pre;  // workgroup-uniform
    const int r0 = suf ? suf_beg - p.N + (j - n_pre) * BK : k_begin + j * BK;  // source row
    const i32x4 rk = suf ? rKs : rK, rv = suf ? rVs : rV;
    const uint32_t st = lds0 + (uint32_t)((j % NSTAGE) * 2 * TB + 1024 * NLD * wave_u);
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
      load_lds16(rk, (uint32_t)r0 * ROWG + voff[t], st + 1024 * t);
      load_lds16(rv, (uint32_t)r0 * ROWG + voff[t], st + TB + 1024 * t);
    }
  };

  for (int j = 0; j < NSTAGE - 1 && j < n_tiles; ++j) issue(j);
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
  f16v o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = kNegBig, l_run = 0.f;

  // Operand addresses inside a stage, as loop-invariant lane offsets (the stage and
  // sub-tile parts are immediates): K row 32 kb + col at logical chunk 2 ds + hl; V^T
  // via transposed reads: lane (group gq, index q) addresses row kbase + q/4 at dims
  // 32 db + 16 gq + 4 (q%4), for kbase = 32 kb + 16 s2 + 4 hl + 8 c (c = 0, 1: the two
  // runs of 4 keys of a 16-key k-step); the swizzle of those rows depends on q, hl, c.
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
  auto kfrag = [&](int base, int ds) {  // base: byte offset of the 32-key sub-tile in LDS
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
  constexpr int KR = NDS < 4 ? NDS : 4;  // K fragments in flight ahead of their product

  // One 64-key tile from LDS stage STG (a compile-time constant, so every operand
  // address is a lane offset plus an immediate).
  auto run_tile = [&](auto stg, int j) {
    constexpr int STG = decltype(stg)::value;
    const bool suf = j >= n_pre;
    const int t0 = suf ? suf_beg + (j - n_pre) * BK : k_begin + j * BK;  // concatenated index
    const int seg_end = suf ? k_stop : pre_end;   // keys at or past this are not in the tile
    const int lane_end = suf ? row_end : pre_end; // this row's limit inside the tile
    const int clean_end = suf ? min(k_stop, full_end) : pre_end;  // no mask below this
    // this wave's loads of tile j are done (later tiles' loads may stay in flight) ...
    if (NSTAGE > 2 && j + 1 < n_tiles)
      __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NLD * (NSTAGE > 2 ? NSTAGE - 2 : 0)) : "memory");
    else
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // ... and every wave's; every wave is also done reading the stage loaded next
    __syncthreads();
    if (j + NSTAGE - 1 < n_tiles) issue(j + NSTAGE - 1);
    // Two workgroups on a CU share its SIMDs; the arbiter favours the older waves, so one
    // would run ahead and the other finish alone at the end. Priority falls with the tiles
    // left, so the one behind catches up and both end together.
    {
      const int rem = n_tiles - j;
      if (rem > 8) __builtin_amdgcn_s_setprio(3);
      else if (rem > 4) __builtin_amdgcn_s_setprio(2);
      else if (rem > 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    constexpr int KB = STG * 2 * TB, VB = KB + TB;  // stage offsets of K and V

    // two 32-key sub-tiles: S^T, softmax, PV
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kt0 = t0 + 32 * kb;
      if (kt0 >= seg_end) break;  // workgroup-uniform
      f16v s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
      half8 kf[KR];
#pragma unroll
      for (int ds = 0; ds < KR; ++ds) kf[ds] = kfrag(KB + 32 * kb * (int)ROWB, ds);
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ds % KR], qb[ds], s, 0, 0, 0);
        if (ds + KR < NDS) kf[ds % KR] = kfrag(KB + 32 * kb * (int)ROWB, ds + KR);
      }
      // the V^T fragments of both 16-key k-steps load while the softmax runs; the
      // scheduling barrier keeps the compiler from sinking the loads to their products,
      // where the wait for LDS would stall the wave
      half8 vf[NDB], vf2[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) vf[db] = vfrag(VB + 32 * kb * (int)ROWB, db);
#pragma unroll
      for (int db = 0; db < NDB; ++db) vf2[db] = vfrag(VB + (32 * kb + 16) * (int)ROWB, db);
      __builtin_amdgcn_sched_barrier(0);
      if (kt0 + 32 > clean_end) {  // boundary sub-tile: mask keys past this row's limit
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (kt0 + 8 * i + 4 * hl + jj >= lane_end) s[4 * i + jj] = -INFINITY;
      }
      float mt = -INFINITY;  // raw-score max; the scale is positive
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
        pb[e >> 3][e & 7] = (_Float16)pf;  // at most 2^8
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[db], pb[0], o[db], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf2[db], pb[1], o[db], 0, 0, 0);
    }
  };

  for (int j = 0; j < n_tiles; j += NSTAGE) {
    run_tile(std::integral_constant<int, 0>(), j);
    if (j + 1 < n_tiles) run_tile(std::integral_constant<int, 1>(), j + 1);
    if constexpr (NSTAGE > 2)
      if (j + 2 < n_tiles) run_tile(std::integral_constant<int, 2>(), j + 2);
  }
  l_run = sum_xor32(l_run);

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

  // Split partial: acc unnormalized against m_run, in the register layout of o (tile,
  // split, wave, 32-dim block db, quad i, lane: one 16-byte piece per lane, so every
  // store instruction moves 1 KB of consecutive bytes); m and l (log2 units) per
  // [row][split]. prefill_merge_kernel, next on the stream, combines the splits.
  const int S = p.n_splits;
  const int rows_valid = min(BQ, p.M - i0);
  const size_t row0 = (size_t)h * p.M + i0;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(p.part_acc + (size_t)tile * BQ * S * D, (uint32_t)(BQ * S * D * 4));
  const __amdgpu_buffer_rsrc_t rM = make_rsrc(p.part_m + row0 * S, (uint32_t)(rows_valid * S * 4));
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(p.part_l + row0 * S, (uint32_t)(rows_valid * S * 4));
  const int r = wave * 32 + col;  // local row; rows past rows_valid fall out of range
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = {o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rA,
                                             part_off<NDB>(split, wave, db, i, lane), 0, 0);
    }
  if (hl == 0) {
    const float mv = l_run > 0.f ? m_run : -INFINITY;  // empty split: weight 0
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, mv), rM, (r * S + split) * 4, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l_run), rL, (r * S + split) * 4, 0, 0);
  }
}

// Combine the split partials of prefill_kernel. One workgroup per (row block, 32-dim
// block db): thread (wave w, lane l) takes the place of the split kernel's lane, row
// 32 w + l % 32 and dims 32 db + 8 i + 4 (l / 32) + 0..3, and reads that piece of every
// split (up to kMergeChunk splits per round of loads) with the row's m and l, then
// applies the LSE rule: out = sum_c 2^(m_c - m*) acc_c / sum_c 2^(m_c - m*) l_c.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams p) {
  constexpr int NDB = D / 32, CH = kMergeChunk;
  const int S = p.n_splits;
  const int tile = blockIdx.x / NDB, db = blockIdx.x - tile * NDB;
  const int h = tile / p.n_iblk, ib = tile - h * p.n_iblk;
  const int i0 = ib * BQ, rows_valid = min(BQ, p.M - i0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5;
  const int r = wave * 32 + (lane & 31);
  const int rr = min(r, rows_valid - 1);  // rows past the end repeat the last row, unstored
  const size_t row0 = (size_t)h * p.M + i0;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(p.part_acc + (size_t)tile * BQ * S * D, (uint32_t)(BQ * S * D * 4));
  const __amdgpu_buffer_rsrc_t rM = make_rsrc(p.part_m + row0 * S, (uint32_t)(rows_valid * S * 4));
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(p.part_l + row0 * S, (uint32_t)(rows_valid * S * 4));
  float mv[kMaxPrefillSplits], lv[kMaxPrefillSplits];
#pragma unroll
  for (int c = 0; c < kMaxPrefillSplits; ++c) {
    mv[c] = c < S ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rM, (rr * S + c) * 4, 0, 0))
                  : -INFINITY;
    lv[c] = c < S ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rL, (rr * S + c) * 4, 0, 0))
                  : 0.f;
  }
  f32x4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float M = -INFINITY, L = 0.f;
  for (int c0 = 0; c0 < S; c0 += CH) {
    f32x4 v[CH][4];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[cc][i] = c0 + cc < S ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                     rA, part_off<NDB>(c0 + cc, wave, db, i, lane), 0, 0))
                               : f32x4{0.f, 0.f, 0.f, 0.f};
    if (c0 == 0) {
#pragma unroll
      for (int c = 0; c < kMaxPrefillSplits; ++c) M = fmaxf(M, mv[c]);
#pragma unroll
      for (int c = 0; c < kMaxPrefillSplits; ++c) {
        mv[c] = fast_exp2(mv[c] - M);  // the split's weight; -inf (empty or absent) -> 0
        L = __builtin_fmaf(mv[c], lv[c], L);
      }
    }
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      float w = 0.f;
#pragma unroll
      for (int c = 0; c < kMaxPrefillSplits; ++c) w = c == c0 + cc ? mv[c] : w;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += w * v[cc][i];
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
  const dim3 grid(8 * ((W + 7) / 8)), mgrid(tiles * (p.D / 32));
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
