// Internal launch interface between the C ABI (pion_prefix.cpp) and the HIP kernels.
// Not installed; the public interface is include/pion_prefix.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pion {

constexpr int kMaxHeads = 128;     // H_q limit (row-group table size)
constexpr int kRowsPerGroup = 8;   // q-heads sharing one kv-head read per workgroup

// Groups of up to kRowsPerGroup q-heads that read the same kv-head. A workgroup of the
// partial-attention kernel serves one group at one query index, so the K/V bytes it
// streams are shared by every q-head of the group (GQA).
struct RowGroups {
  int n;
  uint8_t g[kMaxHeads];
  uint8_t cnt[kMaxHeads];
  uint8_t heads[kMaxHeads][kRowsPerGroup];
};

// One resident prefix as the kernels see it.
struct KVView {
  int fmt;              // 0 fp16, 1 mlx4g32
  int H, N, D;
  const uint16_t *K, *V;                 // fp16 [H, N, D]
  const uint32_t *Kc, *Vc;               // mlx4g32 codes [H, N, D/8]
  const uint16_t *Ks, *Kb, *Vs, *Vb;     // mlx4g32 scales / biases [H, N, D/32]
};

// Split-over-keys attention. Workgroup (x, y): y = head group * M + query index,
// x = key span. Spans [0, pre_splits) cover the prefix (dense chunks of pre_chunk
// tokens, or with `blocks` one selected block each); spans [pre_splits, S_total) cover
// the fp16 suffix in chunks of suf_chunk tokens, clipped to the causal limit.
// Partials (acc unnormalized against m, m and l in log2 units) go to
// part_acc [H_q*M][S_total][D], part_m / part_l [H_q*M][S_total]; the last workgroup
// of each y (ticket on counters[y], which must start at zero and is left at zero)
// merges them into out [H_q*M][D] and lse [H_q*M].
struct PartialParams {
  const uint16_t *Q;    // fp16 [H_q, M, D]
  int H_q, M;
  float qscale;         // log2(e) / sqrt(D)
  KVView kv;
  int pre_splits, pre_chunk;
  const int32_t *blocks;  // [H_kv, K_top] or null
  int K_top, B;
  const uint16_t *Ksuf, *Vsuf;  // fp16 [H_kv, S_suf, D]
  int S_suf, suf_chunk;
  int S_total;
  int x_begin;            // span index of this launch's blockIdx.x == 0
  float *part_acc, *part_m, *part_l;
  int *counters;          // [y_groups], zero between calls
  float *out, *lse;       // lse may be null
  RowGroups rg;
};

// q-head -> kv-head, for kernels that need the whole map.
struct HeadMap {
  int H_q;
  uint8_t m[kMaxHeads];
};


// Launches spans [x_begin, x_begin + x_count). mlx4_prefix selects the kernel that reads
// an mlx4g32 prefix (those spans must all be prefix spans); otherwise the fp16 kernel.
hipError_t launch_partial(const PartialParams &p, int rows_per_group, int y_groups,
                          int x_count, bool mlx4_prefix, hipStream_t s);
// Zero the ticket counters of a fresh workspace.
hipError_t launch_zero_counters(int *counters, int n, hipStream_t s);

hipError_t launch_quantize_mlx4g32(const uint16_t *x, int64_t rows, int D, uint32_t *codes,
                                   uint16_t *scales, uint16_t *biases, hipStream_t s);

// Block means of K (fp32 [H, nb, D]) for blocks of B tokens.
hipError_t launch_block_mean(const KVView &kv, int B, float *kmean, hipStream_t s);
// score [H_kv, nb] = sum over q-heads h of g of q_h . kmean[g, b]
hipError_t launch_block_score(const uint16_t *Q, const HeadMap &hm, const float *kmean,
                              int H_kv, int nb, int D, float *score, hipStream_t s);
// blocks [H_kv, K_top]: best min(K_top, nb) blocks per kv-head, ascending, -1 padded
hipError_t launch_block_topk(const float *score, int H_kv, int nb, int K_top,
                             int32_t *blocks, hipStream_t s);

}  // namespace pion
