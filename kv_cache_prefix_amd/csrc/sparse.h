// Launch interface of the sparse-auto selection kernels (block means and the block
// score + top-K select). Internal; the public interface is include/pion_prefix.h.
#pragma once

#include "kernels.h"

namespace pion {

// Block means of K (fp32 [H, nb, D]) for blocks of B tokens.
hipError_t launch_block_mean(const KVView &kv, int B, float *kmean, hipStream_t s);
// blocks [H_kv, K_top]: per kv-head g the best min(K_top, nb) blocks by the score
// (sum over q-heads h of g of q_h) . kmean[g, b], ascending, -1 padded. Q: fp16 [H_q, D]
// (fp32 with q32). keys: scratch
// [H_kv, nb]; cand: scratch [H_kv, ceil(nb / 64), min(K_top, 64)]; counters[0, H_kv):
// zero before, left zero.
hipError_t launch_block_select(const void *Q, bool q32, const HeadMap &hm, const float *kmean,
                               int H_kv, int nb, int D, int K_top, uint32_t *keys,
                               uint64_t *cand, int *counters, int32_t *blocks, hipStream_t s);

}  // namespace pion
