// Launch interface of the grouped-query MFMA kernel (attn_gqa_mfma.hip). Internal; the
// public interface is include/pion_prefix.h.
#pragma once

#include "kernels.h"

namespace pion {

constexpr int kGqaMaxRows = kRowsPerGroup;  // q-heads per row group
constexpr int kGqaMaxSegs = 64;             // key segments per span

// The spans [x_begin, x_begin + x_count) of every problem of `p` (fp16 slots, M = 1,
// row groups of up to kGqaMaxRows q-heads, seg_per_span <= kGqaMaxSegs), with the
// results and merge of launch_partial.
hipError_t launch_gqa_mfma(const PartialParams &p, int x_count, hipStream_t s);

}  // namespace pion
