// Launch interface of the mlx4g32 encoder for a pair of tensors (the K and V of one
// store). Internal; the public interface is include/pion_prefix.h.
#pragma once

#include "kernels.h"

namespace pion {

// The encoder over two row sets of the same shape in one launch: rows [0, rows) of xa
// into (codes_a, sb_a) and of xb into (codes_b, sb_b), each group's (scale | bias << 16)
// as one 32-bit word (the slot layout). Equal to two launch_quantize_mlx4g32 calls with
// sb_stride 2, bit for bit.
hipError_t launch_quantize_mlx4g32_pair(const uint16_t *xa, uint32_t *codes_a, uint32_t *sb_a,
                                        const uint16_t *xb, uint32_t *codes_b, uint32_t *sb_b,
                                        int64_t rows, int D, hipStream_t s);

}  // namespace pion
