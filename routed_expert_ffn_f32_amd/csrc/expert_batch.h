// Batched decode on the int8 matrix cores: int4 gs64 tables, batches above
// the small-batch limits and below the prefill threshold (expert_batch.hip).
#pragma once

#include "internal.h"

namespace coli {

// True when a batch of T tokens fits the launches below (every buffer
// offset within 31 bits, the grid within its limits).
bool batch_mfma_fits(int T, int k, int has_shared, int h, int I);

// Rows of `cols` float32 activations (cols a multiple of 64) as byte planes:
// per group of 64 columns a power-of-two scale and three balanced base-256
// digits of each column's 23-bit integer (expert_batch.hip describes the
// format).  planes [n][3][cols] bytes, scales [n][cols/64] float32.
hipError_t launch_batch_quantize(const float *src, int n, int cols, uint8_t *planes, float *scales,
                                 hipStream_t s);

// gate/up of every active slot on the byte planes of the hidden rows (P.xq
// and P.xs in the format above): midf [P][I] float32 for every assignment
// position (routed: p = sorted position; shared: p = T*k + t).
hipError_t launch_batch_gate_up(const DecodeProblem &P, hipStream_t s);

// down of every active slot on the byte planes of midf (P.mq and P.ms in the
// format above): y [P][h] float32 per assignment position.
hipError_t launch_batch_down(const DecodeProblem &P, hipStream_t s);

}  // namespace coli
