// Batched decode on the int8 matrix cores: int4 gs64 tables, batches above
// the small-batch limits and below the prefill threshold (expert_batch.hip).
#pragma once

#include "internal.h"

namespace coli {

// True when a batch of T tokens fits the launches below (every buffer
// offset within 31 bits, the grid within its limits).
bool batch_mfma_fits(int T, int k, int has_shared, int h, int I);

// gate/up of every active slot on the byte planes of the hidden rows (P.xq
// and P.xs, written by the router launch; format in byte_planes.h and
// expert_batch.hip): the byte planes of mid (P.mq [P][3I] bytes, P.ms
// [P][I/64]) for every assignment position (routed: p = sorted position;
// shared: p = T*k + t).  I a multiple of 64.
hipError_t launch_batch_gate_up(const DecodeProblem &P, hipStream_t s);

// down of every active slot on the byte planes of mid (P.mq and P.ms): y
// [P][h] float32 per assignment position.
hipError_t launch_batch_down(const DecodeProblem &P, hipStream_t s);

}  // namespace coli
