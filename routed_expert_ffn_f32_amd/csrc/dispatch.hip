// Dispatch kernel: the stable counting sort of dispatch_block.h on one
// workgroup, for batches routed by the standalone selection kernel.
#include "dispatch_block.h"

namespace coli {
namespace {

__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(const int32_t *__restrict__ idx, int n, int E,
                                                                    int32_t *__restrict__ offsets,
                                                                    int32_t *__restrict__ sorted_ids,
                                                                    int32_t *__restrict__ inv,
                                                                    int32_t *__restrict__ active,
                                                                    int32_t *__restrict__ n_active) {
  dispatch_block(idx, n, E, offsets, sorted_ids, inv, active, n_active);
}

}  // namespace

hipError_t launch_dispatch(const int32_t *idx, int n, int E, int32_t *offsets, int32_t *sorted_ids,
                           int32_t *inv, int32_t *active, int32_t *n_active, hipStream_t s) {
  return launch(dispatch_kernel, 1, kDispatchThreads, 0, s, idx, n, E, offsets, sorted_ids, inv, active, n_active);
}

}  // namespace coli
