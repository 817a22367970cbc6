// Dispatch kernels: the stable counting sort of dispatch_block.h, on one
// workgroup for small batches, over many (a count launch, then a scatter
// launch) for large ones; for batches routed by the standalone selection
// kernel.
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

__global__ __launch_bounds__(kDispatchThreads) void dispatch_count_kernel(const int32_t *__restrict__ idx, int n,
                                                                          int E, int32_t *__restrict__ cnt) {
  dispatch_count_block(idx, n, E, cnt);
}

__global__ __launch_bounds__(kDispatchThreads) void dispatch_scatter_kernel(
    const int32_t *__restrict__ idx, int n, int E, const int32_t *__restrict__ cnt, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_ids, int32_t *__restrict__ inv, int32_t *__restrict__ active,
    int32_t *__restrict__ n_active) {
  dispatch_scatter_block(idx, n, E, cnt, offsets, sorted_ids, inv, active, n_active);
}

}  // namespace

size_t dispatch_count_ints(int n, int E) {
  return n > kDispatchPerBlock ? (size_t)((n + kDispatchPerBlock - 1) / kDispatchPerBlock) * (E + 1) : 0;
}

hipError_t launch_dispatch(const int32_t *idx, int n, int E, int32_t *offsets, int32_t *sorted_ids,
                           int32_t *inv, int32_t *active, int32_t *n_active, int32_t *cnt, hipStream_t s) {
  if (n <= kDispatchPerBlock || !cnt)
    return launch(dispatch_kernel, 1, kDispatchThreads, 0, s, idx, n, E, offsets, sorted_ids, inv, active, n_active);
  const int nb = (n + kDispatchPerBlock - 1) / kDispatchPerBlock;
  const LaunchEvents ev = split_launch_events();  // profiled: both launches inside the pair
  launch_events = LaunchEvents{ev.start, nullptr};
  const hipError_t e = launch(dispatch_count_kernel, nb, kDispatchThreads, 0, s, idx, n, E, cnt);
  launch_events = LaunchEvents{nullptr, ev.stop};
  if (e != hipSuccess) {
    launch_events = LaunchEvents{nullptr, nullptr};
    return e;
  }
  return launch(dispatch_scatter_kernel, nb, kDispatchThreads, 0, s, idx, n, E, static_cast<const int32_t *>(cnt),
                offsets, sorted_ids, inv, active, n_active);
}

}  // namespace coli
