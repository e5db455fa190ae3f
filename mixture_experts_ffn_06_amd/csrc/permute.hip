// Sort (token, slot) pairs by expert: histogram -> exclusive scan -> stable
// scatter.
//
// forward_prefill.rs (page 3, step 3 "Sort tokens by expert") produces
// sorted token ids, expert offsets and a token-to-slot map from the top-k
// indices; forward.rs (page 1) names the same step moe_route with counts,
// offsets, a cursor and pair<->slot maps.  A shared atomic cursor makes the
// order inside an expert run-dependent; here a pair's place inside its
// expert's segment is its rank among the earlier pairs (ascending
// p = t*k + j) with the same expert, so the result is one fixed permutation.
//
// One block of 16 waves.  Wave w owns a contiguous run of pairs and walks it
// 64 pairs at a time: a same-expert lane mask from one ballot per expert-id
// bit gives each lane its rank among equal experts of lower lanes, and a
// per-wave running count per expert (LDS, wave-private) turns it into the
// pair's rank inside the wave's run.  Per-wave counts are then scanned over
// waves and experts (expert offsets), and a second walk scatters every pair.
// Everything stays inside one block: no grid-wide hand-off, no atomics.
#include "common.h"
#include "kernels.h"
#include "routing.h"

namespace moe {

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int *__restrict__ topk_idx, int te, int E,
    int *__restrict__ counts, int *__restrict__ offsets,
    int *__restrict__ sorted_pair, int *__restrict__ slot_of_pair,
    int *__restrict__ lrank, int *__restrict__ active, int *__restrict__ nactive) {
  extern __shared__ int wcnt[];          // [kPermWaves][E]
  __shared__ int scan_tmp[kPermWaves];
  permute_block(topk_idx, te, E, wcnt, scan_tmp, counts, offsets, sorted_pair, slot_of_pair,
                lrank, active, nactive);
}

hipError_t launch_permute(const Dims &d, const int *topk_idx, const Work &w,
                          hipStream_t s) {
  const size_t lds = static_cast<size_t>(kPermWaves) * d.E * sizeof(int);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(permute_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kPermWaves * 1024 * static_cast<int>(sizeof(int)));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), lds, s, topk_idx,
                     d.te, d.E, w.counts, w.offsets, w.sorted_pair, w.slot_of_pair,
                     w.lrank, w.active, w.nactive);
  return hipGetLastError();
}

}  // namespace moe
