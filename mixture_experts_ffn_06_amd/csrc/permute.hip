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
#include "launch.h"
#include "routing.h"

namespace moe {

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int *__restrict__ topk_idx, int te, int E,
    int *__restrict__ counts, int *__restrict__ offsets,
    int *__restrict__ sorted_pair, int *__restrict__ slot_of_pair,
    int *__restrict__ lrank, int *__restrict__ active, int *__restrict__ nactive, int *__restrict__ rboff,
    int *__restrict__ queue) {
  extern __shared__ int wcnt[];          // [kPermWaves][E]
  __shared__ int scan_tmp[kPermWaves];
  permute_block(topk_idx, te, E, wcnt, scan_tmp, counts, offsets, sorted_pair, slot_of_pair,
                lrank, active, nactive, rboff, queue);
}

// ---------------------------------------------------------------------------
// Many pairs (te >= kPermMultiMin): the same sort over chunks of `chunk`
// consecutive pairs, one block per chunk, in three launches:
//   1. each block counts its chunk's pairs per expert (blk[b][e]);
//   2. one block turns the counts into expert totals, offsets, the active
//      list, and every (chunk, expert) start: offsets[e] plus the counts of
//      that expert in the earlier chunks;
//   3. each block ranks its chunk as the single-block sort does and scatters
//      from its starts.
// Chunks are contiguous ranges of p in chunk order, so the result is the
// same stable permutation as the single-block sort.
__global__ __launch_bounds__(kPermThreads) void permute_hist_kernel(const int *__restrict__ topk_idx, int te,
                                                                    int E, int chunk, int *__restrict__ blk) {
  extern __shared__ int hist[];   // [E]
  for (int i = threadIdx.x; i < E; i += kPermThreads) hist[i] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * chunk, c1 = min(te, c0 + chunk);
  for (int p = c0 + threadIdx.x; p < c1; p += kPermThreads) atomicAdd(&hist[topk_idx[p]], 1);
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kPermThreads) blk[static_cast<size_t>(blockIdx.x) * E + i] = hist[i];
}

__global__ __launch_bounds__(kPermThreads) void permute_scan_kernel(int nblk, int E, int *__restrict__ blk,
                                                                    int *__restrict__ counts, int *__restrict__ offsets,
                                                                    int *__restrict__ active, int *__restrict__ nactive,
                                                                    int *__restrict__ rboff, int *__restrict__ queue) {
  __shared__ int scan_tmp[kPermWaves];
  const int x = threadIdx.x;
  int tot = 0;
  if (x < E)
    for (int b = 0; b < nblk; ++b) tot += blk[static_cast<size_t>(b) * E + x];
  const int off = expert_offsets(tot, E, scan_tmp, counts, offsets, active, nactive, rboff, queue);
  if (x < E) {
    int run = off;
    for (int b = 0; b < nblk; ++b) {
      const int c = blk[static_cast<size_t>(b) * E + x];
      blk[static_cast<size_t>(b) * E + x] = run;
      run += c;
    }
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int *__restrict__ topk_idx, int te, int E, int chunk, const int *__restrict__ blk,
    int *__restrict__ sorted_pair, int *__restrict__ slot_of_pair, int *__restrict__ lrank) {
  extern __shared__ int wcnt[];   // [kPermWaves][E]
  const int c0 = blockIdx.x * chunk, c1 = min(te, c0 + chunk);
  chunk_ranks(topk_idx, c0, c1, E, wcnt, lrank);
  const int x = threadIdx.x;
  chunk_bases(E, wcnt, x < E ? blk[static_cast<size_t>(blockIdx.x) * E + x] : 0);
  chunk_scatter(topk_idx, c0, c1, E, wcnt, lrank, sorted_pair, slot_of_pair);
}

hipError_t launch_permute(const Dims &d, const int *topk_idx, const Work &w,
                          hipStream_t s) {
  const size_t lds = static_cast<size_t>(kPermWaves) * d.E * sizeof(int);
  static const hipError_t su = [] {
    for (const void *k : {reinterpret_cast<const void *>(permute_kernel),
                          reinterpret_cast<const void *>(permute_scatter_kernel)}) {
      const hipError_t e = lds_setup(k, kPermWaves * 1024 * static_cast<int>(sizeof(int)));
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (su != hipSuccess) return su;
  const int nblk = permute_chunks(d.te), chunk = perm_chunk(d.te);
  if (nblk == 0) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), lds, s, topk_idx,
                       d.te, d.E, w.counts, w.offsets, w.sorted_pair, w.slot_of_pair,
                       w.lrank, w.active, w.nactive, w.rboff, w.queue);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nblk), dim3(kPermThreads), d.E * sizeof(int), s,
                     topk_idx, d.te, d.E, chunk, w.perm_blk);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kPermThreads), 0, s, nblk, d.E, w.perm_blk,
                     w.counts, w.offsets, w.active, w.nactive, w.rboff, w.queue);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(kPermThreads), lds, s, topk_idx, d.te, d.E,
                     chunk, w.perm_blk, w.sorted_pair, w.slot_of_pair, w.lrank);
  return hipGetLastError();
}

}  // namespace moe
