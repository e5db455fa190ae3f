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

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;   // 16

// Block-wide exclusive scan of one int per thread.
__device__ int block_exclusive_scan(int v, int *tmp /*[kPermWaves]*/, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kPermWaves; ++i) {
    const int c = tmp[i];
    base += i < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

// Mask of the lanes whose expert equals this lane's (among `valid` lanes).
__device__ __forceinline__ uint64_t same_expert_mask(int e, bool valid, int E) {
  uint64_t same = __ballot(valid);
  for (int b = 0; (1 << b) < E; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    same &= bit ? bb : ~bb;
  }
  return same;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int *__restrict__ topk_idx, int te, int E,
    int *__restrict__ counts, int *__restrict__ offsets,
    int *__restrict__ sorted_pair, int *__restrict__ slot_of_pair,
    int *__restrict__ lrank, int *__restrict__ active, int *__restrict__ nactive) {
  extern __shared__ int wcnt[];          // [kPermWaves][E]
  __shared__ int scan_tmp[kPermWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
  __syncthreads();

  // ---- pass 1: rank of each pair inside its wave's run ----
  const int per = (te + kPermWaves * 64 - 1) / (kPermWaves * 64) * 64;
  const int p0 = wave * per, p1 = min(te, p0 + per);
  int *mine = wcnt + wave * E;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint64_t above = (lane == 63) ? 0ull : (~0ull << (lane + 1));
  int e_next = (p0 + lane < p1) ? topk_idx[p0 + lane] : 0;
  for (int base = p0; base < p1; base += 64) {
    const int p = base + lane;
    const bool valid = p < p1;
    const int e = e_next;
    e_next = (p + 64 < p1) ? topk_idx[p + 64] : 0;   // prefetch the next group
    const uint64_t same = same_expert_mask(e, valid, E);
    const int cur = valid ? mine[e] : 0;
    const int r = cur + __popcll(same & below);
    if (valid) lrank[p] = r;
    if (valid && (same & above) == 0) mine[e] = r + 1;   // last lane of its group
  }
  __syncthreads();

  // ---- expert totals, offsets, per-wave bases ----
  constexpr int EPT = 1024 / kPermThreads;   // experts per thread (E <= 1024)
  (void)EPT;
  const int x = tid;                          // one expert per thread
  int tot = 0;
  if (x < E)
    for (int w = 0; w < kPermWaves; ++w) tot += wcnt[w * E + x];
  int all_pairs, all_active;
  const int off = block_exclusive_scan(x < E ? tot : 0, scan_tmp, &all_pairs);
  const int aoff = block_exclusive_scan(x < E && tot > 0 ? 1 : 0, scan_tmp, &all_active);
  if (x < E) {
    counts[x] = tot;
    offsets[x] = off;
    if (tot > 0) active[aoff] = x;
    int run = off;
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = wcnt[w * E + x];
      wcnt[w * E + x] = run;
      run += c;
    }
  }
  if (tid == 0) {
    offsets[E] = all_pairs;
    *nactive = all_active;
  }
  __syncthreads();

  // ---- pass 2: scatter (each thread rereads the ranks it wrote) ----
  for (int base = p0; base < p1; base += 64) {
    const int p = base + lane;
    if (p < p1) {
      const int e = topk_idx[p];
      const int pos = mine[e] + lrank[p];
      sorted_pair[pos] = p;
      slot_of_pair[p] = pos;
    }
  }
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
