// Sort (token, slot) pairs by expert: histogram -> exclusive scan -> stable
// scatter, plus the M-tile list of the grouped GEMM.
//
// forward_prefill.rs (page 3, step 3 "Sort tokens by expert") produces
// sorted token ids, expert offsets and a token-to-slot map from the top-k
// indices; forward.rs (page 1) names the same step moe_route with counts,
// offsets, a cursor and pair<->slot maps.  A shared atomic cursor makes the
// order inside an expert run-dependent; here a pair's place inside its
// expert's segment is its rank among the earlier pairs (ascending
// p = t*k + j) with the same expert, so the result is one fixed permutation.
//
// One launch.  Every block ranks one chunk of kPermuteChunk pairs: per wave a
// same-expert lane mask is built from one ballot per expert-id bit, the rank
// is a popcount of the lower lanes, and per-wave counts are prefix-summed
// over the chunk's waves in LDS.  The block then publishes its per-expert
// counts and takes a ticket; the last block to finish scans counts over
// chunks and experts, scatters every pair, and writes the tile list.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPermThreads = kPermuteChunk;          // one pair per thread
constexpr int kPermWaves = kPermThreads / kWave;     // 16
constexpr int kScanLds = 6144;                       // ints for chunk bases

int permute_chunks(int te) { return (te + kPermuteChunk - 1) / kPermuteChunk; }

// Block-wide exclusive scan of one int per thread (1024 threads).
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

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int *__restrict__ topk_idx, int te, int E, int G, int bm,
    int m_shared, int *__restrict__ counts, int *__restrict__ offsets,
    int *__restrict__ sorted_pair, int *__restrict__ slot_of_pair,
    int *__restrict__ blk, int *__restrict__ lrank, unsigned *ticket,
    int2 *__restrict__ tiles, int *__restrict__ ntiles,
    int *__restrict__ active, int *__restrict__ nactive) {
  __shared__ uint16_t wcnt[kPermWaves * 1024];   // per-wave counts, E <= 1024
  __shared__ int scan_tmp[kPermWaves];
  __shared__ int base_lds[kScanLds];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- phase 1: rank pairs inside this chunk ----
  for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
  __syncthreads();
  const int p = blockIdx.x * kPermuteChunk + tid;
  const bool valid = p < te;
  const int e = valid ? topk_idx[p] : 0;
  uint64_t same = __ballot(valid);
  for (int b = 0; (1 << b) < E; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    same &= bit ? bb : ~bb;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(same & below);
  const uint64_t above = (lane == 63) ? 0ull : (~0ull << (lane + 1));
  if (valid && (same & above) == 0) wcnt[wave * E + e] = static_cast<uint16_t>(rank + 1);
  __syncthreads();
  for (int x = tid; x < E; x += kPermThreads) {
    int run = 0;
    for (int wv = 0; wv < kPermWaves; ++wv) {
      const int c = wcnt[wv * E + x];
      wcnt[wv * E + x] = static_cast<uint16_t>(run);
      run += c;
    }
    blk[static_cast<size_t>(blockIdx.x) * E + x] = run;
  }
  __syncthreads();
  if (valid) lrank[p] = wcnt[wave * E + e] + rank;

  // ---- hand-off: the last chunk to finish does the global part ----
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev == static_cast<unsigned>(G - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // ---- phase 2: per-expert totals, chunk bases (relative), expert scan ----
  // blk[g][x] <- sum_{g' < g} blk[g'][x]; processed in slabs of chunks so the
  // loads of one slab are independent.
  int tot = 0;  // thread x < E: running total of expert x
  const int slab = kScanLds / E;  // chunks per slab (>= 6 for E <= 1024)
  for (int g0 = 0; g0 < G; g0 += slab) {
    const int gn = min(slab, G - g0);
    for (int i = tid; i < gn * E; i += kPermThreads)
      base_lds[i] = blk[static_cast<size_t>(g0) * E + i];
    __syncthreads();
    for (int x = tid; x < E; x += kPermThreads) {
      for (int g = 0; g < gn; ++g) {
        const int c = base_lds[g * E + x];
        base_lds[g * E + x] = tot;
        tot += c;
      }
    }
    __syncthreads();
    for (int i = tid; i < gn * E; i += kPermThreads)
      blk[static_cast<size_t>(g0) * E + i] = base_lds[i];
    __syncthreads();
  }
  // exclusive scans over experts (E <= 1024: one expert per thread)
  const int cnt = tid < E ? tot : 0;
  int all_pairs, all_tiles, all_active;
  const int off = block_exclusive_scan(cnt, scan_tmp, &all_pairs);
  const int nt = (cnt + bm - 1) / bm;
  const int toff = block_exclusive_scan(nt, scan_tmp, &all_tiles);
  const int aoff = block_exclusive_scan(cnt > 0 ? 1 : 0, scan_tmp, &all_active);
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = off;
    base_lds[tid] = off;   // reuse: expert offsets for the scatter
    if (cnt > 0) active[aoff] = tid;
    for (int i = 0; i < nt; ++i) tiles[toff + i] = make_int2(tid, i * bm);
  }
  if (tid == 0) {
    offsets[E] = all_pairs;
    const int sh_tiles = (m_shared + bm - 1) / bm;
    for (int i = 0; i < sh_tiles; ++i) tiles[all_tiles + i] = make_int2(E, i * bm);
    *ntiles = all_tiles + sh_tiles;
    *nactive = all_active;
  }
  __syncthreads();
  __threadfence();

  // ---- phase 3: scatter every pair ----
  for (int q = tid; q < te; q += kPermThreads) {
    const int eq = topk_idx[q];
    const int g = q / kPermuteChunk;
    const int pos = base_lds[eq] + blk[static_cast<size_t>(g) * E + eq] + lrank[q];
    sorted_pair[pos] = q;
    slot_of_pair[q] = pos;
  }
  if (tid == 0) *ticket = 0u;
}

hipError_t launch_permute(const Dims &d, const int *topk_idx, const Work &w,
                          int max_tiles, hipStream_t s) {
  (void)max_tiles;
  const int G = permute_chunks(d.te);
  const int m_shared = d.Is > 0 ? d.m : 0;
  hipLaunchKernelGGL(permute_kernel, dim3(G), dim3(kPermThreads), 0, s,
                     topk_idx, d.te, d.E, G, d.bm, m_shared, w.counts,
                     w.offsets, w.sorted_pair, w.slot_of_pair, w.blk, w.lrank,
                     w.ticket, w.tiles, w.ntiles, w.active, w.nactive);
  return hipGetLastError();
}

}  // namespace moe
