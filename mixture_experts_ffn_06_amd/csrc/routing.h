// Gating + top-k and the stable sort by expert as device functions, shared by
// their own kernels and by the fused single-block routing kernel.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Gating + top-k of one token by one wave (router.hip describes the gating).
// Lane l holds experts l, l+64, ...  Experts are ranked by score + bias:
// softmax without a bias ranks by the logit itself (same order as the
// probability, without its rounding), softmax with a bias by p + bias, p the
// fp32 probability over all E; sigmoid by 1/(1+e^-l) + bias; sqrtsoftplus by
// sqrt(softplus(l)) + bias.  Equal scores: lower expert index first.
//
// Selection without cross-lane shuffles: scores become order-preserving
// 32-bit keys, and the k-th largest key T is found bit by bit from the top
// (keep a bit if at least k keys reach the prefix; each count is a ballot
// and a popcount).  Keys above T are selected, then keys equal to T in
// ascending expert order until k are taken.  The k selected (key, expert,
// logit) go to LDS; lane j < k counts the selected entries that precede its
// own (larger key, or equal key and lower index), which is its output
// position, and the entries are re-read in that order.
//
// lrow may point to global memory or LDS; sk is LDS of kTopkScratch words
// owned by the wave; idx_copy, if not null, receives the k indices too.
constexpr int kMaxEPerLane = 16;  // E <= 1024
constexpr int kTopkScratch = 3 * 32;

// Unsigned key with the order of the float (-0 taken as +0, so equal scores
// stay equal and fall back to the index order).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// sqrt(ln(1 + e^l)), with softplus written as max(l, 0) + ln(1 + e^-|l|) so
// that e^l never overflows.
__device__ __forceinline__ float sqrt_softplus(float l) {
  return sqrtf(fmaxf(l, 0.0f) + log1pf(expf(-fabsf(l))));
}

template <int EPL>
__device__ __forceinline__ void topk_token(const float *lrow, int E, int k, int gating,
                                           int renorm, float scale, const float *bias,
                                           int *idx_out, float *w_out, int *idx_copy,
                                           uint32_t *sk) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  float l[EPL];
  uint32_t key[EPL];
  bool valid[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    valid[i] = e < E;
    l[i] = valid[i] ? lrow[e] : 0.f;
  }
  // softmax over all E: its maximum and normaliser, needed to rank with a
  // bias and for unrenormalised weights
  float lmax = -INFINITY, z = 1.f;
  if (gating == 0 && (bias || !renorm)) {
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (valid[i]) lmax = fmaxf(lmax, l[i]);
    lmax = wave_max(lmax);
    z = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (valid[i]) z += expf(l[i] - lmax);
    z = wave_sum(z);
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    float c = l[i];
    if (gating == 0) {
      if (bias) c = expf(l[i] - lmax) / z;
    } else if (gating == 1) {
      c = 1.0f / (1.0f + expf(-l[i]));
    } else {
      c = sqrt_softplus(l[i]);
    }
    if (bias) c += valid[i] ? bias[e] : 0.f;
    key[i] = valid[i] ? order_key(c) : 0u;
  }
  // T = the largest value with at least k keys >= T (the k-th largest key),
  // two bits per step: of the candidates T | d << b (d = 3, 2, 1, 0) the
  // largest that at least k keys reach (d = 0 always does); the three counts
  // are independent, so the serial chain is 16 steps instead of 32
  uint32_t T = 0;
  for (int b = 30; b >= 0; b -= 2) {
    const uint32_t t1 = T | (1u << b), t2 = T | (2u << b), t3 = T | (3u << b);
    int c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      c1 += __popcll(__ballot(valid[i] && key[i] >= t1));
      c2 += __popcll(__ballot(valid[i] && key[i] >= t2));
      c3 += __popcll(__ballot(valid[i] && key[i] >= t3));
    }
    T = c3 >= k ? t3 : c2 >= k ? t2 : c1 >= k ? t1 : T;
  }
  int need = k;
#pragma unroll
  for (int i = 0; i < EPL; ++i) need -= __popcll(__ballot(valid[i] && key[i] > T));
  // selection, then compaction into LDS in ascending expert order
  int base = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const uint64_t eq = __ballot(valid[i] && key[i] == T);
    const bool take_eq = ((eq >> lane) & 1ull) && __popcll(eq & below) < need;
    need -= min(need, __popcll(eq));
    const bool sel = (valid[i] && key[i] > T) || take_eq;
    const uint64_t sm = __ballot(sel);
    if (sel) {
      const int pos = base + __popcll(sm & below);
      sk[pos] = key[i];
      sk[32 + pos] = static_cast<uint32_t>(lane + kWave * i);
      sk[64 + pos] = __float_as_uint(l[i]);
    }
    base += __popcll(sm);
  }
  __builtin_amdgcn_wave_barrier();
  // output position of entry j = number of entries ranked before it
  uint32_t my_key = 0, my_idx = 0, my_lbits = 0;
  int rank = 0;
  if (lane < k) {
    my_key = sk[lane];
    my_idx = sk[32 + lane];
    my_lbits = sk[64 + lane];
    for (int j = 0; j < k; ++j) {
      const uint32_t ok = sk[j], oi = sk[32 + j];
      rank += (ok > my_key || (ok == my_key && oi < my_idx)) ? 1 : 0;
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < k) {
    sk[rank] = my_idx;
    sk[32 + rank] = my_lbits;
  }
  __builtin_amdgcn_wave_barrier();
  // lane j < k: expert chosen j-th, and its logit
  const int my_e = lane < k ? static_cast<int>(sk[lane]) : -1;
  const float my_l = lane < k ? __uint_as_float(sk[32 + lane]) : 0.f;
  // Gate weights of the selected experts.
  float wj = 0.f;
  if (gating == 0) {
    if (renorm) {
      // softmax of the selected logits, shifted by their largest
      const float l0 = wave_max(lane < k ? my_l : -INFINITY);
      const float ex = lane < k ? expf(my_l - l0) : 0.f;
      wj = ex / wave_sum(ex);
    } else {
      wj = expf(my_l - lmax) / z;
    }
  } else {
    float sj = 0.f;
    if (lane < k) sj = gating == 1 ? 1.0f / (1.0f + expf(-my_l)) : sqrt_softplus(my_l);
    wj = renorm ? sj / wave_sum(sj) : sj;
  }
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = wj * scale;
    if (idx_copy) idx_copy[lane] = my_e;
  }
}

// ---------------------------------------------------------------------------
// Stable sort of the te = m*k (token, slot) pairs by expert (permute.hip
// describes the method) by one block of kPermThreads threads.  topk_idx may
// point to global memory or LDS; wcnt is LDS of kPermWaves * E ints and
// scan_tmp LDS of kPermWaves ints.
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;   // 16

// Block-wide exclusive scan of one int per thread.
__device__ __forceinline__ int block_exclusive_scan(int v, int *tmp /*[kPermWaves]*/, int *total) {
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

// Pass 1 over the pairs [c0, c1): each wave takes a contiguous run and walks
// it 64 pairs at a time; a pair's rank among the earlier pairs of the same
// expert in its wave's run goes to lrank[p], the run's count per expert to
// wcnt[wave][e] (wcnt is zeroed here).
__device__ __forceinline__ void chunk_ranks(const int *topk_idx, int c0, int c1, int E, int *wcnt,
                                            int *__restrict__ lrank) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
  __syncthreads();
  const int n = c1 - c0;
  const int per = (n + kPermWaves * 64 - 1) / (kPermWaves * 64) * 64;
  const int p0 = c0 + wave * per, p1 = min(c1, p0 + per);
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
}

// Turns the per-wave counts of chunk_ranks into start positions, the runs of
// each expert following base[e] in wave order (thread x: expert x).
__device__ __forceinline__ void chunk_bases(int E, int *wcnt, int base_x) {
  const int x = threadIdx.x;
  if (x < E) {
    int run = base_x;
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = wcnt[w * E + x];
      wcnt[w * E + x] = run;
      run += c;
    }
  }
  __syncthreads();
}

// Pass 2 over [c0, c1): every thread rereads the ranks it wrote.
__device__ __forceinline__ void chunk_scatter(const int *topk_idx, int c0, int c1, int E, const int *wcnt,
                                              const int *__restrict__ lrank, int *__restrict__ sorted_pair,
                                              int *__restrict__ slot_of_pair) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = c1 - c0;
  const int per = (n + kPermWaves * 64 - 1) / (kPermWaves * 64) * 64;
  const int p0 = c0 + wave * per, p1 = min(c1, p0 + per);
  const int *mine = wcnt + wave * E;
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

// Expert totals -> counts, offsets, the active list and, per active slot,
// the prefix of its 16-row blocks (rboff[s] = sum over the active slots
// before s of ceil(rows / 16), rboff[nactive] = their total: the
// small-batch kernels' items), and zeroes the GEMMs' unit queues; returns
// offsets[x] for thread x (E <= kPermThreads).
__device__ __forceinline__ int expert_offsets(int tot, int E, int *scan_tmp, int *__restrict__ counts,
                                              int *__restrict__ offsets, int *__restrict__ active,
                                              int *__restrict__ nactive, int *__restrict__ rboff,
                                              int *__restrict__ queue) {
  const int x = threadIdx.x;
  if (x < kQueueInts / kQueueStride) queue[kQueueStride * x] = 0;
  int all_pairs, all_active, all_rb;
  const int off = block_exclusive_scan(x < E ? tot : 0, scan_tmp, &all_pairs);
  const int aoff = block_exclusive_scan(x < E && tot > 0 ? 1 : 0, scan_tmp, &all_active);
  const int rb = block_exclusive_scan(x < E ? (tot + 15) >> 4 : 0, scan_tmp, &all_rb);
  if (x < E) {
    counts[x] = tot;
    offsets[x] = off;
    if (tot > 0) {
      active[aoff] = x;
      rboff[aoff] = rb;
    }
  }
  if (x == 0) {
    offsets[E] = all_pairs;
    *nactive = all_active;
    rboff[all_active] = all_rb;
  }
  return off;
}

// The whole sort by one wave, for the few pairs of a decode-sized batch (no
// block barriers).  Pairs are ranked 64 at a time in pair order (the rank of
// a pair among the earlier pairs of its expert: running counts in cnt, LDS
// of E ints), the expert totals are scanned by the wave (lane l takes
// experts [l P, l P + P), P = ceil(E / 64)), and each pair goes to its
// expert's start plus its rank: the same stable order as permute_block.
// lrank: te ints of LDS or global memory.  Also zeroes the GEMMs' unit
// queues.
__device__ __forceinline__ void permute_wave(
    const int *topk_idx, int te, int E, int *cnt, int *__restrict__ lrank,
    int *__restrict__ counts, int *__restrict__ offsets, int *__restrict__ sorted_pair,
    int *__restrict__ slot_of_pair, int *__restrict__ active, int *__restrict__ nactive,
    int *__restrict__ rboff, int *__restrict__ queue) {
  const int lane = threadIdx.x & 63;
  if (lane < kQueueInts / kQueueStride) queue[kQueueStride * lane] = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint64_t above = (lane == 63) ? 0ull : (~0ull << (lane + 1));
  for (int e = lane; e < E; e += kWave) cnt[e] = 0;
  __builtin_amdgcn_wave_barrier();
  for (int base = 0; base < te; base += kWave) {
    const int p = base + lane;
    const bool valid = p < te;
    const int e = valid ? topk_idx[p] : 0;
    const uint64_t same = same_expert_mask(e, valid, E);
    const int r = (valid ? cnt[e] : 0) + __popcll(same & below);
    if (valid) lrank[p] = r;
    __builtin_amdgcn_wave_barrier();
    if (valid && (same & above) == 0) cnt[e] = r + 1;   // last lane of its group
    __builtin_amdgcn_wave_barrier();
  }
  // totals -> starts, the active list and the 16-row block prefix
  const int per = (E + kWave - 1) / kWave;
  const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
  int tot = 0, act = 0, rb = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    tot += c;
    act += c > 0 ? 1 : 0;
    rb += (c + 15) >> 4;
  }
  int itot = tot, iact = act, irb = rb;   // inclusive scans over the lanes
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int a = __shfl_up(itot, o), b = __shfl_up(iact, o), c = __shfl_up(irb, o);
    if (lane >= o) {
      itot += a;
      iact += b;
      irb += c;
    }
  }
  const int all_pairs = __shfl(itot, kWave - 1), all_active = __shfl(iact, kWave - 1),
            all_rb = __shfl(irb, kWave - 1);
  int off = itot - tot, aoff = iact - act, rbo = irb - rb;
  __builtin_amdgcn_wave_barrier();
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    counts[e] = c;
    offsets[e] = off;
    if (c > 0) {
      active[aoff] = e;
      rboff[aoff] = rbo;
      ++aoff;
      rbo += (c + 15) >> 4;
    }
    cnt[e] = off;   // cnt now holds the expert's first position
    off += c;
  }
  if (lane == 0) {
    offsets[E] = all_pairs;
    *nactive = all_active;
    rboff[all_active] = all_rb;
  }
  __builtin_amdgcn_wave_barrier();
  for (int p = lane; p < te; p += kWave) {
    const int pos = cnt[topk_idx[p]] + lrank[p];
    sorted_pair[pos] = p;
    slot_of_pair[p] = pos;
  }
}

// The whole sort in one block.
__device__ __forceinline__ void permute_block(
    const int *topk_idx, int te, int E, int *wcnt, int *scan_tmp,
    int *__restrict__ counts, int *__restrict__ offsets,
    int *__restrict__ sorted_pair, int *__restrict__ slot_of_pair,
    int *__restrict__ lrank, int *__restrict__ active, int *__restrict__ nactive, int *__restrict__ rboff,
    int *__restrict__ queue) {
  chunk_ranks(topk_idx, 0, te, E, wcnt, lrank);
  const int x = threadIdx.x;
  int tot = 0;
  if (x < E)
    for (int w = 0; w < kPermWaves; ++w) tot += wcnt[w * E + x];
  const int off = expert_offsets(tot, E, scan_tmp, counts, offsets, active, nactive, rboff, queue);
  chunk_bases(E, wcnt, off);
  chunk_scatter(topk_idx, 0, te, E, wcnt, lrank, sorted_pair, slot_of_pair);
}

}  // namespace moe
