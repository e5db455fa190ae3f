// Router product and gating + top-k.
//
// Router logits l[t,e] = sum_h x[t,h] * Wr[e,h], accumulated in fp32
// (forward_prefill.rs, page 3, step 1 "Gate GEMM"; the page keeps this
// product on its own scalar kernel because a different reduction order flips
// top-k choices on borderline tokens -- selection numerics are part of the
// contract, so this file fixes one reduction order per path).
//
// Gating (page 3, step 2 "Batched topK dispatch"): softmax over all E with
// optional renormalisation over the k selected (norm_topk_prob), or sigmoid
// scores ranked with a selection-only bias, renormalised and multiplied by the
// routed scaling factor.
#include "common.h"
#include "kernels.h"
#include "launch.h"
#include "routing.h"

namespace moe {

// ---------------------------------------------------------------------------
// VALU router: one wave per expert, kRouterTok tokens per block.
// Lane l accumulates the h = l, l+64, ... terms; a wave reduction finishes.
constexpr int kRouterTok = 16;
constexpr int kRouterWaves = 4;

template <int DT>
__global__ __launch_bounds__(256) void router_valu_kernel(
    const void *__restrict__ x, const void *__restrict__ wr,
    float *__restrict__ logits, int m, int E, int H) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kRouterWaves + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * kRouterTok;
  if (e >= E) return;
  const int nt = min(kRouterTok, m - t0);
  float acc[kRouterTok];
#pragma unroll
  for (int i = 0; i < kRouterTok; ++i) acc[i] = 0.f;
  for (int h = lane; h < H; h += kWave) {
    const float wv = load_as_f32<DT>(wr, static_cast<size_t>(e) * H + h);
#pragma unroll
    for (int i = 0; i < kRouterTok; ++i)
      if (i < nt) acc[i] = fmaf(load_as_f32<DT>(x, static_cast<size_t>(t0 + i) * H + h), wv, acc[i]);
  }
#pragma unroll
  for (int i = 0; i < kRouterTok; ++i) {
    const float v = wave_sum(acc[i]);
    if (lane == 0 && i < nt) logits[static_cast<size_t>(t0 + i) * E + e] = v;
  }
}

// ---------------------------------------------------------------------------
// MFMA router for bf16: a block computes 16*MBW tokens x 16*NBW experts with
// its NW waves (4, or 8 for the largest tiles) splitting H; each wave
// streams its K range of the token and expert rows straight into MFMA
// operands (16x16x32 bf16, fp32 accumulate) and the NW partial tiles are
// summed through LDS in a fixed order (wave 0's, then 1, 2, ...).  Small
// tiles keep enough blocks in flight at decode sizes; larger ones cut the
// re-reads of x and Wr at prefill sizes.
//
// With SPLIT (m <= 16 * MBW): blockIdx.y picks one of gridDim.y K ranges and
// the block writes its partial tile to logits + blockIdx.y * m * E.
//
// With QUANT (fp8 layers, H a multiple of 512): the pass over x also
// quantises it for the expert GEMMs (the quant_x_kernel rule: per token per
// 128 columns, scale = amax / 448, code = round-to-nearest-even of x /
// scale, an all-zero group gets scale 1).  Each wave's K range is then whole
// 128-column groups and one batch of four 32-wide steps is one group: the
// four lanes of a token row hold its 128 values.  Group g is written by the
// block of expert tile g % (expert tiles) (every expert tile reads the same
// x rows), so the quantisation work is spread over all blocks.
template <int MBW, int NBW, bool SPLIT, bool QUANT = false, int NW = 4>
__global__ __launch_bounds__(NW * 64) void router_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    float *__restrict__ logits, int m, int E, int H,
    uint8_t *__restrict__ xq = nullptr, float *__restrict__ sx = nullptr) {
  __shared__ f32x4_t part[NW - 1][MBW * NBW][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Without SPLIT the grid is one-dimensional: block b runs on XCD b % 8
  // (blocks are dealt to the XCDs round-robin), and the ne expert tiles of a
  // token tile go to consecutive slots of one XCD, so its x rows come from
  // HBM once and from that XCD's L2 for the other expert tiles.
  const int ne = SPLIT ? static_cast<int>(gridDim.x) : (E + 16 * NBW - 1) / (16 * NBW);
  int et = blockIdx.x, tt = SPLIT ? 0 : static_cast<int>(blockIdx.y);
  if (!SPLIT) {
    const int j = static_cast<int>(blockIdx.x) >> 3;
    et = j % ne;
    tt = (j / ne) * 8 + (static_cast<int>(blockIdx.x) & 7);
    if (tt * 16 * MBW >= m) return;
  }
  const int t0 = SPLIT ? 0 : tt * 16 * MBW, e0 = et * 16 * NBW;
  if (SPLIT) logits += static_cast<size_t>(blockIdx.y) * m * E;
  const int kofs = (lane >> 4) * 8;
  const uint16_t *ap[MBW];
  const uint16_t *bp[NBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
    ap[i] = x + static_cast<size_t>(min(t0 + 16 * i + (lane & 15), m - 1)) * H + kofs;
#pragma unroll
  for (int j = 0; j < NBW; ++j)
    bp[j] = wr + static_cast<size_t>(min(e0 + 16 * j + (lane & 15), E - 1)) * H + kofs;
  f32x4_t acc[MBW][NBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int steps = H / 32;
  const int parts = SPLIT ? NW * gridDim.y : NW, part_id = SPLIT ? NW * blockIdx.y + wave : wave;
  const int s0 = steps * part_id / parts, s1 = steps * (part_id + 1) / parts;
  constexpr int BATCH = 4;
  for (int s = s0; s < s1; s += BATCH) {
    uint4 av[BATCH][MBW], bv[BATCH][NBW];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const bool in = s + q < s1;
      const int o = (s + q) * 32;
#pragma unroll
      for (int i = 0; i < MBW; ++i)
        av[q][i] = in ? *reinterpret_cast<const uint4 *>(ap[i] + o) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        bv[q][j] = in ? *reinterpret_cast<const uint4 *>(bp[j] + o) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q)
#pragma unroll
      for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, av[q][i]), __builtin_bit_cast(bf16x8_t, bv[q][j]),
              acc[i][j], 0, 0, 0);
    if constexpr (QUANT) {
      const int g = s >> 2;   // this batch's 128-column group
      if (g % ne == et) {
#pragma unroll
        for (int i = 0; i < MBW; ++i) {
          float v[BATCH][8];
          float am = 0.f;
#pragma unroll
          for (int q = 0; q < BATCH; ++q) {
            const uint32_t u[4] = {av[q][i].x, av[q][i].y, av[q][i].z, av[q][i].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              v[q][2 * c] = bf16_to_f32(static_cast<uint16_t>(u[c] & 0xffffu));
              v[q][2 * c + 1] = bf16_to_f32(static_cast<uint16_t>(u[c] >> 16));
              am = fmaxf(am, fmaxf(fabsf(v[q][2 * c]), fabsf(v[q][2 * c + 1])));
            }
          }
          am = fmaxf(am, __shfl_xor(am, 16));   // the four lanes of this token row
          am = fmaxf(am, __shfl_xor(am, 32));
          const float sc = am > 0.f ? am / kE4M3Max : 1.0f;
          const int t = t0 + 16 * i + (lane & 15);
          if (t < m) {
#pragma unroll
            for (int q = 0; q < BATCH; ++q) {
              uint32_t c[4];
#pragma unroll
              for (int h = 0; h < 4; ++h)
                c[h] = static_cast<uint32_t>(fp8_pack2(v[q][2 * h] / sc, v[q][2 * h + 1] / sc)) & 0xffffu;
              *reinterpret_cast<uint2 *>(xq + static_cast<size_t>(t) * H + (s + q) * 32 + kofs) =
                  make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
            }
            if ((lane >> 4) == 0) sx[static_cast<size_t>(t) * (H / kQBlock) + g] = sc;
          }
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) part[wave - 1][i * NBW + j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      f32x4_t v = acc[i][j];
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) v += part[w][i * NBW + j][lane];
      const int e = e0 + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * i + (lane >> 4) * 4 + r;
        if (t < m && e < E) logits[static_cast<size_t>(t) * E + e] = v[r];
      }
    }
}

template <int MBW, int NBW, int NW = 4>
static hipError_t launch_router_mfma(const Dims &d, const Inputs &in, const Work &w,
                                     hipStream_t s) {
  // one-dimensional: ne expert tiles x the token tiles rounded up to 8
  const int ne = (d.E + 16 * NBW - 1) / (16 * NBW), nt = (d.m + 16 * MBW - 1) / (16 * MBW);
  const dim3 grid(static_cast<unsigned>(ne * ((nt + 7) / 8) * 8));
  if (router_quant_fused(d))
    hipLaunchKernelGGL((router_mfma_kernel<MBW, NBW, false, true, NW>), grid, dim3(NW * 64), 0, s,
                       static_cast<const uint16_t *>(in.x),
                       static_cast<const uint16_t *>(in.router_w), w.logits, d.m, d.E, d.H, w.xq, w.sx);
  else
    hipLaunchKernelGGL((router_mfma_kernel<MBW, NBW, false, false, NW>), grid, dim3(NW * 64), 0, s,
                       static_cast<const uint16_t *>(in.x),
                       static_cast<const uint16_t *>(in.router_w), w.logits, d.m, d.E, d.H,
                       static_cast<uint8_t *>(nullptr), static_cast<float *>(nullptr));
  return hipGetLastError();
}

hipError_t launch_router(const Dims &d, const Inputs &in, const Work &w,
                         hipStream_t s) {
  if (d.wdt != kF32) {
    if (route_fused_ok(d)) {   // partial tiles, summed by topk_permute_kernel
      const dim3 grid((d.E + 15) / 16, router_splits(d));
      hipLaunchKernelGGL((router_mfma_kernel<1, 1, true>), grid, dim3(256), 0, s,
                         static_cast<const uint16_t *>(in.x),
                         static_cast<const uint16_t *>(in.router_w), w.rpart, d.m, d.E, d.H);
      return hipGetLastError();
    }
    if (d.m <= 64) return launch_router_mfma<1, 1>(d, in, w, s);
    // 32 x 64 tiles unless they leave CUs idle (then 16 x 32: more re-reads
    // of x and Wr, but four times the blocks), 64 x 64 when those fill them
    const long big_tiles = static_cast<long>((d.E + 63) / 64) * ((d.m + 31) / 32);
    if (big_tiles < 256) return launch_router_mfma<1, 2>(d, in, w, s);
    // 64 x 64 tiles once they alone fill the CUs: half the re-reads of Wr;
    // eight waves splitting K where it divides into 1024-column parts (twice
    // the loads in flight per CU: the loop waits for each batch's loads)
    if (static_cast<long>((d.E + 63) / 64) * ((d.m + 63) / 64) >= 256)
      return d.H % 1024 == 0 ? launch_router_mfma<4, 4, 8>(d, in, w, s) : launch_router_mfma<4, 4>(d, in, w, s);
    return launch_router_mfma<2, 4>(d, in, w, s);
  }
  dim3 grid((d.E + kRouterWaves - 1) / kRouterWaves,
            (d.m + kRouterTok - 1) / kRouterTok);
  hipLaunchKernelGGL(router_valu_kernel<kF32>, grid, dim3(256), 0, s, in.x,
                     in.router_w, w.logits, d.m, d.E, d.H);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode-sized batches (m <= 16): the router product runs on at least
// kRouterBlocksTarget blocks (split over K as well as over experts when E is
// small); blocks write partial tiles.  One block of 16 waves then sums the
// partials in split order, runs gating + top-k (wave t: token t) and the sort
// by expert, with the logits and indices handed between the steps in LDS: two
// launches instead of three.  (One CU pulls only a small share of HBM
// bandwidth, so the partials that single block reads are kept few.)
constexpr int kFusedThreads = 1024;
constexpr int kRouterBlocksTarget = 32;

bool route_fused_ok(const Dims &d) { return d.wdt != kF32 && d.m <= 16; }

bool router_quant_fused(const Dims &d) {
  return d.wdt == kFP8 && !route_fused_ok(d) && d.H % (4 * kQBlock) == 0;
}

int router_splits(const Dims &d) {
  const int eb = (d.E + 15) / 16;
  int ks = kRouterBlocksTarget / eb;
  ks = ks < 1 ? 1 : (ks > kRouterMaxSplits ? kRouterMaxSplits : ks);
  while (ks > 1 && d.H / 32 < 4 * ks) ks /= 2;   // >= one 32-wide step per wave
  return ks;
}

template <int EPL>
__global__ __launch_bounds__(kFusedThreads) void topk_permute_kernel(Dims d, Inputs in, Work w, int ks,
                                                                     int *topk_idx, float *topk_w) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint32_t sk[kFusedThreads / kWave][kTopkScratch];
  const int wave = threadIdx.x >> 6;
  const int m = d.m, E = d.E;
  float *lg = reinterpret_cast<float *>(smem);                // [m][E]
  int *idx_s = reinterpret_cast<int *>(lg + m * E);           // [m * k]
  int *wcnt = idx_s + ((m * d.k + 3) & ~3);                   // [16][E]
  int *lrank = wcnt + kPermWaves * E;                         // [m * k]
  // ---- logits: partial tiles summed in split order.  The first
  // kSumPre * kFusedThreads logits have all of their partials loaded before
  // any is summed or stored (one round trip to memory, not one per logit
  // group); larger m * E continue in a plain loop. ----
  const int mE = m * E;
  constexpr int kSumPre = 4;
  {
    float part[kSumPre][kRouterMaxSplits];
#pragma unroll
    for (int u = 0; u < kSumPre; ++u) {
      const int i = threadIdx.x + u * kFusedThreads;
#pragma unroll
      for (int q = 0; q < kRouterMaxSplits; ++q)
        part[u][q] = (i < mE && q < ks) ? w.rpart[static_cast<size_t>(q) * mE + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kSumPre; ++u) {
      const int i = threadIdx.x + u * kFusedThreads;
      float v = part[u][0];
#pragma unroll
      for (int q = 1; q < kRouterMaxSplits; ++q)
        if (q < ks) v += part[u][q];
      if (i < mE) {
        lg[i] = v;
        w.logits[i] = v;
      }
    }
  }
  for (int i = threadIdx.x + kSumPre * kFusedThreads; i < mE; i += kFusedThreads) {
    float v = w.rpart[i];
    for (int q = 1; q < ks; ++q) v += w.rpart[static_cast<size_t>(q) * mE + i];
    lg[i] = v;
    w.logits[i] = v;
  }
  __syncthreads();
  // ---- gating + top-k: wave t takes token t ----
  if (wave < m)
    topk_token<EPL>(lg + wave * E, E, d.k, d.gating, d.renorm, d.scale, in.bias,
                    topk_idx + static_cast<size_t>(wave) * d.k, topk_w + static_cast<size_t>(wave) * d.k,
                    idx_s + wave * d.k, sk[wave]);
  __syncthreads();
  // ---- stable sort by expert: the few pairs of a decode batch by one wave ----
  if (wave == 0)
    permute_wave(idx_s, d.te, E, wcnt, lrank, w.counts, w.offsets, w.sorted_pair, w.slot_of_pair,
                 w.active, w.nactive, w.rboff, w.queue);
}

hipError_t launch_topk_permute(const Dims &d, const Inputs &in, const Work &w, int *topk_idx,
                               float *topk_w, hipStream_t s) {
  const size_t lds = static_cast<size_t>(d.m) * d.E * 4 + static_cast<size_t>((d.m * d.k + 3) & ~3) * 4 +
                     static_cast<size_t>(kPermWaves) * d.E * 4 + static_cast<size_t>(d.m) * d.k * 4;
  const int epl = (d.E + kWave - 1) / kWave;
  const int ks = router_splits(d);
#define MOE_FUSED_CASE(N)                                                                      \
  if (epl <= N) {                                                                              \
    static const hipError_t su =                                                               \
        lds_setup(reinterpret_cast<const void *>(topk_permute_kernel<N>), 144 << 10);         \
    if (su != hipSuccess) return su;                                                           \
    hipLaunchKernelGGL(topk_permute_kernel<N>, dim3(1), dim3(kFusedThreads), lds, s, d, in, w, \
                       ks, topk_idx, topk_w);                                                  \
    return hipGetLastError();                                                                  \
  }
  MOE_FUSED_CASE(1)
  MOE_FUSED_CASE(2)
  MOE_FUSED_CASE(4)
  MOE_FUSED_CASE(8)
  MOE_FUSED_CASE(16)
#undef MOE_FUSED_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Gating + top-k: one wave per token (topk_token in routing.h).
constexpr int kTopkWaves = 4;

template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(
    const float *__restrict__ logits, int m, int E, int k, int gating,
    int renorm, float scale, const float *__restrict__ bias,
    int *__restrict__ topk_idx, float *__restrict__ topk_w) {
  __shared__ uint32_t sk[kTopkWaves][kTopkScratch];
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  if (t >= m) return;
  topk_token<EPL>(logits + static_cast<size_t>(t) * E, E, k, gating, renorm, scale, bias,
                  topk_idx + static_cast<size_t>(t) * k, topk_w + static_cast<size_t>(t) * k, nullptr,
                  sk[threadIdx.x >> 6]);
}

hipError_t launch_topk(const Dims &d, const Inputs &in, const Work &w,
                       int *topk_idx, float *topk_w, hipStream_t s) {
  const dim3 grid((d.m + kTopkWaves - 1) / kTopkWaves);
  const int epl = (d.E + kWave - 1) / kWave;
#define MOE_TOPK_CASE(N)                                                      \
  if (epl <= N) {                                                             \
    hipLaunchKernelGGL(topk_kernel<N>, grid, dim3(256), 0, s, w.logits, d.m,  \
                       d.E, d.k, d.gating, d.renorm, d.scale, in.bias,        \
                       topk_idx, topk_w);                                     \
    return hipGetLastError();                                                 \
  }
  MOE_TOPK_CASE(1)
  MOE_TOPK_CASE(2)
  MOE_TOPK_CASE(4)
  MOE_TOPK_CASE(8)
  MOE_TOPK_CASE(16)
#undef MOE_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
