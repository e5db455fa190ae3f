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
// MFMA router for bf16 and m > 16: a block computes 64 tokens x 64 experts;
// wave w owns tokens 16w..16w+15 and all four 16-expert column blocks, with
// operands read straight from global memory (the expert rows are shared by
// the four waves through L1).  fp32 accumulation, K in 32-wide steps.
__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    float *__restrict__ logits, int m, int E, int H) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * 64 + wave * 16;
  const int e0 = blockIdx.x * 64;
  if (t0 >= m) return;
  const int kofs = (lane >> 4) * 8;
  const uint16_t *ap = x + static_cast<size_t>(min(t0 + (lane & 15), m - 1)) * H + kofs;
  const uint16_t *bp[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    bp[nb] = wr + static_cast<size_t>(min(e0 + nb * 16 + (lane & 15), E - 1)) * H + kofs;
  f32x4_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 0; k < H; k += 32) {
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(ap + k));
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(bp[nb] + k));
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int e = e0 + nb * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + (lane >> 4) * 4 + i;
      if (t < m && e < E) logits[static_cast<size_t>(t) * E + e] = acc[nb][i];
    }
  }
}

hipError_t launch_router(const Dims &d, const Inputs &in, const Work &w,
                         hipStream_t s) {
  if (d.wdt != kF32 && d.m > 16) {
    const dim3 grid((d.E + 63) / 64, (d.m + 63) / 64);
    hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(256), 0, s,
                       static_cast<const uint16_t *>(in.x),
                       static_cast<const uint16_t *>(in.router_w), w.logits,
                       d.m, d.E, d.H);
    return hipGetLastError();
  }
  dim3 grid((d.E + kRouterWaves - 1) / kRouterWaves,
            (d.m + kRouterTok - 1) / kRouterTok);
  if (d.wdt == kF32)
    hipLaunchKernelGGL(router_valu_kernel<kF32>, grid, dim3(256), 0, s, in.x,
                       in.router_w, w.logits, d.m, d.E, d.H);
  else
    hipLaunchKernelGGL(router_valu_kernel<kBF16>, grid, dim3(256), 0, s, in.x,
                       in.router_w, w.logits, d.m, d.E, d.H);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gating + top-k: one wave per token.  Lane l holds experts l, l+64, ...
// Selection repeats k times: every lane offers its best untaken expert, a
// butterfly reduction picks the larger score (equal scores: lower index).
// Softmax ranks by the logit itself (same order as the softmax probability,
// without its rounding); sigmoid ranks by sigmoid(l) + bias.
constexpr int kTopkWaves = 4;
constexpr int kMaxEPerLane = 16;  // E <= 1024

template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(
    const float *__restrict__ logits, int m, int E, int k, int gating,
    int renorm, float scale, const float *__restrict__ bias,
    int *__restrict__ topk_idx, float *__restrict__ topk_w,
    unsigned *__restrict__ ticket) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  // The permutation kernel that follows counts finished chunks on `ticket`;
  // it must start from zero on every call.
  if (blockIdx.x == 0 && threadIdx.x == 0) *ticket = 0u;
  if (t >= m) return;
  const float *lrow = logits + static_cast<size_t>(t) * E;
  float l[EPL], c[EPL];
  unsigned taken = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    l[i] = e < E ? lrow[e] : 0.f;
    if (gating == 0) {
      c[i] = l[i];
    } else {
      c[i] = 1.0f / (1.0f + expf(-l[i]));
      if (bias) c[i] += e < E ? bias[e] : 0.f;
    }
    if (e >= E) taken |= 1u << i;
  }
  int my_e = -1;        // lane j < k: expert chosen in round j
  float my_l = 0.f;     // its logit
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
    float bl = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (!(taken & (1u << i))) {
        const int e = lane + kWave * i;
        if (c[i] > bv || (c[i] == bv && e < be)) { bv = c[i]; be = e; bl = l[i]; }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oe = __shfl_xor(be, o);
      const float ol = __shfl_xor(bl, o);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; bl = ol; }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) { my_e = be; my_l = bl; }
  }
  // Gate weights of the selected experts.
  float wj = 0.f;
  if (gating == 0) {
    const float l0 = __shfl(my_l, 0);  // largest selected logit
    if (renorm) {
      const float ex = lane < k ? expf(my_l - l0) : 0.f;
      wj = ex / wave_sum(ex);
    } else {
      float lmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E) lmax = fmaxf(lmax, l[i]);
      lmax = wave_max(lmax);
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E) z += expf(l[i] - lmax);
      z = wave_sum(z);
      wj = expf(my_l - lmax) / z;
    }
  } else {
    const float sj = lane < k ? 1.0f / (1.0f + expf(-my_l)) : 0.f;
    wj = renorm ? sj / wave_sum(sj) : sj;
  }
  if (lane < k) {
    topk_idx[static_cast<size_t>(t) * k + lane] = my_e;
    topk_w[static_cast<size_t>(t) * k + lane] = wj * scale;
  }
}

hipError_t launch_topk(const Dims &d, const Inputs &in, const Work &w,
                       int *topk_idx, float *topk_w, hipStream_t s) {
  const dim3 grid((d.m + kTopkWaves - 1) / kTopkWaves);
  const int epl = (d.E + kWave - 1) / kWave;
#define MOE_TOPK_CASE(N)                                                      \
  if (epl <= N) {                                                             \
    hipLaunchKernelGGL(topk_kernel<N>, grid, dim3(256), 0, s, w.logits, d.m,  \
                       d.E, d.k, d.gating, d.renorm, d.scale, in.bias,        \
                       topk_idx, topk_w, w.ticket);                           \
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
