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
// MFMA router for bf16: a block computes 16*MBW tokens x 16*NBW experts with
// its four waves splitting H; each wave streams its K range of the token and
// expert rows straight into MFMA operands (16x16x32 bf16, fp32 accumulate)
// and the four partial tiles are summed through LDS in a fixed order.  Small
// tiles keep enough blocks in flight at decode sizes; larger ones cut the
// re-reads of x and Wr at prefill sizes.
template <int MBW, int NBW>
__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    float *__restrict__ logits, int m, int E, int H) {
  __shared__ f32x4_t part[3][MBW * NBW][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * 16 * MBW, e0 = blockIdx.x * 16 * NBW;
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
  const int s0 = steps * wave / 4, s1 = steps * (wave + 1) / 4;
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
      for (int w = 0; w < 3; ++w) v += part[w][i * NBW + j][lane];
      const int e = e0 + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * i + (lane >> 4) * 4 + r;
        if (t < m && e < E) logits[static_cast<size_t>(t) * E + e] = v[r];
      }
    }
}

template <int MBW, int NBW>
static hipError_t launch_router_mfma(const Dims &d, const Inputs &in, const Work &w,
                                     hipStream_t s) {
  const dim3 grid((d.E + 16 * NBW - 1) / (16 * NBW), (d.m + 16 * MBW - 1) / (16 * MBW));
  hipLaunchKernelGGL((router_mfma_kernel<MBW, NBW>), grid, dim3(256), 0, s,
                     static_cast<const uint16_t *>(in.x),
                     static_cast<const uint16_t *>(in.router_w), w.logits, d.m, d.E, d.H);
  return hipGetLastError();
}

hipError_t launch_router(const Dims &d, const Inputs &in, const Work &w,
                         hipStream_t s) {
  if (d.wdt != kF32) {
    if (d.m <= 64) return launch_router_mfma<1, 1>(d, in, w, s);
    return launch_router_mfma<2, 4>(d, in, w, s);
  }
  dim3 grid((d.E + kRouterWaves - 1) / kRouterWaves,
            (d.m + kRouterTok - 1) / kRouterTok);
  hipLaunchKernelGGL(router_valu_kernel<kF32>, grid, dim3(256), 0, s, in.x,
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
    int *__restrict__ topk_idx, float *__restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
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
