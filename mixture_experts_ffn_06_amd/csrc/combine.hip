// Unpermute + weighted top-k reduce + shared-expert blend.
//
// out[t, n] = sum_{j<k} w[t,j] * y[slot(t*k+j), n]  (+ g_t * y_shared[t, n])
//
// g_t = 1 without a shared-expert gate vector, else sigmoid(x[t] . gate)
// (forward_prefill.rs, page 3, step 8: the shared-expert blend).  Every
// block of token t computes that dot product itself, in one fixed order
// (8-element runs per thread, a wave butterfly, then the waves in order), so
// the factor is the same in every block and on every call.
//
// forward_prefill.rs (page 3, step 7 "Unpermute + weighted reduce") gathers
// each token's sorted expert rows through the token-to-slot map and applies
// the gate weights; forward.rs (page 2, MoeV41::forward) sums routed and
// shared rows into one fp32 accumulator and rounds once.  Here the expert
// rows arrive in fp32 (unrounded since their down product) and the sum runs
// in fp32 in a fixed order (j ascending, then the shared row) with no
// atomics, so two calls give bit-identical outputs.
#include "common.h"
#include "kernels.h"

namespace moe {

// Eight consecutive elements of an activation-format row as fp32.
template <bool F32>
__device__ __forceinline__ void load8(const void *base, size_t i, float (&v)[8]) {
  if constexpr (F32) {
    const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + i);
    const float4 a = src[0], b = src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + i);
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(static_cast<uint16_t>(u[j] & 0xffffu));
      v[2 * j + 1] = bf16_to_f32(static_cast<uint16_t>(u[j] >> 16));
    }
  }
}

// sigmoid(x[t] . gate) by the whole block (H a multiple of 8).
template <bool F32>
__device__ __forceinline__ float shared_gate_factor(const void *x, const void *gate, int t, int H) {
  __shared__ float part[256 / kWave];
  float acc = 0.f;
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) {
    float a[8], g[8];
    load8<F32>(x, static_cast<size_t>(t) * H + h, a);
    load8<F32>(gate, h, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(a[i], g[i], acc);
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  float dot = 0.f;
#pragma unroll
  for (int w = 0; w < 256 / kWave; ++w) dot += part[w];
  return 1.0f / (1.0f + expf(-dot));
}

// One block per token row chunk; 8 columns per thread (two 16-byte y loads).
template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ y, const float *__restrict__ y_sh,
    const int *__restrict__ slot_of_pair, const float *__restrict__ topk_w,
    const void *__restrict__ x, const void *__restrict__ sgate,
    int m, int H, int k, void *__restrict__ out) {
  const int t = blockIdx.y;
  const int n0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  // every thread of the block takes part in the gate's reduction
  const float gsh = (y_sh && sgate) ? shared_gate_factor<F32>(x, sgate, t, H) : 1.0f;
  if (n0 >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const float wj = topk_w[static_cast<size_t>(t) * k + j];
    const size_t row = static_cast<size_t>(slot_of_pair[static_cast<size_t>(t) * k + j]);
    float v[8];
    load8<true>(y, row * H + n0, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
  }
  if (y_sh) {
    float v[8];
    load8<true>(y_sh, static_cast<size_t>(t) * H + n0, v);
    if (sgate) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(gsh, v[i], acc[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
  }
  if constexpr (F32) {
    float4 *dst = reinterpret_cast<float4 *>(static_cast<float *>(out) + static_cast<size_t>(t) * H + n0);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    uint4 q;
    q.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    q.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    q.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    q.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + static_cast<size_t>(t) * H + n0) = q;
  }
}

// Without a shared-expert gate (k <= kCombineK): one thread per 8 output
// columns of one token over a flat grid of m * H / 8 threads (no idle
// threads past a row's end), and every y row of the token loaded before any
// is summed, so the k gathers are in flight together.  The sum is the same
// as combine_kernel's: j ascending, then the shared row.
constexpr int kCombineK = 8;

template <bool F32>
__global__ __launch_bounds__(256) void combine_flat_kernel(
    const float *__restrict__ y, const float *__restrict__ y_sh,
    const int *__restrict__ slot_of_pair, const float *__restrict__ topk_w,
    int m, int H, int k, void *__restrict__ out) {
  const int cpr = H / 8;
  const long gid = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= static_cast<long>(m) * cpr) return;
  const int t = static_cast<int>(gid / cpr);
  const int n0 = static_cast<int>(gid - static_cast<long>(t) * cpr) * 8;
  size_t row[kCombineK];
  float wj[kCombineK];
#pragma unroll
  for (int j = 0; j < kCombineK; ++j) {
    row[j] = j < k ? static_cast<size_t>(slot_of_pair[static_cast<size_t>(t) * k + j]) : 0;
    wj[j] = j < k ? topk_w[static_cast<size_t>(t) * k + j] : 0.f;
  }
  float v[kCombineK][8];
#pragma unroll
  for (int j = 0; j < kCombineK; ++j)
    if (j < k) load8<true>(y, row[j] * H + n0, v[j]);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < kCombineK; ++j)
    if (j < k) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[j], v[j][i], acc[i]);
    }
  if (y_sh) {
    float u[8];
    load8<true>(y_sh, static_cast<size_t>(t) * H + n0, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += u[i];
  }
  if constexpr (F32) {
    float4 *dst = reinterpret_cast<float4 *>(static_cast<float *>(out) + static_cast<size_t>(t) * H + n0);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    uint4 q;
    q.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    q.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    q.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    q.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + static_cast<size_t>(t) * H + n0) = q;
  }
}

hipError_t launch_combine(const Dims &d, const Inputs &in, const Work &w, const int *topk_idx,
                          const float *topk_w, void *out, hipStream_t s) {
  (void)topk_idx;
  const float *ysh = d.Is > 0 ? w.y_sh : nullptr;
  const void *sg = d.Is > 0 ? in.sgate : nullptr;
  if (!sg && d.k <= kCombineK) {
    const long threads = static_cast<long>(d.m) * (d.H / 8);
    const dim3 fgrid(static_cast<unsigned>((threads + 255) / 256));
    if (d.wdt == kF32)
      hipLaunchKernelGGL(combine_flat_kernel<true>, fgrid, dim3(256), 0, s, w.y, ysh, w.slot_of_pair,
                         topk_w, d.m, d.H, d.k, out);
    else
      hipLaunchKernelGGL(combine_flat_kernel<false>, fgrid, dim3(256), 0, s, w.y, ysh, w.slot_of_pair,
                         topk_w, d.m, d.H, d.k, out);
    return hipGetLastError();
  }
  const dim3 grid((d.H / 8 + 255) / 256, d.m);
  if (d.wdt == kF32)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, w.y, ysh,
                       w.slot_of_pair, topk_w, in.x, sg, d.m, d.H, d.k, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, w.y, ysh,
                       w.slot_of_pair, topk_w, in.x, sg, d.m, d.H, d.k, out);
  return hipGetLastError();
}

}  // namespace moe
