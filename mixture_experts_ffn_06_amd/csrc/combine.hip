// Unpermute + weighted top-k reduce + shared-expert blend.
//
// out[t, n] = sum_{j<k} w[t,j] * y[slot(t*k+j), n]  (+ y_shared[t, n])
//
// forward_prefill.rs (page 3, step 7 "Unpermute + weighted reduce") gathers
// each token's sorted expert rows through the token-to-slot map and applies
// the gate weights; forward.rs (page 2, MoeV41::forward) sums routed and
// shared rows into one fp32 accumulator and rounds once.  Here the sum runs
// in fp32 in a fixed order (j ascending, then the shared row) with no
// atomics, so two calls give bit-identical outputs.
#include "common.h"
#include "kernels.h"

namespace moe {

// One block per token row chunk; 8 columns per thread (16-byte y loads).
template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(
    const void *__restrict__ y, const void *__restrict__ y_sh,
    const int *__restrict__ slot_of_pair, const float *__restrict__ topk_w,
    int m, int H, int k, void *__restrict__ out) {
  const int t = blockIdx.y;
  const int n0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (n0 >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const float wj = topk_w[static_cast<size_t>(t) * k + j];
    const size_t row = static_cast<size_t>(slot_of_pair[static_cast<size_t>(t) * k + j]);
    if constexpr (F32) {
      const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(y) + row * H + n0);
      const float4 a = src[0], b = src[1];
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
    } else {
      const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(y) + row * H + n0);
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wj, bf16_to_f32(static_cast<uint16_t>(u[i] & 0xffffu)), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj, bf16_to_f32(static_cast<uint16_t>(u[i] >> 16)), acc[2 * i + 1]);
      }
    }
  }
  if (y_sh) {
    if constexpr (F32) {
      const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(y_sh) + static_cast<size_t>(t) * H + n0);
      const float4 a = src[0], b = src[1];
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    } else {
      const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(y_sh) + static_cast<size_t>(t) * H + n0);
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_to_f32(static_cast<uint16_t>(u[i] & 0xffffu));
        acc[2 * i + 1] += bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
      }
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

hipError_t launch_combine(const Dims &d, const Work &w, const int *topk_idx,
                          const float *topk_w, void *out, hipStream_t s) {
  (void)topk_idx;
  const dim3 grid((d.H / 8 + 255) / 256, d.m);
  const void *ysh = d.Is > 0 ? w.y_sh : nullptr;
  if (d.wdt == kF32)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, w.y, ysh,
                       w.slot_of_pair, topk_w, d.m, d.H, d.k, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, w.y, ysh,
                       w.slot_of_pair, topk_w, d.m, d.H, d.k, out);
  return hipGetLastError();
}

}  // namespace moe
