// Activation quantisation of the fp8 layer: x [m,H] bf16 -> e4m3 codes with
// one fp32 scale per token per 128 columns (scale = amax / 448, code =
// round-to-nearest-even of x / scale; an all-zero group gets scale 1).
//
// forward.rs (page 1) quantises expert inputs per row and block before its
// block-scaled expert GEMMs; forward.rs (page 2) does the same with its q8_1
// rows.  Both divisions are IEEE-correct fp32 divisions (no fast-math
// reciprocal), so the codes are a pure function of x.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kQuantWaves = 4;

// One wave per (token, 128-column group); two columns per lane.
__global__ __launch_bounds__(256) void quant_x_kernel(
    const uint16_t *__restrict__ x, int m, int H, uint8_t *__restrict__ xq,
    float *__restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const int groups = H / kQBlock;
  const int gid = blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  if (gid >= m * groups) return;
  const int t = gid / groups, g = gid - t * groups;
  const size_t base = static_cast<size_t>(t) * H + g * kQBlock + 2 * lane;
  const uint32_t two = *reinterpret_cast<const uint32_t *>(x + base);
  const float v0 = bf16_to_f32(static_cast<uint16_t>(two & 0xffffu));
  const float v1 = bf16_to_f32(static_cast<uint16_t>(two >> 16));
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const float s = amax > 0.f ? amax / kE4M3Max : 1.0f;
  const int codes = fp8_pack2(v0 / s, v1 / s);
  *reinterpret_cast<uint16_t *>(xq + base) = static_cast<uint16_t>(codes & 0xffff);
  if (lane == 0) sx[static_cast<size_t>(t) * groups + g] = s;
}

hipError_t launch_quant_x(const Dims &d, const Inputs &in, const Work &w,
                          hipStream_t s) {
  const int n = d.m * (d.H / kQBlock);
  hipLaunchKernelGGL(quant_x_kernel, dim3((n + kQuantWaves - 1) / kQuantWaves),
                     dim3(256), 0, s, static_cast<const uint16_t *>(in.x), d.m,
                     d.H, w.xq, w.sx);
  return hipGetLastError();
}

}  // namespace moe
