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
constexpr int kQuantBlocks = 2048;   // grid cap; waves then loop

// x is [m, H] row-major with H a multiple of 128, so the 128-column groups
// of all tokens are consecutive 128-element runs of the flat array, and the
// scales [m, H/128] are indexed by the flat group number.  A wave takes four
// consecutive groups per step: lane l loads 16 bytes (8 columns) of group
// 4 s + l / 16, the 16 lanes of a group find its amax with four exchanges,
// and each lane stores its 8 codes as one 8-byte write.
__global__ __launch_bounds__(kQuantWaves * kWave) void quant_x_kernel(
    const uint16_t *__restrict__ x, long ngroups, uint8_t *__restrict__ xq, float *__restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const long nsteps = (ngroups + 3) / 4;
  const long stride = static_cast<long>(gridDim.x) * kQuantWaves;
  for (long st = static_cast<long>(blockIdx.x) * kQuantWaves + (threadIdx.x >> 6); st < nsteps; st += stride) {
    const long g = st * 4 + (lane >> 4);
    const bool on = g < ngroups;
    const long e0 = g * kQBlock + (lane & 15) * 8;   // first of the lane's 8 elements
    uint4 q = make_uint4(0, 0, 0, 0);
    if (on) q = *reinterpret_cast<const uint4 *>(x + e0);
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(static_cast<uint16_t>(u[i] & 0xffffu));
      v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
    }
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));   // within the 16-lane group
    const float s = am > 0.f ? am / kE4M3Max : 1.0f;
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = static_cast<uint32_t>(fp8_pack2(v[2 * i] / s, v[2 * i + 1] / s)) & 0xffffu;
    if (on) {
      *reinterpret_cast<uint2 *>(xq + e0) = make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
      if ((lane & 15) == 0) sx[g] = s;
    }
  }
}

hipError_t launch_quant_x(const Dims &d, const Inputs &in, const Work &w,
                          hipStream_t s) {
  const long ngroups = static_cast<long>(d.m) * (d.H / kQBlock);
  const long steps = (ngroups + 3) / 4;
  long blocks = (steps + kQuantWaves - 1) / kQuantWaves;
  if (blocks > kQuantBlocks) blocks = kQuantBlocks;
  hipLaunchKernelGGL(quant_x_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kQuantWaves * kWave), 0, s,
                     static_cast<const uint16_t *>(in.x), ngroups, w.xq, w.sx);
  return hipGetLastError();
}

}  // namespace moe
