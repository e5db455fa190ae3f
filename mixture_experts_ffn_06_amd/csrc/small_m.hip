// Small-m (m <= 16) expert path: stream each selected expert's weights once.
//
// With at most 16 tokens every expert holds at most 16 rows, so the work is
// a bandwidth-bound GEMV over the selected experts' weights (forward.rs,
// page 1: rows <= 16 take the decode kernels; forward.rs, page 2: the
// single-token arm runs gate/up as one launch and down as another over all
// selected experts; forward_layer.rs, page 4: one dispatch covers all
// selected experts of a decode step).
//
// gate/up: block = (active expert d, 16 h columns).  Its four waves split H;
// each wave streams the 16 w1 rows and the 16 matching w3 rows of its K range
// straight into MFMA B registers (16 B per lane, all loads of a batch in
// flight together), with the expert's <= 16 token rows as the M side of a
// 16x16x32 bf16 MFMA.  The four partial sums meet in LDS, and wave 0 forms
// SiLU(g) * u and writes the bf16 h rows.
// down: block = (active expert d, 16 output columns), the same split-K
// scheme over I, writing bf16 y rows.  A shared expert is one more slot
// (after the active routed experts) whose rows are the m tokens.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kSmWaves = 4;
constexpr int kSmBatch = 8;   // K steps (of 32) whose loads are issued together

// Partial product of one wave over K steps [s0, s1): acc += A . B^T for one
// 16x16 block.  a_row / b_row point at the lane's row, K offset included.
__device__ __forceinline__ void sm_stream(const uint16_t *a_row, bool a_ok,
                                          const uint16_t *b_row0,
                                          const uint16_t *b_row1, int s0,
                                          int s1, f32x4_t &acc0, f32x4_t &acc1) {
  for (int s = s0; s < s1; s += kSmBatch) {
    uint4 av[kSmBatch], bv0[kSmBatch], bv1[kSmBatch];
#pragma unroll
    for (int i = 0; i < kSmBatch; ++i) {
      const bool in = s + i < s1;
      const int o = (s + i) * 32;
      bv0[i] = in ? *reinterpret_cast<const uint4 *>(b_row0 + o) : make_uint4(0, 0, 0, 0);
      if (b_row1) bv1[i] = in ? *reinterpret_cast<const uint4 *>(b_row1 + o) : make_uint4(0, 0, 0, 0);
      av[i] = (in && a_ok) ? *reinterpret_cast<const uint4 *>(a_row + o) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kSmBatch; ++i) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av[i]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bv0[i]), acc0, 0, 0, 0);
      if (b_row1)
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bv1[i]), acc1, 0, 0, 0);
    }
  }
}

// One slot of the small-m grid: a routed expert with >= 1 row, or the shared
// expert.  Returns false for slots past the last one.
struct SmSlot {
  bool shared;
  int e, seg0, rows, inter;
};

__device__ __forceinline__ bool sm_slot(const Dims &d, const Work &w, int slot, SmSlot &o) {
  const int na = *w.nactive;
  if (slot < na) {
    o.shared = false;
    o.e = w.active[slot];
    o.seg0 = w.offsets[o.e];
    o.rows = w.offsets[o.e + 1] - o.seg0;   // <= m <= 16
    o.inter = d.I;
    return true;
  }
  if (slot == na && d.Is > 0) {
    o.shared = true;
    o.e = d.E;
    o.seg0 = 0;
    o.rows = d.m;
    o.inter = d.Is;
    return true;
  }
  return false;
}

__global__ __launch_bounds__(256) void sm_gateup_kernel(Dims d, Inputs in, Work w) {
  __shared__ f32x4_t part[kSmWaves][2][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  SmSlot sl;
  if (!sm_slot(d, w, blockIdx.x, sl)) return;
  const int c0 = blockIdx.y * 16;
  if (c0 >= sl.inter) return;
  const int seg0 = sl.seg0, rows = sl.rows;
  const int r = lane & 15;
  const int kofs = (lane >> 4) * 8;
  const bool a_ok = r < rows;
  const int tok = !a_ok ? 0 : (sl.shared ? r : w.sorted_pair[seg0 + r] / d.k);
  const uint16_t *a_row = static_cast<const uint16_t *>(in.x) + static_cast<size_t>(tok) * d.H + kofs;
  const uint16_t *W = sl.shared ? static_cast<const uint16_t *>(in.sw13)
                                : static_cast<const uint16_t *>(in.w13) + static_cast<size_t>(sl.e) * 2 * d.I * d.H;
  const uint16_t *bg = W + static_cast<size_t>(c0 + r) * d.H + kofs;
  const uint16_t *bu = W + static_cast<size_t>(sl.inter + c0 + r) * d.H + kofs;
  const int steps = d.H / 32;
  const int s0 = steps * wave / kSmWaves, s1 = steps * (wave + 1) / kSmWaves;
  f32x4_t g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
  sm_stream(a_row, a_ok, bg, bu, s0, s1, g, u);
  part[wave][0][lane] = g;
  part[wave][1][lane] = u;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int wv = 1; wv < kSmWaves; ++wv) {
    g += part[wv][0][lane];
    u += part[wv][1][lane];
  }
  uint16_t *h = static_cast<uint16_t *>(sl.shared ? w.h_sh : w.h) + static_cast<size_t>(seg0) * sl.inter;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (lane >> 4) * 4 + i;
    if (row < rows) h[static_cast<size_t>(row) * sl.inter + c0 + (lane & 15)] = f32_to_bf16(silu(g[i]) * u[i]);
  }
}

__global__ __launch_bounds__(256) void sm_down_kernel(Dims d, Inputs in, Work w) {
  __shared__ f32x4_t part[kSmWaves][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  SmSlot sl;
  if (!sm_slot(d, w, blockIdx.x, sl)) return;
  const int seg0 = sl.seg0, rows = sl.rows, K = sl.inter;
  const int n0 = blockIdx.y * 16;
  const int r = lane & 15;
  const int kofs = (lane >> 4) * 8;
  const bool a_ok = r < rows;
  const uint16_t *a_row = static_cast<const uint16_t *>(sl.shared ? w.h_sh : w.h) +
                          static_cast<size_t>(seg0 + (a_ok ? r : 0)) * K + kofs;
  const uint16_t *b = (sl.shared ? static_cast<const uint16_t *>(in.sw2)
                                 : static_cast<const uint16_t *>(in.w2) + static_cast<size_t>(sl.e) * d.H * d.I) +
                      static_cast<size_t>(n0 + r) * K + kofs;
  const int steps = K / 32;
  const int s0 = steps * wave / kSmWaves, s1 = steps * (wave + 1) / kSmWaves;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, unused = {0.f, 0.f, 0.f, 0.f};
  sm_stream(a_row, a_ok, b, nullptr, s0, s1, acc, unused);
  part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int wv = 1; wv < kSmWaves; ++wv) acc += part[wv][lane];
  uint16_t *y = static_cast<uint16_t *>(sl.shared ? w.y_sh : w.y) + static_cast<size_t>(seg0) * d.H;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (lane >> 4) * 4 + i;
    if (row < rows) y[static_cast<size_t>(row) * d.H + n0 + (lane & 15)] = f32_to_bf16(acc[i]);
  }
}

// H, I multiples of 32 and m <= 16 are checked by the caller.
static int sm_slots(const Dims &d) { return (d.te < d.E ? d.te : d.E) + (d.Is > 0 ? 1 : 0); }

hipError_t launch_small_m_gateup(const Dims &d, const Inputs &in, const Work &w,
                                 hipStream_t s) {
  const int imax = d.Is > d.I ? d.Is : d.I;
  hipLaunchKernelGGL(sm_gateup_kernel, dim3(sm_slots(d), imax / 16), dim3(256), 0, s, d, in, w);
  return hipGetLastError();
}

hipError_t launch_small_m_down(const Dims &d, const Inputs &in, const Work &w,
                               hipStream_t s) {
  hipLaunchKernelGGL(sm_down_kernel, dim3(sm_slots(d), d.H / 16), dim3(256), 0, s, d, in, w);
  return hipGetLastError();
}

}  // namespace moe
