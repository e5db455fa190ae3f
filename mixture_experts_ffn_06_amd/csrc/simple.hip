// Expert path in plain fp32 VALU arithmetic, for every storage format.
//
// The layer's fp32 configuration runs here permanently, and the path serves
// as an independent GPU cross-check of the MFMA kernels at small sizes.  One
// thread computes one output element as a dot product; fp8 operands are
// summed per 128-wide K block and each block partial is multiplied by the
// activation and weight block scales before it joins the fp32 accumulator
// (the two-level fp32 block-scale accumulation of forward_prefill.rs, page 3,
// notes on the ported fp8 grouped GEMM).
//
// MX weights (OCP MXFP4 / MXFP8, E8M0 scale per 32 elements along K) are
// decoded element by element here (code value times 2^(e - 127), exact in
// fp32); their x, h and y are bf16 as on the bf16 path.  This is the MX
// formats' path for batches of more than 16 tokens.
//
// Rows are in sorted order: routed rows s in [0, te) belong to the expert e
// with offsets[e] <= s < offsets[e+1] and to token sorted_pair[s] / k; the
// shared expert's rows follow as s = te + t.
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ int expert_of_row(const int *offsets, int E, int s) {
  int lo = 0, hi = E - 1;        // largest e with offsets[e] <= s
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= s) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr bool is_mx(int dt) { return dt == kMXFP4 || dt == kMXFP8; }

// Weight element k of row `row` of an MX matrix with K columns: packed
// codes (two e2m1 per byte, even element in the low nibble, or one e4m3 per
// byte) and one E8M0 scale byte per 32 elements of a row.
template <int DT>
__device__ __forceinline__ float mx_weight(const void *w, const uint8_t *sc, size_t row, int K, int k) {
  const uint8_t *b = static_cast<const uint8_t *>(w);
  float v;
  if constexpr (DT == kMXFP4) {
    const uint8_t byte = b[row * (K / 2) + k / 2];
    const uint32_t c = (k & 1) ? (byte >> 4) : (byte & 0xfu);
    const uint32_t e = (c >> 1) & 3u, mt = c & 1u;
    const float mag = e == 0 ? 0.5f * static_cast<float>(mt) : ldexpf(1.0f + 0.5f * static_cast<float>(mt), static_cast<int>(e) - 1);
    v = (c & 8u) ? -mag : mag;
  } else {
    v = fp8_to_f32(b[row * K + k]);
  }
  return ldexpf(v, static_cast<int>(sc[row * (K / 32) + k / 32]) - 127);
}

struct RowInfo {
  int t;            // token
  const void *w13;  // this row's [2I', H] weights
  const void *w2;   // [H, I']
  const float *s13; // fp8 scales
  const float *s2;
  int inter;        // I'
  void *h;          // h row base
  float *hs;        // h scale row base
  float *y;         // y row base (fp32)
};

template <int DT>
__device__ __forceinline__ RowInfo row_info(const Dims &d, const Inputs &in,
                                            const Work &w, int s) {
  RowInfo r;
  // bytes per weight element (MXFP4: half a byte, counted per expert below)
  constexpr int B = is_mx(DT) ? 2 : StorageBytes<DT>::value;   // h element bytes
  if (s < d.te) {
    const int e = expert_of_row(w.offsets, d.E, s);
    r.t = w.sorted_pair[s] / d.k;
    r.inter = d.I;
    const size_t ew = static_cast<size_t>(2) * d.I * d.H;   // w13 (and w2) elements per expert
    const size_t ewb = DT == kMXFP4 ? ew / 2 : (is_mx(DT) ? ew : ew * StorageBytes<DT>::value);
    r.w13 = static_cast<const char *>(in.w13) + static_cast<size_t>(e) * ewb;
    r.w2 = static_cast<const char *>(in.w2) + static_cast<size_t>(e) * (ewb / 2);
    if constexpr (is_mx(DT)) {   // E8M0 scale bytes, one per 32 elements
      r.s13 = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(in.w13_scale) + static_cast<size_t>(e) * (ew / 32));
      r.s2 = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(in.w2_scale) + static_cast<size_t>(e) * (ew / 64));
    } else {
      r.s13 = DT == kFP8 ? in.w13_scale + static_cast<size_t>(e) * (2 * d.I / kQBlock) * (d.H / kQBlock) : nullptr;
      r.s2 = DT == kFP8 ? in.w2_scale + static_cast<size_t>(e) * (d.H / kQBlock) * (d.I / kQBlock) : nullptr;
    }
    r.h = static_cast<char *>(w.h) + static_cast<size_t>(s) * d.I * B;
    r.hs = DT == kFP8 ? w.h_scale + static_cast<size_t>(s) * (d.I / kQBlock) : nullptr;
    r.y = w.y + static_cast<size_t>(s) * d.H;
  } else {
    r.t = s - d.te;
    r.inter = d.Is;
    r.w13 = in.sw13;
    r.w2 = in.sw2;
    r.s13 = in.sw13_scale;
    r.s2 = in.sw2_scale;
    r.h = static_cast<char *>(w.h_sh) + static_cast<size_t>(r.t) * d.Is * B;
    r.hs = DT == kFP8 ? w.h_sh_scale + static_cast<size_t>(r.t) * (d.Is / kQBlock) : nullptr;
    r.y = w.y_sh + static_cast<size_t>(r.t) * d.H;
  }
  return r;
}

// Gate/up + SwiGLU: block = (row s, 128 columns of h); thread = one column.
template <int DT>
__global__ __launch_bounds__(128) void simple_gateup_kernel(Dims d, Inputs in, Work w) {
  __shared__ float red[2];
  const int s = blockIdx.x;
  const int c = blockIdx.y * kQBlock + threadIdx.x;
  const RowInfo r = row_info<DT>(d, in, w, s);
  if (blockIdx.y * kQBlock >= r.inter) return;   // whole block: uniform
  const bool valid = c < r.inter;
  const int H = d.H;
  float g = 0.f, u = 0.f;
  if (valid) {
    const size_t rg = static_cast<size_t>(c) * H, ru = static_cast<size_t>(r.inter + c) * H;
    if constexpr (is_mx(DT)) {
      const uint8_t *sc = reinterpret_cast<const uint8_t *>(r.s13);
      for (int h = 0; h < H; ++h) {
        const float a = load_as_f32<kBF16>(in.x, static_cast<size_t>(r.t) * H + h);
        g = fmaf(a, mx_weight<DT>(r.w13, sc, c, H, h), g);
        u = fmaf(a, mx_weight<DT>(r.w13, sc, r.inter + c, H, h), u);
      }
    } else if constexpr (DT == kFP8) {
      const uint8_t *xa = w.xq + static_cast<size_t>(r.t) * H;
      const float *sa = w.sx + static_cast<size_t>(r.t) * (H / kQBlock);
      const int kb_n = H / kQBlock;
      for (int kb = 0; kb < kb_n; ++kb) {
        float pg = 0.f, pu = 0.f;
        for (int i = 0; i < kQBlock; ++i) {
          const int h = kb * kQBlock + i;
          const float a = fp8_to_f32(xa[h]);
          pg = fmaf(a, load_as_f32<kFP8>(r.w13, rg + h), pg);
          pu = fmaf(a, load_as_f32<kFP8>(r.w13, ru + h), pu);
        }
        const float sg = r.s13[(c / kQBlock) * kb_n + kb];
        const float su = r.s13[((r.inter + c) / kQBlock) * kb_n + kb];
        g = fmaf(pg, sa[kb] * sg, g);
        u = fmaf(pu, sa[kb] * su, u);
      }
    } else {
      for (int h = 0; h < H; ++h) {
        const float a = load_as_f32<DT>(in.x, static_cast<size_t>(r.t) * H + h);
        g = fmaf(a, load_as_f32<DT>(r.w13, rg + h), g);
        u = fmaf(a, load_as_f32<DT>(r.w13, ru + h), u);
      }
    }
  }
  const float hv = silu(g) * u;
  if constexpr (DT == kF32) {
    if (valid) static_cast<float *>(r.h)[c] = hv;
  } else if constexpr (DT == kBF16 || is_mx(DT)) {
    if (valid) static_cast<uint16_t *>(r.h)[c] = f32_to_bf16(hv);
  } else {
    const float wm = wave_max(fabsf(hv));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = wm;
    __syncthreads();
    const float amax = fmaxf(red[0], red[1]);
    const float sc = amax > 0.f ? amax / kE4M3Max : 1.0f;
    const int code = fp8_pack2(hv / sc, 0.f) & 0xff;
    static_cast<uint8_t *>(r.h)[c] = static_cast<uint8_t>(code);
    if (threadIdx.x == 0) r.hs[blockIdx.y] = sc;
  }
}

// Down: block = (row s, 256 output columns); thread = one column.
template <int DT>
__global__ __launch_bounds__(256) void simple_down_kernel(Dims d, Inputs in, Work w) {
  const int s = blockIdx.x;
  const int n = blockIdx.y * 256 + threadIdx.x;
  if (n >= d.H) return;
  const RowInfo r = row_info<DT>(d, in, w, s);
  const int K = r.inter;
  const size_t rw = static_cast<size_t>(n) * K;
  float acc = 0.f;
  if constexpr (is_mx(DT)) {
    const uint8_t *sc = reinterpret_cast<const uint8_t *>(r.s2);
    for (int j = 0; j < K; ++j)
      acc = fmaf(load_as_f32<kBF16>(r.h, j), mx_weight<DT>(r.w2, sc, n, K, j), acc);
  } else if constexpr (DT == kFP8) {
    const int kb_n = K / kQBlock;
    for (int kb = 0; kb < kb_n; ++kb) {
      float p = 0.f;
      for (int i = 0; i < kQBlock; ++i) {
        const int j = kb * kQBlock + i;
        p = fmaf(fp8_to_f32(static_cast<const uint8_t *>(r.h)[j]),
                 load_as_f32<kFP8>(r.w2, rw + j), p);
      }
      acc = fmaf(p, r.hs[kb] * r.s2[(n / kQBlock) * kb_n + kb], acc);
    }
  } else {
    for (int j = 0; j < K; ++j)
      acc = fmaf(load_as_f32<DT>(r.h, j), load_as_f32<DT>(r.w2, rw + j), acc);
  }
  r.y[n] = acc;
}

template <int DT>
static hipError_t simple_gateup(const Dims &d, const Inputs &in, const Work &w,
                                hipStream_t s) {
  const int rows = d.te + (d.Is > 0 ? d.m : 0);
  const int imax = d.Is > d.I ? d.Is : d.I;
  hipLaunchKernelGGL(simple_gateup_kernel<DT>,
                     dim3(rows, (imax + kQBlock - 1) / kQBlock), dim3(128), 0,
                     s, d, in, w);
  return hipGetLastError();
}

template <int DT>
static hipError_t simple_down(const Dims &d, const Inputs &in, const Work &w,
                              hipStream_t s) {
  const int rows = d.te + (d.Is > 0 ? d.m : 0);
  hipLaunchKernelGGL(simple_down_kernel<DT>, dim3(rows, (d.H + 255) / 256),
                     dim3(256), 0, s, d, in, w);
  return hipGetLastError();
}

hipError_t launch_simple_gateup(const Dims &d, const Inputs &in, const Work &w,
                                hipStream_t s) {
  switch (d.wdt) {
    case kF32: return simple_gateup<kF32>(d, in, w, s);
    case kBF16: return simple_gateup<kBF16>(d, in, w, s);
    case kMXFP4: return simple_gateup<kMXFP4>(d, in, w, s);
    case kMXFP8: return simple_gateup<kMXFP8>(d, in, w, s);
    default: return simple_gateup<kFP8>(d, in, w, s);
  }
}

hipError_t launch_simple_down(const Dims &d, const Inputs &in, const Work &w,
                              hipStream_t s) {
  switch (d.wdt) {
    case kF32: return simple_down<kF32>(d, in, w, s);
    case kBF16: return simple_down<kBF16>(d, in, w, s);
    case kMXFP4: return simple_down<kMXFP4>(d, in, w, s);
    case kMXFP8: return simple_down<kMXFP8>(d, in, w, s);
    default: return simple_down<kFP8>(d, in, w, s);
  }
}

}  // namespace moe
