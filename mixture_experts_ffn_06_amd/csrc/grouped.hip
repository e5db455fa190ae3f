// Grouped expert GEMMs on MFMA (bf16 and fp8-e4m3 with 128x128 block scales).
//
// forward_prefill.rs (page 3, MoeLayer::forward_prefill doc comment) sorts
// token rows by expert so that each expert's weight matrix is loaded once
// for all of its tokens instead of once per token, then runs a grouped gate/up
// GEMM, SiLU gating and a grouped down GEMM (steps 4-6).  Its notes on the
// ported fp8 grouped GEMM describe a weight-stationary per-expert kernel with
// double-buffered prefetch and two-level fp32 block-scale accumulation.
//
// This file keeps those ideas and lays them out for CDNA4:
//  * Work units are (group, M tile of <= 128 rows, N tile); group e < E is a
//    routed expert with its rows in sorted order, group E is the shared
//    expert with one row per token.  A persistent grid walks the units;
//    consecutive units of an expert share an N tile (same weight slice, other
//    M tile) and are mapped onto the same XCD so the repeated weight reads of a
//    busy expert hit that XCD's L2.
//  * Each wave owns its own weight rows (no other wave reads them), so weight
//    fragments go straight from HBM into registers in the MFMA B layout, one
//    K stage ahead.  The token rows (A) are shared by all waves: they are
//    gathered through the sort permutation into LDS, double-buffered.
//  * gate/up: a wave holds a 16-column slice of w1 and the same 16 columns of
//    w3, so SiLU(g) * u is formed in registers (SwiGLU epilogue fused).  For
//    fp8 the block of 8 waves covers 128 h columns, the span of one h scale
//    group, and quantises h in the epilogue (amax over the 128 columns of a
//    row through LDS).
//  * fp8 two-level accumulation: every 128-wide K block is one MFMA
//    (16x16x128, fp32 out) started from zero; its result times
//    (activation row scale * weight block scale) is added to the fp32
//    accumulator.
#include "common.h"
#include "kernels.h"

namespace moe {

enum : int { kGateUp = 0, kDown = 1 };

template <int DT, int MODE, int NW>
struct GCfg {
  static constexpr int BM = 128;                      // rows per M tile
  static constexpr int MB = BM / 16;                  // m-blocks
  static constexpr int ESZ = DT == kBF16 ? 2 : 1;     // operand bytes
  static constexpr int STAGE_K = DT == kBF16 ? 128 : 256;
  static constexpr int ROW_BYTES = STAGE_K * ESZ;     // 256
  static constexpr int LDS_STRIDE = ROW_BYTES + 16;   // pad: spread banks
  static constexpr int KSTEP = DT == kBF16 ? 32 : 128;
  static constexpr int STEPS = STAGE_K / KSTEP;       // MFMAs per stage per (mb, nb)
  static constexpr int THREADS = NW * kWave;
  static constexpr int CHUNKS = BM * ROW_BYTES / 16 / THREADS;  // A loads/thread/stage
  static constexpr int ROWS_PER_PASS = THREADS / (ROW_BYTES / 16);
  static constexpr int BV = DT == kBF16 ? 1 : 2;      // uint4 per lane per (nb, step)
  static constexpr int NCOLS = MODE == kGateUp ? 16 * NW : 32 * NW;  // output cols / tile
  static constexpr int LDS_BYTES = 2 * BM * LDS_STRIDE;
};

struct GroupedArgs {
  Dims d;
  Inputs in;
  Work w;
  int ntile_routed;   // N tiles of a routed expert
  int ntile_shared;   // N tiles of the shared expert
};

// Per-lane B fragment for one stage: [nb][step][BV] uint4.
template <int DT, int MODE, int NW>
struct BFrag {
  uint4 v[2][GCfg<DT, MODE, NW>::STEPS][GCfg<DT, MODE, NW>::BV];
};

// Weight fragments of one K stage; steps at or past K (a partial last
// stage) read nothing and hold zeros.
template <int DT, int MODE, int NW>
__device__ __forceinline__ void load_b(BFrag<DT, MODE, NW> &f, const uint8_t *b0,
                                       const uint8_t *b1, int kbyte, int kbytes) {
  using C = GCfg<DT, MODE, NW>;
#pragma unroll
  for (int s = 0; s < C::STEPS; ++s) {
    const bool in = kbyte + s * C::KSTEP * C::ESZ < kbytes;
#pragma unroll
    for (int v = 0; v < C::BV; ++v) {
      const int o = kbyte + s * C::KSTEP * C::ESZ + v * 16;
      f.v[0][s][v] = in ? *reinterpret_cast<const uint4 *>(b0 + o) : make_uint4(0, 0, 0, 0);
      f.v[1][s][v] = in ? *reinterpret_cast<const uint4 *>(b1 + o) : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int DT, int MODE, int NW>
__global__ __launch_bounds__(NW * 64) void grouped_kernel(GroupedArgs a) {
  using C = GCfg<DT, MODE, NW>;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int uoff[1026];        // unit prefix over groups (E + 1 groups)
  const Dims &d = a.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = d.E + (d.Is > 0 ? 1 : 0);
  const int *offsets = a.w.offsets;

  // ---- unit prefix: units(g) = ceil(rows_g / BM) * ntile_g ----
  {
    constexpr int PER = (1025 + C::THREADS - 1) / C::THREADS;
    int loc[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid * PER + i;
      int u = 0;
      if (g < G) {
        const int rows = g < d.E ? offsets[g + 1] - offsets[g] : d.m;
        u = (rows + C::BM - 1) / C::BM * (g < d.E ? a.ntile_routed : a.ntile_shared);
      }
      loc[i] = u;
      sum += u;
    }
    // block inclusive scan of `sum`
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    __shared__ int wsum[NW];
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) base += i < wave ? wsum[i] : 0;
    int run = base + incl - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid * PER + i;
      if (g <= G) uoff[g] = run;   // uoff[G] = total
      run += loc[i];
    }
    __syncthreads();
  }
  const int total = uoff[G];
  const int P = gridDim.x;
  const int per_xcd = P / 8;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  uint8_t *lds_a[2] = {lds, lds + C::BM * C::LDS_STRIDE};

  for (int r = 0;; ++r) {
    const int u = r * P + xcd * per_xcd + slot;
    if (r * P >= total) break;
    if (u >= total) continue;
    // ---- decode the unit ----
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uoff[mid] <= u) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const bool shared = g == d.E;
    const int grows = shared ? d.m : offsets[g + 1] - offsets[g];
    const int nmt = (grows + C::BM - 1) / C::BM;
    const int local = u - uoff[g];
    const int ntile = local / nmt;
    const int row0 = (local - ntile * nmt) * C::BM;
    const int rows = min(C::BM, grows - row0);
    const int nmb = (rows + 15) >> 4;
    const int seg0 = shared ? 0 : offsets[g];   // first sorted row of the group
    const int inter = shared ? d.Is : d.I;
    const int K = MODE == kGateUp ? d.H : inter;
    const int nstage = K / C::STAGE_K + (K % C::STAGE_K ? 1 : 0);

    // ---- operand pointers ----
    const uint8_t *Wb;        // this group's weight matrix
    const float *Ws = nullptr;  // its block scales
    if (MODE == kGateUp) {
      Wb = static_cast<const uint8_t *>(shared ? a.in.sw13 : a.in.w13) +
           (shared ? 0 : static_cast<size_t>(g) * 2 * d.I * d.H * C::ESZ);
      if (DT == kFP8)
        Ws = shared ? a.in.sw13_scale
                    : a.in.w13_scale + static_cast<size_t>(g) * (2 * d.I / kQBlock) * (d.H / kQBlock);
    } else {
      Wb = static_cast<const uint8_t *>(shared ? a.in.sw2 : a.in.w2) +
           (shared ? 0 : static_cast<size_t>(g) * d.H * d.I * C::ESZ);
      if (DT == kFP8)
        Ws = shared ? a.in.sw2_scale
                    : a.in.w2_scale + static_cast<size_t>(g) * (d.H / kQBlock) * (d.I / kQBlock);
    }
    int nrow0, nrow1;   // first weight row of this wave's two n-blocks
    if (MODE == kGateUp) {
      nrow0 = ntile * C::NCOLS + wave * 16;
      nrow1 = inter + nrow0;
    } else {
      nrow0 = ntile * C::NCOLS + wave * 32;
      nrow1 = nrow0 + 16;
    }
    // A wave past the last column of a partial N tile streams row 0 (valid
    // memory) and stores nothing.
    const bool wave_on = nrow0 < (MODE == kGateUp ? inter : d.H);
    if (!wave_on) nrow0 = nrow1 = 0;
    const size_t wrow_bytes = static_cast<size_t>(K) * C::ESZ;
    const int lk = (lane >> 4) * (C::KSTEP / 4) * C::ESZ;  // lane's K byte offset in a step
    const uint8_t *b0 = Wb + static_cast<size_t>(nrow0 + (lane & 15)) * wrow_bytes + lk;
    const uint8_t *b1 = Wb + static_cast<size_t>(nrow1 + (lane & 15)) * wrow_bytes + lk;

    // A rows handled by this thread: r = tid / 16 + pass * ROWS_PER_PASS
    const int chunk = tid & 15;
    const uint8_t *arow[C::CHUNKS];
    const float *srow[C::CHUNKS];
#pragma unroll
    for (int i = 0; i < C::CHUNKS; ++i) {
      const int rr = (tid >> 4) + i * C::ROWS_PER_PASS;
      arow[i] = nullptr;
      srow[i] = nullptr;
      if (rr < rows) {
        if (MODE == kGateUp) {
          const int tok = shared ? row0 + rr : a.w.sorted_pair[seg0 + row0 + rr] / d.k;
          if (DT == kFP8) {
            arow[i] = a.w.xq + static_cast<size_t>(tok) * d.H;
            srow[i] = a.w.sx + static_cast<size_t>(tok) * (d.H / kQBlock);
          } else {
            arow[i] = static_cast<const uint8_t *>(a.in.x) + static_cast<size_t>(tok) * d.H * 2;
          }
        } else {
          const size_t hr = static_cast<size_t>(seg0 + row0 + rr);
          const uint8_t *hb = static_cast<const uint8_t *>(shared ? a.w.h_sh : a.w.h);
          arow[i] = hb + hr * inter * C::ESZ;
          if (DT == kFP8)
            srow[i] = (shared ? a.w.h_sh_scale : a.w.h_scale) + hr * (inter / kQBlock);
        }
      }
    }

    f32x4_t acc[C::MB][2];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 areg[C::CHUNKS];
    auto load_a = [&](int st) {
      const int kb = st * C::ROW_BYTES + chunk * 16;
#pragma unroll
      for (int i = 0; i < C::CHUNKS; ++i) {
        const bool ok = arow[i] != nullptr && kb < K * C::ESZ;
        areg[i] = ok ? *reinterpret_cast<const uint4 *>(arow[i] + kb) : make_uint4(0, 0, 0, 0);
      }
    };
    // fp8 stages hold two 128-K blocks; keep both row scales in LDS.
    __shared__ float sa2[2][2][C::BM];
    auto store_a = [&](int buf, int st) {
#pragma unroll
      for (int i = 0; i < C::CHUNKS; ++i) {
        const int rr = (tid >> 4) + i * C::ROWS_PER_PASS;
        *reinterpret_cast<uint4 *>(lds_a[buf] + rr * C::LDS_STRIDE + chunk * 16) = areg[i];
      }
      if constexpr (DT == kFP8) {
        if (chunk < C::STEPS) {
#pragma unroll
          for (int i = 0; i < C::CHUNKS; ++i) {
            const int rr = (tid >> 4) + i * C::ROWS_PER_PASS;
            const int kblk = st * C::STEPS + chunk;
            float v = 0.f;
            if (srow[i] && kblk * kQBlock < K) v = srow[i][kblk];
            sa2[buf][chunk][rr] = v;
          }
        }
      }
    };

    BFrag<DT, MODE, NW> bf[2];
    auto compute = [&](int buf, const BFrag<DT, MODE, NW> &f, int st) {
      const uint8_t *la = lds_a[buf] + (lane & 15) * C::LDS_STRIDE + lk;
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int s = 0; s < C::STEPS; ++s) {
          const bf16x8_t b0v = __builtin_bit_cast(bf16x8_t, f.v[0][s][0]);
          const bf16x8_t b1v = __builtin_bit_cast(bf16x8_t, f.v[1][s][0]);
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) {
            if (mb < nmb) {
              const uint4 av = *reinterpret_cast<const uint4 *>(la + mb * 16 * C::LDS_STRIDE + s * C::KSTEP * 2);
              const bf16x8_t a8 = __builtin_bit_cast(bf16x8_t, av);
              acc[mb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b0v, acc[mb][0], 0, 0, 0);
              acc[mb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b1v, acc[mb][1], 0, 0, 0);
            }
          }
        }
      } else {
        const int kbn = K / kQBlock;
#pragma unroll
        for (int s = 0; s < C::STEPS; ++s) {
          const int kblk = st * C::STEPS + s;
          if (kblk * kQBlock >= K) break;
          float sw0, sw1;
          if (MODE == kGateUp) {
            sw0 = Ws[(nrow0 / kQBlock) * kbn + kblk];
            sw1 = Ws[(nrow1 / kQBlock) * kbn + kblk];
          } else {
            sw0 = Ws[(nrow0 / kQBlock) * kbn + kblk];
            sw1 = sw0;  // both n-blocks lie in one 128-row block
          }
          i32x8_t b0v, b1v;
          {
            const uint4 p0 = f.v[0][s][0], p1 = f.v[0][s][1];
            b0v = i32x8_t{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
            const uint4 q0 = f.v[1][s][0], q1 = f.v[1][s][1];
            b1v = i32x8_t{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
          }
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) {
            if (mb < nmb) {
              const uint8_t *ap = la + mb * 16 * C::LDS_STRIDE + s * C::KSTEP;
              const uint4 p0 = *reinterpret_cast<const uint4 *>(ap);
              const uint4 p1 = *reinterpret_cast<const uint4 *>(ap + 16);
              const i32x8_t a8 = i32x8_t{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
              const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
              const f32x4_t p0r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b0v, z, 0, 0, 0, 127, 0, 127);
              const f32x4_t p1r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b1v, z, 0, 0, 0, 127, 0, 127);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float sa = sa2[buf][s][mb * 16 + (lane >> 4) * 4 + i];
                acc[mb][0][i] = fmaf(p0r[i], sa * sw0, acc[mb][0][i]);
                acc[mb][1][i] = fmaf(p1r[i], sa * sw1, acc[mb][1][i]);
              }
            }
          }
        }
      }
    };

    // ---- K loop: A double-buffered in LDS, B one stage ahead in registers ----
    load_a(0);
    load_b<DT, MODE, NW>(bf[0], b0, b1, 0, K * C::ESZ);
    __syncthreads();            // previous unit's readers are done with LDS
    store_a(0, 0);
    __syncthreads();
    for (int st = 0; st < nstage; st += 2) {
      // even stage: compute from buffer 0 / bf[0]
      if (st + 1 < nstage) {
        load_a(st + 1);
        load_b<DT, MODE, NW>(bf[1], b0, b1, (st + 1) * C::ROW_BYTES, K * C::ESZ);
      }
      compute(0, bf[0], st);
      if (st + 1 < nstage) store_a(1, st + 1);
      __syncthreads();
      if (st + 1 >= nstage) break;
      // odd stage: compute from buffer 1 / bf[1]
      if (st + 2 < nstage) {
        load_a(st + 2);
        load_b<DT, MODE, NW>(bf[0], b0, b1, (st + 2) * C::ROW_BYTES, K * C::ESZ);
      }
      compute(1, bf[1], st + 1);
      if (st + 2 < nstage) store_a(0, st + 2);
      __syncthreads();
    }

    // ---- epilogue ----
    const int col_l = lane & 15;
    const int rsub = (lane >> 4) * 4;
    if constexpr (MODE == kGateUp) {
      const int hc = nrow0 + col_l;   // h column
      const size_t hrow_elems = inter;
      uint8_t *hbase = static_cast<uint8_t *>(shared ? a.w.h_sh : a.w.h) +
                       static_cast<size_t>(seg0 + row0) * hrow_elems * C::ESZ;
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          if (mb < nmb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int rr = mb * 16 + rsub + i;
              if (wave_on && rr < rows) {
                const float hv = silu(acc[mb][0][i]) * acc[mb][1][i];
                reinterpret_cast<uint16_t *>(hbase)[static_cast<size_t>(rr) * hrow_elems + hc] = f32_to_bf16(hv);
              }
            }
          }
        }
      } else {
        // fp8: amax of each row over the block's 128 columns
        float *wmax = reinterpret_cast<float *>(lds);   // [NW][BM]
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float hv = mb < nmb ? silu(acc[mb][0][i]) * acc[mb][1][i] : 0.f;
            acc[mb][0][i] = hv;
            float am = fabsf(hv);
            am = fmaxf(am, __shfl_xor(am, 1));
            am = fmaxf(am, __shfl_xor(am, 2));
            am = fmaxf(am, __shfl_xor(am, 4));
            am = fmaxf(am, __shfl_xor(am, 8));
            if (col_l == 0) wmax[wave * C::BM + mb * 16 + rsub + i] = am;
          }
        }
        __syncthreads();
        float *hs = (shared ? a.w.h_sh_scale : a.w.h_scale) +
                    static_cast<size_t>(seg0 + row0) * (inter / kQBlock) + ntile;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          if (mb < nmb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int rr = mb * 16 + rsub + i;
              float amax = 0.f;
#pragma unroll
              for (int w2 = 0; w2 < NW; ++w2) amax = fmaxf(amax, wmax[w2 * C::BM + rr]);
              const float sc = amax > 0.f ? amax / kE4M3Max : 1.0f;
              if (rr < rows) {
                const int code = fp8_pack2(acc[mb][0][i] / sc, 0.f) & 0xff;
                hbase[static_cast<size_t>(rr) * hrow_elems + hc] = static_cast<uint8_t>(code);
                if (wave == 0 && col_l == 0) hs[static_cast<size_t>(rr) * (inter / kQBlock)] = sc;
              }
            }
          }
        }
      }
    } else {
      uint16_t *ybase = static_cast<uint16_t *>(shared ? a.w.y_sh : a.w.y) +
                        static_cast<size_t>(seg0 + row0) * d.H;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        if (mb < nmb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = mb * 16 + rsub + i;
            if (wave_on && rr < rows) {
              ybase[static_cast<size_t>(rr) * d.H + nrow0 + col_l] = f32_to_bf16(acc[mb][0][i]);
              ybase[static_cast<size_t>(rr) * d.H + nrow1 + col_l] = f32_to_bf16(acc[mb][1][i]);
            }
          }
        }
      }
    }
  }
}

static int cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

template <int DT, int MODE, int NW>
static hipError_t launch_one(const GroupedArgs &ga, int wg_per_cu, hipStream_t s) {
  using C = GCfg<DT, MODE, NW>;
  auto kern = grouped_kernel<DT, MODE, NW>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = (cu_count() * wg_per_cu + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), C::LDS_BYTES, s, ga);
  return hipGetLastError();
}

hipError_t launch_grouped_gateup(const Dims &d, const Inputs &in,
                                 const Work &w, hipStream_t s) {
  GroupedArgs ga{d, in, w, 0, 0};
  if (d.wdt == kBF16) {
    using C = GCfg<kBF16, kGateUp, 4>;
    ga.ntile_routed = (d.I + C::NCOLS - 1) / C::NCOLS;
    ga.ntile_shared = (d.Is + C::NCOLS - 1) / C::NCOLS;
    return launch_one<kBF16, kGateUp, 4>(ga, 2, s);
  }
  using C = GCfg<kFP8, kGateUp, 8>;
  ga.ntile_routed = d.I / C::NCOLS;
  ga.ntile_shared = d.Is / C::NCOLS;
  return launch_one<kFP8, kGateUp, 8>(ga, 1, s);
}

hipError_t launch_grouped_down(const Dims &d, const Inputs &in, const Work &w,
                               hipStream_t s) {
  GroupedArgs ga{d, in, w, 0, 0};
  if (d.wdt == kBF16) {
    using C = GCfg<kBF16, kDown, 4>;
    ga.ntile_routed = ga.ntile_shared = (d.H + C::NCOLS - 1) / C::NCOLS;
    return launch_one<kBF16, kDown, 4>(ga, 2, s);
  }
  using C = GCfg<kFP8, kDown, 4>;
  ga.ntile_routed = ga.ntile_shared = d.H / C::NCOLS;
  return launch_one<kFP8, kDown, 4>(ga, 2, s);
}

}  // namespace moe
