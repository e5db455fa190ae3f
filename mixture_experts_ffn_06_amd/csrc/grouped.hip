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

// Direct global -> LDS loads of 16 or 4 bytes per lane (global_load_lds_
// dwordx4 / _dword): lane l's bytes land at lds_dst + 16 l (or 4 l).  Completion is
// counted by the issuing wave's vmcnt.
__device__ __forceinline__ void dma16_to_lds(const void *src, void *lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const void *src, void *lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 4, 0, 0);
}

// A value known to be equal on all lanes, moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Wait until at most N vector-memory operations of this wave are
// outstanding (expcnt and lgkmcnt left unconstrained).  The empty asm
// statements keep the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// Block barrier for the LDS ring.  __syncthreads() also releases memory at
// workgroup scope, which on this target waits for every outstanding load --
// including the direct-to-LDS loads of the stages still in flight.  The ring
// only needs the execution barrier: each wave waits for its own loads with
// wait_vm<>() first, and LDS reads of a slot are complete (their values have
// been consumed) before a wave reaches the barrier that frees the slot.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Tile geometry.  A block is NW waves; a tile is BM = 64 token rows (4 MFMA
// m-blocks) by NB 16-row weight blocks per wave.  K advances in stages of 128
// elements: bf16 = 4 MFMA steps of 32, fp8 = one 16x16x128 step (= one fp8
// scale block).  Operands move in 1 KB chunks, one wave load instruction of
// 16 bytes per lane: consecutive lanes take consecutive 16-byte pieces of a
// row (a full 64 or 128-byte row segment per 4 or 8 lanes, so the loads
// coalesce), and the piece positions inside a row are XOR-swizzled by the row
// so that the MFMA-order reads (16 rows per ds_read_b128) hit 16 different
// bank groups.
template <int DT, int MODE, int NB, int NW, int DEPTH>
struct GCfg {
  static constexpr int THREADS = NW * kWave;
  static constexpr int BM = 64;
  static constexpr int MB = BM / 16;
  static constexpr int ESZ = DT == kBF16 ? 2 : 1;          // operand bytes
  static constexpr int KSTEP = DT == kBF16 ? 32 : 128;     // K of one MFMA
  static constexpr int STAGE_K = 128;
  static constexpr int STEPS = STAGE_K / KSTEP;            // MFMA steps per stage
  static constexpr int BV = DT == kBF16 ? 1 : 2;           // chunks per operand
  static constexpr int RB = KSTEP * ESZ;                   // bytes of one row in one MFMA step
  static constexpr int CPR = RB / 16;                      // 16-byte chunks per such row
  static constexpr int RPI = 16 / BV;                      // rows covered by one load instruction
  static constexpr int SWZ_DIV = 16 / CPR;
  static constexpr int A_CH = MB * STEPS * BV;             // A chunks per stage
  static constexpr int A_CPW = A_CH / NW;                  // ... issued per wave
  static constexpr int B_CPW = NB * STEPS * BV;            // B chunks per wave
  static constexpr bool SCALED = DT == kFP8;
  static constexpr int LPS = A_CPW + B_CPW + (SCALED ? 1 : 0);  // loads per stage per wave
  static constexpr int A_BYTES = A_CH * 1024;
  static constexpr int B_BYTES = NW * B_CPW * 1024;
  // fp8: one 256-byte scale area per wave and stage: lanes 0-15 carry the
  // row scales of the wave's A m-block, lanes 16.. the weight block scales
  // of its NB weight blocks.
  static constexpr int S_BYTES = SCALED ? NW * 256 : 0;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int LDS_BYTES = DEPTH * STAGE_BYTES;
  // output columns of one tile: gate/up pairs NB/2 gate with NB/2 up blocks
  static constexpr int WCOLS = MODE == kGateUp ? 16 * NB / 2 : 16 * NB;
  static constexpr int NCOLS = NW * WCOLS;
  static_assert(A_CH % NW == 0, "A chunks split evenly over waves");
  static_assert((STEPS * BV) % A_CPW == 0, "a wave's A chunks lie in one m-block");
  static_assert(LPS * (DEPTH - 1) < 64, "vmcnt range");
};

struct GroupedArgs {
  Dims d;
  Inputs in;
  Work w;
  int ntile_routed;   // N tiles of a routed expert
  int ntile_shared;   // N tiles of the shared expert
};

// LDS reads outside the compiler's wait tracking.  The compiler cannot see
// which LDS bytes the in-flight direct loads will write, and it guards every
// LDS read with a wait for all of them; the ring already orders those with
// wait_vm<>() + ring_barrier(), so these reads are issued as plain
// instructions, each followed in the same asm statement by the wait for it.
__device__ __forceinline__ uint32_t lds_off(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) void *)p));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// All LDS operands of one fp8 stage for one wave, read in a single asm
// statement that ends with the wait for them (so no use or copy of a result
// can be scheduled before its data has arrived):
//   b[0..3]  B chunks (weight block 0: chunks 0,1; block 1: chunks 2,3)
//   a[0..7]  A chunks (m-block mb: chunks 2mb, 2mb+1)
//   s[0..3]  row scales of m-blocks 0..3 for this lane's 4 rows
//   w        weight scales (floats 16..19 of the wave's scale area)
//   (b0/b1, a0/a1: addresses of the lane's first / second 16-byte piece in
//   weight block 0 / m-block 0; blocks are 2 KB apart)
template <int SCALE_STRIDE>
__device__ __forceinline__ void lds_read_fp8_stage(uint32_t b0, uint32_t b1, uint32_t a0, uint32_t a1,
                                                   uint32_t sr, uint32_t sw, u32x4_t (&b)[4],
                                                   u32x4_t (&a)[8], u32x4_t (&sc)[4], u32x4_t &w) {
  asm volatile(
      "ds_read_b128 %0, %17\n"
      "ds_read_b128 %1, %18\n"
      "ds_read_b128 %2, %17 offset:2048\n"
      "ds_read_b128 %3, %18 offset:2048\n"
      "ds_read_b128 %4, %19\n"
      "ds_read_b128 %5, %20\n"
      "ds_read_b128 %6, %19 offset:2048\n"
      "ds_read_b128 %7, %20 offset:2048\n"
      "ds_read_b128 %8, %19 offset:4096\n"
      "ds_read_b128 %9, %20 offset:4096\n"
      "ds_read_b128 %10, %19 offset:6144\n"
      "ds_read_b128 %11, %20 offset:6144\n"
      "ds_read_b128 %12, %21\n"
      "ds_read_b128 %13, %21 offset:%23\n"
      "ds_read_b128 %14, %21 offset:%24\n"
      "ds_read_b128 %15, %21 offset:%25\n"
      "ds_read_b128 %16, %22 offset:64\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]),
        "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]),
        "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7]),
        "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(sc[2]), "=&v"(sc[3]), "=&v"(w)
      : "v"(b0), "v"(b1), "v"(a0), "v"(a1), "v"(sr), "v"(sw),
        "i"(SCALE_STRIDE), "i"(2 * SCALE_STRIDE), "i"(3 * SCALE_STRIDE));
}

__device__ __forceinline__ i32x8_t as_i32x8(u32x4_t a, u32x4_t b) {
  return i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

__device__ __forceinline__ i32x8_t as_i32x8(uint4 a, uint4 b) {
  return i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

template <int DT, int MODE, int NB, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64, 1) void grouped_kernel(GroupedArgs a) {
  using C = GCfg<DT, MODE, NB, NW, DEPTH>;
  extern __shared__ __align__(1024) uint8_t lds[];
  __shared__ int uoff[1026];          // unit prefix over groups (E + 1 groups)
  __shared__ int wsum[NW];
  __shared__ float wmax[NW][C::BM];   // fp8 gate/up epilogue: row amax per wave
  const Dims &d = a.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
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
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
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

  for (int r = 0; r * P < total; ++r) {
    // Consecutive units (same expert and N tile, next M tile) go to
    // consecutive slots of one XCD, so a busy expert's weight slice is read
    // from HBM once and then hit in that XCD's L2.
    const int u = r * P + xcd * per_xcd + slot;
    if (u >= total) continue;
    // ---- decode the unit ----
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uoff[mid] <= u) lo = mid; else hi = mid - 1;
    }
    // Every value of the unit is block-uniform; readfirstlane lets the
    // compiler keep them (and the weight-scale loads they address) scalar.
    const int g = uniform(lo);
    const bool shared = g == d.E;
    const int grows = uniform(shared ? d.m : offsets[g + 1] - offsets[g]);
    const int nmt = (grows + C::BM - 1) / C::BM;
    const int local = u - uniform(uoff[g]);
    const int ntile = local / nmt;
    const int row0 = (local - ntile * nmt) * C::BM;
    const int rows = min(C::BM, grows - row0);
    const int nmb = (rows + 15) >> 4;
    const int seg0 = shared ? 0 : uniform(offsets[g]);   // first sorted row
    const int inter = shared ? d.Is : d.I;
    const int K = MODE == kGateUp ? d.H : inter;
    const int kbytes = K * C::ESZ;
    const int nstage = (K + C::STAGE_K - 1) / C::STAGE_K;

    // ---- weights of this wave: NB blocks of 16 rows ----
    const uint8_t *Wb;
    const float *Ws = nullptr;
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
    const int col0 = ntile * C::NCOLS + wave * C::WCOLS;   // first output column
    // A wave past the last column of a partial N tile streams row 0 (valid
    // memory) and stores nothing.
    const bool wave_on = col0 < (MODE == kGateUp ? inter : d.H);
    int wrow[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (MODE == kGateUp)
        wrow[j] = j < NB / 2 ? col0 + 16 * j : inter + col0 + 16 * (j - NB / 2);
      else
        wrow[j] = col0 + 16 * j;
      if (!wave_on) wrow[j] = 0;
    }
    // Piece position p of row r inside a step block holds the row's
    // 16-byte piece p ^ swz(r).
    auto swz = [](int r) { return (r / C::SWZ_DIV) % C::CPR; };
    const int lrow = lane / C::CPR;                  // row of this lane in a load instruction
    const uint8_t *bp[NB][C::BV];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < C::BV; ++i) {
        const int r = i * C::RPI + lrow;
        bp[j][i] = Wb + static_cast<size_t>(wrow[j] + r) * kbytes + ((lane % C::CPR) ^ swz(r)) * 16;
      }

    // ---- the A rows this wave loads ----
    // Rows past the tile's last row repeat that row (valid memory; their
    // results are never stored).
    auto a_row = [&](int rr) -> const uint8_t * {
      rr = min(rr, rows - 1);
      if (MODE == kGateUp) {
        const int tok = shared ? row0 + rr : a.w.sorted_pair[seg0 + row0 + rr] / d.k;
        if (DT == kFP8) return a.w.xq + static_cast<size_t>(tok) * d.H;
        return static_cast<const uint8_t *>(a.in.x) + static_cast<size_t>(tok) * d.H * 2;
      }
      return static_cast<const uint8_t *>(shared ? a.w.h_sh : a.w.h) +
             static_cast<size_t>(seg0 + row0 + rr) * inter * C::ESZ;
    };
    const uint8_t *ap[C::A_CPW];
#pragma unroll
    for (int il = 0; il < C::A_CPW; ++il) {
      const int c = wave * C::A_CPW + il;
      const int mb = c / (C::STEPS * C::BV), i = c % C::BV;
      const int r = i * C::RPI + lrow;
      ap[il] = a_row(mb * 16 + r) + ((lane % C::CPR) ^ swz(r)) * 16;
    }
    // fp8 row scales: lanes 0-15 fetch rows amb*16 + lane of the wave's m-block
    const int amb = wave * C::A_CPW / (C::STEPS * C::BV);
    const float *srow = nullptr;
    if constexpr (C::SCALED) {
      const int rr = min(amb * 16 + (lane & 15), rows - 1);
      if (MODE == kGateUp) {
        const int tok = shared ? row0 + rr : a.w.sorted_pair[seg0 + row0 + rr] / d.k;
        srow = a.w.sx + static_cast<size_t>(tok) * (d.H / kQBlock);
      } else {
        srow = (shared ? a.w.h_sh_scale : a.w.h_scale) +
               static_cast<size_t>(seg0 + row0 + rr) * (inter / kQBlock);
      }
    }
    // fp8: lane 16 + j fetches the scales of weight block j (row block
    // wrow[j] / 128, one scale per 128-wide K block)
    const float *wsrc = nullptr;
    if constexpr (C::SCALED) {
      const int j = min(max(lane - 16, 0), NB - 1);
      int wr = wrow[0];
#pragma unroll
      for (int q = 1; q < NB; ++q) wr = j == q ? wrow[q] : wr;
      wsrc = Ws + static_cast<size_t>(wr / kQBlock) * (K / kQBlock);
    }

    // ---- issue all loads of one stage into its LDS slot ----
    // K offsets past the end (partial last bf16 stage) read offset 0 instead;
    // the steps they feed are skipped.
    auto issue = [&](int st) {
      uint8_t *sl = lds + (st % DEPTH) * C::STAGE_BYTES;
#pragma unroll
      for (int il = 0; il < C::A_CPW; ++il) {
        const int c = wave * C::A_CPW + il;
        const int s = (c / C::BV) % C::STEPS;
        int kb = (st * C::STAGE_K + s * C::KSTEP) * C::ESZ;
        if (kb >= kbytes) kb = 0;
        dma16_to_lds(ap[il] + kb, sl + c * 1024);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int s = 0; s < C::STEPS; ++s)
#pragma unroll
          for (int i = 0; i < C::BV; ++i) {
            int kb = (st * C::STAGE_K + s * C::KSTEP) * C::ESZ;
            if (kb >= kbytes) kb = 0;
            const int c = (j * C::STEPS + s) * C::BV + i;
            dma16_to_lds(bp[j][i] + kb, sl + C::A_BYTES + (wave * C::B_CPW + c) * 1024);
          }
      if constexpr (C::SCALED) {
        // lanes 0-15: row scales of the wave's m-block (the rows of their A
        // chunks); lanes 16 .. 16+NB-1: the block scales of its weights
        // (all 64 lanes take part: the rest repeat a row scale into the
        // unused tail of the wave's area)
        const float *sp = (lane < 16 || lane >= 16 + NB) ? srow + st : wsrc + st;
        dma4_to_lds(sp, sl + C::A_BYTES + C::B_BYTES + wave * 256);
      }
    };

    f32x4_t acc[C::MB][NB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[mb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int st) {
      const uint8_t *sl = lds + (st % DEPTH) * C::STAGE_BYTES;
      // lane L reads row L % 16, pieces of K slice L / 16, at their
      // swizzled positions
      const int rr = lane & 15, g = lane >> 4;
      const int off0 = rr * C::RB + (((C::BV * g) ^ swz(rr)) * 16);
      const uint8_t *sb = sl + C::A_BYTES + wave * C::B_CPW * 1024 + off0;
      const uint8_t *sa = sl + off0;
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int s = 0; s < C::STEPS; ++s) {
          if (st * C::STAGE_K + s * C::KSTEP < K) {
            bf16x8_t b[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j)
              b[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(sb + (j * C::STEPS + s) * 1024));
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) {
              if (mb < nmb) {
                const bf16x8_t a8 = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4 *>(sa + (mb * C::STEPS + s) * 1024));
#pragma unroll
                for (int j = 0; j < NB; ++j)
                  acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b[j], acc[mb][j], 0, 0, 0);
              }
            }
          }
        }
      } else {
        // one 128-wide K block per stage: partial MFMA from zero, then
        // acc += partial * (A row scale * weight block scale)
        static_assert(NB == 2, "fp8 stage reads are laid out for two weight blocks");
        const uint32_t sc = lds_off(sl + C::A_BYTES + C::B_BYTES);
        constexpr int LW = (C::STEPS * C::BV) / C::A_CPW;   // first loader wave of an m-block
        static_assert(C::MB == 4 && C::A_CH == 8, "fp8 stage read layout");
        u32x4_t bq[4], aq[8], sv[4], sw4;
        // second 16-byte piece of the lane's 32-byte K slice
        const int off1 = rr * C::RB + (((C::BV * g + 1) ^ swz(rr)) * 16);
        // row scales: rows mb*16 + 4*(lane/16) + i of m-block mb sit in the
        // area of wave mb*LW; weight scales: lanes 16, 17 of this wave's area
        lds_read_fp8_stage<LW * 256>(lds_off(sb), lds_off(sb - off0 + off1), lds_off(sa),
                                     lds_off(sa - off0 + off1), sc + (lane >> 4) * 16,
                                     sc + wave * 256, bq, aq, sv, sw4);
        const i32x8_t b[2] = {as_i32x8(bq[0], bq[1]), as_i32x8(bq[2], bq[3])};
        const float sw[2] = {__uint_as_float(sw4.x), __uint_as_float(sw4.y)};
        const i32x8_t av[4] = {as_i32x8(aq[0], aq[1]), as_i32x8(aq[2], aq[3]), as_i32x8(aq[4], aq[5]),
                               as_i32x8(aq[6], aq[7])};
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          if (mb < nmb) {
            const float sr[4] = {__uint_as_float(sv[mb].x), __uint_as_float(sv[mb].y),
                                 __uint_as_float(sv[mb].z), __uint_as_float(sv[mb].w)};
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
              const f32x4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[mb], b[j], z, 0, 0, 0, 127, 0, 127);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[mb][j][i] = fmaf(p[i], sr[i] * sw[j], acc[mb][j][i]);
            }
          }
        }
      }
    };

    // ---- K loop: DEPTH-stage ring of LDS slots filled by direct loads ----
    __syncthreads();   // the previous unit is done with every slot
#pragma unroll
    for (int st = 0; st < DEPTH - 1; ++st)
      if (st < nstage) issue(st);
    for (int st = 0; st < nstage; ++st) {
      if (st > 0) ring_barrier();    // slot (st - 1) % DEPTH is free again
      const int ahead = st + DEPTH - 1;
      if (ahead < nstage) issue(ahead);
      // stages issued after `st`: min(DEPTH - 1, nstage - 1 - st)
      const int later = min(DEPTH - 1, nstage - 1 - st);
      static_assert(DEPTH <= 3, "wait ladder covers DEPTH - 1 <= 2");
      if (later >= 2) wait_vm<2 * C::LPS>();
      else if (later == 1) wait_vm<C::LPS>();
      else wait_vm<0>();
      ring_barrier();                // every wave's loads of stage st landed
      compute(st);
    }
    __syncthreads();

    // ---- epilogue ----
    const int cl = lane & 15;
    const int rsub = (lane >> 4) * 4;
    if constexpr (MODE == kGateUp) {
      constexpr int HALF = NB / 2;
      uint8_t *hbase = static_cast<uint8_t *>(shared ? a.w.h_sh : a.w.h) +
                       static_cast<size_t>(seg0 + row0) * inter * C::ESZ;
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = mb * 16 + rsub + i;
            if (wave_on && rr < rows) {
#pragma unroll
              for (int j = 0; j < HALF; ++j)
                reinterpret_cast<uint16_t *>(hbase)[static_cast<size_t>(rr) * inter + col0 + 16 * j + cl] =
                    f32_to_bf16(silu(acc[mb][j][i]) * acc[mb][j + HALF][i]);
            }
          }
        }
      } else {
        // fp8: h is quantised per row per 128 columns = this tile's columns
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float am = 0.f;
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
              const float hv = silu(acc[mb][j][i]) * acc[mb][j + HALF][i];
              acc[mb][j][i] = hv;
              am = fmaxf(am, fabsf(hv));
            }
            am = fmaxf(am, __shfl_xor(am, 1));
            am = fmaxf(am, __shfl_xor(am, 2));
            am = fmaxf(am, __shfl_xor(am, 4));
            am = fmaxf(am, __shfl_xor(am, 8));
            if (cl == 0) wmax[wave][mb * 16 + rsub + i] = am;
          }
        }
        __syncthreads();
        float *hs = (shared ? a.w.h_sh_scale : a.w.h_scale) +
                    static_cast<size_t>(seg0 + row0) * (inter / kQBlock) + ntile;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = mb * 16 + rsub + i;
            if (rr < rows) {
              float amax = 0.f;
#pragma unroll
              for (int w = 0; w < NW; ++w) amax = fmaxf(amax, wmax[w][rr]);
              const float sc = amax > 0.f ? amax / kE4M3Max : 1.0f;
#pragma unroll
              for (int j = 0; j < HALF; ++j)
                hbase[static_cast<size_t>(rr) * inter + col0 + 16 * j + cl] =
                    static_cast<uint8_t>(fp8_pack2(acc[mb][j][i] / sc, 0.f) & 0xff);
              if (wave == 0 && cl == 0) hs[static_cast<size_t>(rr) * (inter / kQBlock)] = sc;
            }
          }
        }
      }
    } else {
      uint16_t *ybase = static_cast<uint16_t *>(shared ? a.w.y_sh : a.w.y) +
                        static_cast<size_t>(seg0 + row0) * d.H;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = mb * 16 + rsub + i;
          if (wave_on && rr < rows) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
              ybase[static_cast<size_t>(rr) * d.H + col0 + 16 * j + cl] = f32_to_bf16(acc[mb][j][i]);
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

template <int DT, int MODE, int NB, int NW, int DEPTH>
static hipError_t launch_one(const GroupedArgs &ga, hipStream_t s) {
  using C = GCfg<DT, MODE, NB, NW, DEPTH>;
  auto kern = grouped_kernel<DT, MODE, NB, NW, DEPTH>;
  static int blocks_per_cu = 0;
  if (blocks_per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, C::THREADS, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    blocks_per_cu = nb > 0 ? nb : 1;
  }
  const int grid = (cu_count() * blocks_per_cu + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), C::LDS_BYTES, s, ga);
  return hipGetLastError();
}

hipError_t launch_grouped_gateup(const Dims &d, const Inputs &in,
                                 const Work &w, hipStream_t s) {
  GroupedArgs ga{d, in, w, 0, 0};
  if (d.wdt == kBF16) {
    using C = GCfg<kBF16, kGateUp, 2, 4, 3>;
    ga.ntile_routed = (d.I + C::NCOLS - 1) / C::NCOLS;
    ga.ntile_shared = (d.Is + C::NCOLS - 1) / C::NCOLS;
    return launch_one<kBF16, kGateUp, 2, 4, 3>(ga, s);
  }
  using C = GCfg<kFP8, kGateUp, 2, 8, 3>;   // 8 x 16 = 128 h columns = one h scale group
  ga.ntile_routed = d.I / C::NCOLS;
  ga.ntile_shared = d.Is / C::NCOLS;
  return launch_one<kFP8, kGateUp, 2, 8, 3>(ga, s);
}

hipError_t launch_grouped_down(const Dims &d, const Inputs &in, const Work &w,
                               hipStream_t s) {
  GroupedArgs ga{d, in, w, 0, 0};
  if (d.wdt == kBF16) {
    using C = GCfg<kBF16, kDown, 2, 4, 3>;
    ga.ntile_routed = ga.ntile_shared = (d.H + C::NCOLS - 1) / C::NCOLS;
    return launch_one<kBF16, kDown, 2, 4, 3>(ga, s);
  }
  using C = GCfg<kFP8, kDown, 2, 4, 3>;
  ga.ntile_routed = ga.ntile_shared = d.H / C::NCOLS;
  return launch_one<kFP8, kDown, 2, 4, 3>(ga, s);
}

}  // namespace moe
