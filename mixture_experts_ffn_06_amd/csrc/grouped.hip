// Grouped down GEMM on MFMA (bf16 and fp8-e4m3 with 128x128 block scales):
// y[rows, H] = h[rows, I] . w2[e]^T for each group's sorted rows.
//
// forward_prefill.rs (page 3, MoeLayer::forward_prefill doc comment) sorts
// token rows by expert so that each expert's weight matrix is loaded once
// for all of its tokens instead of once per token, then runs a grouped gate/up
// GEMM, SiLU gating and a grouped down GEMM (steps 4-6).  Its notes on the
// ported fp8 grouped GEMM describe a weight-stationary per-expert kernel with
// double-buffered prefetch and two-level fp32 block-scale accumulation.  (The
// gate/up GEMM is gateup.hip.)
//
// Layout on CDNA4:
//  * Work units are (group, M tile of BM rows, N tile); group e < E is a
//    routed expert with its rows in sorted order, group E is the shared
//    expert with one row per token.  BM (96 to 192) covers all rows of a
//    typical expert, so each weight byte is streamed from HBM once per call;
//    a persistent grid walks the units, consecutive units on one XCD.
//  * A block is WM x WN waves.  Per K stage every operand byte the block needs
//    -- the h rows (A, one contiguous segment per group) and the w2 rows (B)
//    -- is brought into LDS exactly once by direct global->LDS loads (no
//    register staging), in 1 KB chunks spread evenly over the waves; the WM
//    waves of a column group share its weight chunks, the WN waves of a row
//    group share the h chunks.  The LDS ring is split in two: the h rows
//    (served from L2) in 2 slots, the weights (from HBM) in DEPTH slots, so
//    that several weight stages are in flight while a stage is multiplied.
//  * Chunks are loaded in row order (consecutive lanes take consecutive 16
//    bytes of a row: coalesced), with the 16-byte pieces of each row
//    XOR-swizzled so that the MFMA-order LDS reads are bank-conflict free.
//  * fp8 two-level accumulation: every 128-wide K block is one MFMA
//    (16x16x128, fp32 out) started from zero; its result times (h row scale
//    * weight block scale) is added to the fp32 accumulator.  The output y
//    stays fp32 (it is not rounded to fp8 again, so the fp8 MFMA's summation
//    error stays ~1e-4 of the output).
#include "common.h"
#include "kernels.h"
#include "launch.h"
#include "lds.h"

namespace moe {

__device__ __forceinline__ i32x8_t as_i32x8(u32x4_t a, u32x4_t b) {
  return i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// Tile geometry.  WM x WN waves; a wave owns MBW 16-row m-blocks and NB
// 16-row weight blocks.  K advances in stages of STAGE_K elements = 128 bytes
// of every row (bf16: two MFMA steps of 32; fp8: one 16x16x128 step = one
// scale block).  A "stage block" is 16 rows x 128 bytes, moved by two 1 KB
// load instructions of 8 whole 128-byte row runs each (row-contiguous runs
// stream from HBM faster than the 64-byte pieces of the MFMA layout).
template <int DT, int NB, int WN, int WM, int MBW, int DEPTH, int STAGE_K>
struct GCfg {
  static constexpr int NW = WN * WM;
  static constexpr int THREADS = NW * kWave;
  static constexpr int MB = MBW * WM;
  static constexpr int BM = 16 * MB;
  static constexpr int ESZ = DT == kBF16 ? 2 : 1;
  static constexpr int KSTEP = DT == kBF16 ? 32 : 128;
  static constexpr int SK = STAGE_K;                  // K elements per stage
  static constexpr int STEPS = STAGE_K / KSTEP;     // MFMA steps per stage
  static constexpr int RB = STAGE_K * ESZ;            // bytes of a row in one stage
  static constexpr int BV = 16 * RB / 1024;           // 1 KB chunks per 16-row block
  static constexpr int CPR = RB / 16;                 // 16-byte pieces per row
  static constexpr int RPI = 1024 / RB;               // rows per load instruction
  static constexpr int SWZ_DIV = 256 / RB;            // rows per 256-byte bank window
  static constexpr int A_CH = MB * BV;                // chunks per stage: A ...
  static constexpr int B_CH = WN * NB * BV;           // ... and B
  static constexpr bool SCALED = DT == kFP8;
  static constexpr int A_BYTES = A_CH * 1024;
  static constexpr int B_BYTES = B_CH * 1024;
  // fp8: one 256-byte scale area per wave: areas 0 .. BM/64-1 hold the row
  // scales of rows 0 .. BM-1, area BM/64 the WN*NB weight-block scales.
  static constexpr int S_BYTES = SCALED ? NW * 256 : 0;
  static constexpr int ROW_WAVES = (BM + 63) / 64;
  // split ring: A in DA slots, then B (+ fp8 scales) in DEPTH slots; each
  // wave loads CPA A chunks and CPB B chunks (+ one scale load) per stage
  static constexpr int DA = 2;
  static constexpr int B_STAGE = B_BYTES + S_BYTES;
  static constexpr int CPA = A_CH / NW;
  static constexpr int CPB = B_CH / NW;
  static constexpr int LA = CPA, LB = CPB + (SCALED ? 1 : 0);
  static constexpr int LDS_BYTES = DA * A_BYTES + DEPTH * B_STAGE;
  // output columns per wave and per block
  static constexpr int WCOLS = 16 * NB;
  static constexpr int NCOLS = WN * WCOLS;
  static_assert(STAGE_K % KSTEP == 0, "stage = whole MFMA steps");
  static_assert(RB == 128, "stage rows of 128 bytes (swizzle, chunk and read layout)");
  static_assert(A_CH % NW == 0 && B_CH % NW == 0, "A and B chunks spread evenly over the waves");
  static_assert(!SCALED || (ROW_WAVES < NW && WN * NB <= 64), "fp8 scale areas");
  static_assert(SCALED ? DEPTH == 3 : (DEPTH >= 3 && (DEPTH - 2) * LB < 64),
                "ring depth (fp8 loop: 3 weight slots; bf16: >= 3) and vmcnt range");
  static_assert(!SCALED || 128 % WCOLS == 0, "fp8: a wave's columns lie in one 128-wide scale block");
};

struct GroupedArgs {
  Dims d;
  Inputs in;
  Work w;
  int ntile_routed;   // N tiles of a routed expert
  int ntile_shared;   // N tiles of the shared expert
  int order;          // kOrderGroups or kOrderSharedFirst (bf16)
};

// A launch with units for at most kFewRounds rounds of the grid deals them to
// the XCDs in chunks of kFewChunk units (else one chunk per block of an XCD).
constexpr int kFewRounds = 8;
constexpr int kFewChunk = 8;

// Order in which the persistent blocks take the units.
enum : int {
  kOrderGroups = 0,       // routed experts in order, then the shared expert
  kOrderSharedFirst = 1   // shared-expert units first (longest first when I_s > I)
};

template <int DT, int NB, int WN, int WM, int MBW, int DEPTH, int STAGE_K>
__global__ __launch_bounds__(WN * WM * 64, 1) void grouped_kernel(GroupedArgs a) {
  using C = GCfg<DT, NB, WN, WM, MBW, DEPTH, STAGE_K>;
  extern __shared__ __align__(1024) uint8_t lds[];
  __shared__ int uoff[1026];          // unit prefix over groups (E + 1 groups)
  __shared__ int wsum[C::NW];
  const Dims &d = a.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int G = d.E + (d.Is > 0 ? 1 : 0);
  const int *offsets = a.w.offsets;
  // this block's next ticket from its XCD's unit queue (the prefix's
  // barriers publish the first one)
  __shared__ int tk_next;
  int *const queue = a.w.queue + kQueueStride * (8 + (blockIdx.x & 7));
  if (tid == 0) tk_next = atomicAdd(queue, 1);

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
    for (int i = 0; i < C::NW; ++i) base += i < wave ? wsum[i] : 0;
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
  const int xcd = blockIdx.x & 7;
  // Units go to the XCDs in chunks of consecutive units (chunk c to XCD
  // c % 8: units of one expert run side by side on one L2), and each XCD's
  // blocks take its units in order, one ticket of the XCD's counter each, so
  // a block that finishes early takes the next unit.  A short launch (units
  // for at most kFewRounds rounds of the grid) deals chunks of kFewChunk
  // units, which spreads long units over the XCDs.
  const int chunk = total <= kFewRounds * P ? kFewChunk : P / 8;

  // Piece position p of row r inside a step block holds the row's 16-byte
  // piece p ^ swz(r).
  auto swz = [](int r) { return (r / C::SWZ_DIV) % C::CPR; };
  const int lrow = lane / C::CPR;                    // row of this lane in a load instruction
  const int lpiece = lane % C::CPR;

  for (;;) {
    __syncthreads();   // tk_next holds this block's ticket
    const int tk = tk_next;
    const int u = (tk / chunk) * (8 * chunk) + xcd * chunk + tk % chunk;   // increasing in tk
    if (u >= total) break;
    // Position u runs unit uu.  The S shared-expert units are last in group
    // order; kOrderSharedFirst runs them first, so that longer units (K = I_s
    // > I) do not form the tail.  (fp8 kernels: compiled out.)
    int uu = u;
    if (DT == kBF16 && a.order == kOrderSharedFirst) {
      const int S = d.Is > 0 ? total - uoff[d.E] : 0;
      if (S > 0 && S < total) uu = u < S ? (total - S) + u : u - S;
    }
    // ---- decode the unit (all values block-uniform) ----
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uoff[mid] <= uu) lo = mid; else hi = mid - 1;
    }
    const int g = uniform(lo);
    const bool shared = g == d.E;
    const int grows = uniform(shared ? d.m : offsets[g + 1] - offsets[g]);
    const int nmt = (grows + C::BM - 1) / C::BM;
    const int local = uu - uniform(uoff[g]);
    const int ntile = local / nmt;
    const int row0 = (local - ntile * nmt) * C::BM;
    const int rows = min(C::BM, grows - row0);
    const int nmb = (rows + 15) >> 4;
    const int seg0 = shared ? 0 : uniform(offsets[g]);   // first sorted row of the group
    const int inter = shared ? d.Is : d.I;
    const int K = inter;
    const int kbytes = K * C::ESZ;
    const int nstage = (K + C::SK - 1) / C::SK;

    // ---- weights of the group ----
    const uint8_t *Wb = static_cast<const uint8_t *>(shared ? a.in.sw2 : a.in.w2) +
                        (shared ? 0 : static_cast<size_t>(g) * d.H * d.I * C::ESZ);
    const float *Ws = nullptr;
    if (DT == kFP8)
      Ws = shared ? a.in.sw2_scale
                  : a.in.w2_scale + static_cast<size_t>(g) * (d.H / kQBlock) * (d.I / kQBlock);
    // Output column of block j of column group cg, and its first weight row.
    // Blocks past the last column of a partial N tile read row 0 (valid
    // memory) and store nothing.
    auto col_of = [&](int cg, int j) -> int { return ntile * C::NCOLS + cg * C::WCOLS + 16 * j; };
    auto wrow_of = [&](int cg, int j) -> int {
      const int c = col_of(cg, j);
      return c >= d.H ? 0 : c;
    };
    // Operand bases (block-uniform) and 32-bit byte offsets from them; the
    // plan limits every operand to < 2 GiB so offsets fit.  The group's h
    // rows are one contiguous segment of the sorted rows.
    const uint8_t *Ab = static_cast<const uint8_t *>(shared ? a.w.h_sh : a.w.h);
    auto a_off = [&](int rr) -> uint32_t {
      rr = min(rr, rows - 1);   // rows past the tile's end repeat its last row
      return static_cast<uint32_t>(seg0 + row0 + rr) * kbytes;
    };

    // ---- this wave's share of every stage's chunks ----
    // A chunk c = wave * CPA + q: A stage block c / BV, instruction c % BV;
    // B chunk c = wave * CPB + q: B stage block (cg, j) = c / BV, instruction
    // c % BV.  dst = c * 1 KB in the stage's A or B slot.  The lane's source
    // is Ab + coffA[q] (Wb + coffB[q]) + the stage's K offset; cpcA / cpcB
    // hold the lane's piece offset inside the stage (bf16 partial stages).
    uint32_t coffA[C::CPA], coffB[C::CPB];
    int cpcA[C::CPA], cpcB[C::CPB];
#pragma unroll
    for (int q = 0; q < C::CPA; ++q) {
      const int c = wave * C::CPA + q;
      const int rl = (c % C::BV) * C::RPI + lrow;     // row inside the stage block
      cpcA[q] = (lpiece ^ swz(rl)) * 16;              // this lane's piece, swizzled
      coffA[q] = a_off((c / C::BV) * 16 + rl) + cpcA[q];
    }
#pragma unroll
    for (int q = 0; q < C::CPB; ++q) {
      const int c = wave * C::CPB + q;
      const int rl = (c % C::BV) * C::RPI + lrow;
      const int blk = c / C::BV;
      cpcB[q] = (lpiece ^ swz(rl)) * 16;
      coffB[q] = static_cast<uint32_t>(wrow_of(blk / NB, blk % NB) + rl) * kbytes + cpcB[q];
    }
    // fp8 scales: waves < ROW_WAVES fetch h row scales (lane l: row 64w + l),
    // the other waves the weight-block scales (lane b: block b = cg*NB + j)
    const float *sbase = nullptr;
    uint32_t soff = 0;
    if constexpr (C::SCALED) {
      if (wave < C::ROW_WAVES) {
        const int rr = min(64 * wave + lane, rows - 1);
        sbase = shared ? a.w.h_sh_scale : a.w.h_scale;
        soff = static_cast<uint32_t>(seg0 + row0 + rr) * (inter / kQBlock);
      } else {
        const int b = min(lane, WN * NB - 1);
        sbase = Ws;
        soff = static_cast<uint32_t>(wrow_of(b / NB, b % NB) / kQBlock) * (K / kQBlock);
      }
    }

    // Buffer resources over the operands (an offset past an extent reads
    // zeros): the h rows of the group's kind, the group's w2, this wave's
    // scale table.
    const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(Ab, static_cast<uint32_t>(shared ? d.m : d.te) * kbytes);
    const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(Wb, static_cast<uint32_t>(d.H) * kbytes);
    __amdgpu_buffer_rsrc_t rS = rA;
    if constexpr (C::SCALED)
      rS = buffer_rsrc(sbase, wave < C::ROW_WAVES
                                  ? static_cast<uint32_t>(shared ? d.m : d.te) * (inter / kQBlock) * 4u
                                  : static_cast<uint32_t>(d.H / kQBlock) * (K / kQBlock) * 4u);

    // A of stage st goes to A slot st % DA, B (and the fp8 scales) to B slot
    // st % DEPTH.  A partial last stage (bf16, K % 64 = 32) loads the pieces
    // past the row end from K = 0: valid memory, and compute skips that step
    // (fp8 K is a multiple of the stage).
    auto src_off = [&](uint32_t co, int pc, uint32_t kb) -> uint32_t {
      if constexpr (DT == kBF16)
        if (kb + pc >= static_cast<uint32_t>(kbytes)) return co - pc;
      return co + kb;
    };
    // (slot_st: the stage whose ring slot the loads fill -- by default the
    // stage itself; past the end of K the last stage is loaded again into
    // the slot of the stage after it, which no one reads)
    auto issue_a = [&](int st, int slot_st) {
      uint8_t *sl = lds + (slot_st % C::DA) * C::A_BYTES;
      const uint32_t kb = static_cast<uint32_t>(st) * C::RB;
#pragma unroll
      for (int q = 0; q < C::CPA; ++q)   // m-blocks past the rows are not loaded
        if ((wave * C::CPA + q) / C::BV < nmb)
          buf16_to_lds(rA, src_off(coffA[q], cpcA[q], kb), sl + (wave * C::CPA + q) * 1024);
    };
    auto issue_b = [&](int st, int slot_st) {
      uint8_t *sl = lds + C::DA * C::A_BYTES + (slot_st % DEPTH) * C::B_STAGE;
      const uint32_t kb = static_cast<uint32_t>(st) * C::RB;
#pragma unroll
      for (int q = 0; q < C::CPB; ++q)
        buf16_to_lds(rW, src_off(coffB[q], cpcB[q], kb), sl + (wave * C::CPB + q) * 1024);
      if constexpr (C::SCALED) buf4_to_lds(rS, 4 * (soff + st), sl + C::B_BYTES + wave * 256);
    };

    f32x4_t acc[MBW][NB];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[mb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // The wave's m-blocks: bf16 MBW consecutive ones from mb0; fp8 every
    // WM-th from wm, so that a tile only partly filled with rows (the common
    // case for 192-row tiles) leaves the WM row waves equal work, and the
    // blocks past the rows are skipped.
    const int mb0 = wm * MBW;
    const int mfirst = C::SCALED ? wm : mb0, mstep = C::SCALED ? WM : 1;
    auto mrow = [&](int mb) { return mfirst + mstep * mb; };
    const bool rows_on = mfirst < nmb;        // any of its rows exist

    // lane L reads row L % 16 of a stage block at the swizzled positions of
    // its 16-byte pieces: bf16 step s is logical piece 4 s + L / 16 (loff[s]);
    // fp8 (one 128-wide step, 32 bytes per lane) takes pieces L / 16 and
    // 4 + L / 16 (loff[0], loff[1]).  Any split of the 128 K bytes over the
    // lanes gives the same product as long as A and B use the same one; this
    // one makes each read instruction touch the same pieces as a bf16 read,
    // which the swizzle keeps free of LDS bank conflicts (pieces 2 L/16 and
    // 2 L/16 + 1 conflicted).
    const int rr16 = lane & 15, kg = lane >> 4;
    constexpr int NOFF = DT == kBF16 ? C::STEPS : 2;
    uint32_t loff[NOFF];
#pragma unroll
    for (int s = 0; s < NOFF; ++s) {
      const int piece = 4 * s + kg;
      loff[s] = rr16 * C::RB + ((piece ^ swz(rr16)) * 16);
    }

    // ---- stage operands: LDS -> registers, issued one stage ahead ----
    // bf16: a[s * MBW + mb], b[s * NB + j] (one 16-byte piece per lane each);
    // fp8: a[2 mb + h], b[2 j + h] (the lane's two pieces of a 128-wide step).
    constexpr int NA = DT == kBF16 ? C::STEPS * MBW : 2 * MBW;
    constexpr int NBR = DT == kBF16 ? C::STEPS * NB : 2 * NB;
    struct Regs {
      u32x4_t a[NA];
      u32x4_t b[NBR];
    };
    constexpr int BLK = 16 * C::RB;   // bytes of a stage block
    auto read_stage = [&](int st, Regs &R) {
      const uint8_t *la = lds + (st % C::DA) * C::A_BYTES + mb0 * BLK;
      const uint8_t *lb = lds + C::DA * C::A_BYTES + (st % DEPTH) * C::B_STAGE + wn * NB * BLK;
      // bf16 a[s * MBW + mb] / b[s * NB + j]: piece loff[s] of block mb / j;
      // fp8 a[2 mb + h] / b[2 j + h]: piece loff[h]
      static_for<0, NA>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int o = DT == kBF16 ? i / MBW : i % 2, blk = DT == kBF16 ? i % MBW : i / 2;
        R.a[i] = lds_load<u32x4_t>(la + loff[o] + blk * BLK);
      });
      static_for<0, NBR>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int o = DT == kBF16 ? i / NB : i % 2, blk = DT == kBF16 ? i % NB : i / 2;
        R.b[i] = lds_load<u32x4_t>(lb + loff[o] + blk * BLK);
      });
    };

    auto compute = [&](int st, const Regs &R) {
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int s = 0; s < C::STEPS; ++s) {
          if (st * C::SK + s * C::KSTEP < K) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
              for (int j = 0; j < NB; ++j)
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, R.a[s * MBW + mb]),
                    __builtin_bit_cast(bf16x8_t, R.b[s * NB + j]), acc[mb][j], 0, 0, 0);
          }
        }
      }
    };

    // fp8 stage st on the fp8 MFMA: its fp32 output is not rounded to fp8
    // again, so the MFMA's short summation (it drops product bits below
    // ~2^-14 of the largest product in each group of eight) stays ~1e-4 of
    // the output.
    // NMB: the wave's first NMB m-blocks (all those with rows), a template
    // parameter so that reads and MFMAs carry no branches and the compiler's
    // read waits stay exact.
    auto compute_fp8 = [&](int st, auto nmbc) {
      constexpr int NMB = decltype(nmbc)::value;
      if constexpr (C::SCALED) {
        const uint8_t *sa = lds + (st % C::DA) * C::A_BYTES;
        const uint8_t *sb = lds + C::DA * C::A_BYTES + (st % DEPTH) * C::B_STAGE;
        const uint8_t *la0 = sa + wm * BLK + loff[0];
        const uint8_t *lb0 = sb + wn * NB * BLK + loff[0];
        const uint32_t d1 = loff[1] - loff[0];   // the lane's second piece
        const uint8_t *ssc = sb + C::B_BYTES;
        // Reads in the order the MFMAs use them -- the weight-block scales
        // and the wave's weight blocks, then per m-block its A pieces and
        // row scales (rows mrow(mb)*16 + 4*kg + i: contiguous floats) -- so
        // the first MFMA waits only for the weights and the first m-block,
        // not for every read of the stage.
        u32x4_t aq[2 * MBW], sv[MBW], sw[NB / 4], bq[2 * NB];
        const uint8_t *lsr = ssc + ((wm * 16) + 4 * kg) * 4;
        const uint8_t *lsw = ssc + C::ROW_WAVES * 256 + wn * NB * 4;
        static_for<0, NB / 4>([&](auto ic) {
          constexpr int q = decltype(ic)::value;
          sw[q] = lds_load<u32x4_t>(lsw + q * 16);
        });
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          bq[2 * j] = lds_load<u32x4_t>(lb0 + j * BLK);
          bq[2 * j + 1] = lds_load<u32x4_t>(lb0 + d1 + j * BLK);
        }
        __builtin_amdgcn_sched_barrier(0);
        // m-blocks past the rows are neither read nor multiplied; an
        // m-block's reads go out two m-blocks ahead of its MFMAs
        auto load_mb = [&](auto ic) {
          constexpr int mb = decltype(ic)::value;
          aq[2 * mb] = lds_load<u32x4_t>(la0 + mb * WM * BLK);
          aq[2 * mb + 1] = lds_load<u32x4_t>(la0 + d1 + mb * WM * BLK);
          sv[mb] = lds_load<u32x4_t>(lsr + mb * WM * 64);
          __builtin_amdgcn_sched_barrier(0);
        };
        static_for<0, (NMB < 2 ? NMB : 2)>([&](auto ic) { load_mb(ic); });
        static_for<0, NMB>([&](auto ic) {
          constexpr int mb = decltype(ic)::value;
          if constexpr (mb + 2 < NMB) load_mb(std::integral_constant<int, mb + 2>{});
          // h row scale x weight-block scale: the wave's blocks are 16 * NB
          // <= 64 consecutive 16-aligned output columns, inside one
          // 128-row weight-scale block
          const float ws = __uint_as_float(sw[0][0]);
          float sc[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[i] = __uint_as_float(sv[mb][i]) * ws;
          const i32x8_t av = as_i32x8(aq[2 * mb], aq[2 * mb + 1]);
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                av, as_i32x8(bq[2 * j], bq[2 * j + 1]), z, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][j][i] = fmaf(p[i], sc[i], acc[mb][j][i]);
          }
          __builtin_amdgcn_sched_barrier(0);   // m-block by m-block, as the reads arrive
        });
      }
    };

    __syncthreads();   // every wave has read its ticket (tk_next is refilled at the unit's end)
    // the ticket after this one, fetched while the unit runs (issued after
    // the unit's own global loads above: loads complete in order)
    int tk_new = 0;
    if (tid == 0) tk_new = atomicAdd(queue, 1);
    if constexpr (DT == kBF16) {
      // ---- bf16: split ring (A 2 slots, B DEPTH slots), one barrier per
      // stage, operands read into registers one stage ahead.  Issue order:
      // B0 A0 B1 .. B(D-2) [stage 0 read] A1 B(D-1) | A2 BD | A3 B(D+1) | ...  Step st
      // waits for its own loads up to A(st+1) (only B(st+D-1) was issued
      // after it; B(st+1) precedes it), passes the barrier -- every wave's
      // stage st+1 has landed, and every wave has read stage st into
      // registers -- refills the slots of stage st with A(st+2) and
      // B(st+D), issues the LDS reads of stage st+1, multiplies stage st
      // from registers, then waits for those reads: the reads of one stage
      // overlap the MFMAs of the previous one. ----
      Regs RA, RB;
      auto step = [&](int st, Regs &cur, Regs &next) {
        if (st + DEPTH - 1 < nstage) wait_vm<C::LB>();
        else wait_vm<0>();
        ring_barrier();
        if (st + 2 < nstage) issue_a(st + 2, st + 2);
        if (st + DEPTH < nstage) issue_b(st + DEPTH, st + DEPTH);
        if (rows_on) {
          if (st + 1 < nstage) read_stage(st + 1, next);
          __builtin_amdgcn_sched_barrier(0);
          compute(st, cur);
          __builtin_amdgcn_sched_barrier(0);
          // the reads of stage st + 1 land before the next barrier, which
          // hands their slots to the loads (unconditional: the compiler then
          // knows on every path that no read is outstanding)
          wait_lgkm<0>();
        }
      };
      issue_b(0, 0);
      issue_a(0, 0);
      static_for<1, DEPTH - 1>([&](auto ic) {
        if (decltype(ic)::value < nstage) issue_b(decltype(ic)::value, decltype(ic)::value);
      });
      // issued after A(0): B(1 .. D-2), where they exist (a wave's A loads
      // per stage vary with the tile's rows, so waits only ever count B loads)
      if (nstage >= DEPTH - 1) wait_vm<(DEPTH - 2) * C::LB>();
      else wait_vm<0>();
      ring_barrier();   // stage 0 landed
      if (rows_on) {
        read_stage(0, RA);
        wait_lgkm<0>();
      }
      if (nstage > 1) issue_a(1, 1);
      if (DEPTH - 1 < nstage) issue_b(DEPTH - 1, DEPTH - 1);
      for (int st = 0; st < nstage; st += 2) {
        step(st, RA, RB);
        if (st + 1 >= nstage) break;
        step(st + 1, RB, RA);
      }
    } else {
      // ---- fp8: split ring (A 2 slots, B 3 slots), one barrier per stage.
      // Issue order: B0 A0 B1 | A1 B2 | A2 B3 | ...  Step st waits for its
      // own loads up to A(st) (only B(st+1) was issued after it; B(st)
      // precedes it), passes the barrier -- every wave's stage st has landed
      // and every wave is done with stage st - 1 -- then refills the slots of
      // stage st - 1 with A(st+1) and B(st+2) and multiplies stage st.  Every
      // step issues both (past the end of K, the last stage again into the
      // free slots), so the count is the same along every path and the loop
      // has no branch around its loads. ----
      const int last = nstage - 1;
      auto run_fp8 = [&](auto nmbc) {
        issue_b(0, 0);
        issue_a(0, 0);
        issue_b(min(1, last), 1);
#pragma unroll 1
        for (int st = 0; st < nstage; ++st) {
          __builtin_amdgcn_sched_barrier(0);   // nothing moves across a stage boundary
          wait_vm<C::LB>();
          wait_lgkm<0>();   // the previous stage's reads have landed
          ring_barrier();
          issue_a(min(st + 1, last), st + 1);
          issue_b(min(st + 2, last), st + 2);
          if constexpr (decltype(nmbc)::value > 0) compute_fp8(st, nmbc);
        }
      };
      // the wave's m-blocks with rows: mrow(mb) = mfirst + WM mb < nmb.
      // Four loop variants (more cost registers): all MBW, MBW - 1, up to
      // MBW - 2 (the m-blocks past the rows are then read and multiplied
      // but not stored: their rows lie past the tile's), none.
      const int nmbw = rows_on ? min(MBW, (nmb - mfirst + WM - 1) / WM) : 0;
      if (nmbw == MBW) run_fp8(std::integral_constant<int, MBW>{});
      else if (nmbw == MBW - 1) run_fp8(std::integral_constant<int, MBW - 1>{});
      else if (nmbw > 0) run_fp8(std::integral_constant<int, MBW - 2>{});
      else run_fp8(std::integral_constant<int, 0>{});
    }
    __syncthreads();

    // ---- epilogue ----
    const int cl = lane & 15;
    const int rsub = (lane >> 4) * 4;
    const int col0 = ntile * C::NCOLS + wn * C::WCOLS;
    float *ybase = (shared ? a.w.y_sh : a.w.y) + static_cast<size_t>(seg0 + row0) * d.H;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = mrow(mb) * 16 + rsub + i;
        if (rr < rows) {
#pragma unroll
          for (int j = 0; j < NB; ++j)
            if (col0 + 16 * j < d.H)
              ybase[static_cast<size_t>(rr) * d.H + col0 + 16 * j + cl] = acc[mb][j][i];
        }
      }
    }
    // every wave has read tk_next (the barrier before the ring)
    if (tid == 0) tk_next = tk_new;
  }
}

template <int DT, int NB, int WN, int WM, int MBW, int DEPTH, int STAGE_K>
static hipError_t launch_one(GroupedArgs ga, hipStream_t s) {
  using C = GCfg<DT, NB, WN, WM, MBW, DEPTH, STAGE_K>;
  auto kern = grouped_kernel<DT, NB, WN, WM, MBW, DEPTH, STAGE_K>;
  static const KernelSetup su = kernel_setup(reinterpret_cast<const void *>(kern), C::THREADS, C::LDS_BYTES);
  if (su.err != hipSuccess) return su.err;
  const int blocks_per_cu = su.blocks_per_cu;
  ga.ntile_routed = (ga.d.H + C::NCOLS - 1) / C::NCOLS;
  ga.ntile_shared = ga.ntile_routed;
  const int grid = (device_cus() * blocks_per_cu + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), C::LDS_BYTES, s, ga);
  return hipGetLastError();
}

// Large tiles when experts average more than 96 rows, small ones otherwise
// (fewer idle rows per tile).
static bool big_tiles(const Dims &d) { return d.te > 96 * d.E; }

hipError_t launch_grouped_down(const Dims &d, const Inputs &in, const Work &w,
                               hipStream_t s) {
  GroupedArgs ga{d, in, w, 0, 0, kOrderGroups};
  if (d.wdt == kBF16) {
    if (big_tiles(d)) return launch_one<kBF16, 4, 4, 2, 4, 3, 64>(ga, s);   // 128 rows x 256 columns, 8 waves
    // 96-row tiles, shared-expert units first (prefill down 143 -> 136 us)
    ga.order = kOrderSharedFirst;
    return launch_one<kBF16, 4, 4, 1, 6, 4, 64>(ga, s);
  }
  // 192 (128) rows x 256 columns, 8 waves
  if (big_tiles(d)) return launch_one<kFP8, 4, 4, 2, 6, 3, 128>(ga, s);
  return launch_one<kFP8, 4, 4, 2, 4, 3, 128>(ga, s);
}

}  // namespace moe
