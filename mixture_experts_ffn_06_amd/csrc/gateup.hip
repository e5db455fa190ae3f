// Grouped gate/up GEMM with the SwiGLU epilogue on the bf16 32x32x16 MFMA
// (bf16 weights, or e4m3 codes converted to their exact bf16 values).
//
// forward_prefill.rs (page 3, MoeLayer::forward_prefill, doc comment
// "Pipeline", steps 4-5) sorts token rows by expert so that each expert's
// weights are loaded once for all of its tokens, then runs the grouped gate/up
// GEMM and the SiLU gate; its notes on the fp8 grouped GEMM describe a
// weight-stationary per-expert kernel with two-level fp32 block-scale
// accumulation.
//
// Layout on CDNA4:
//  * A unit is (group, N tile, M tile): 128 h columns (128 gate rows of w1
//    and the matching 128 up rows of w3) against up to 160 token rows of one
//    group (a routed expert's sorted rows, or the m tokens for the shared
//    expert, group E).  A group's rows split evenly over ceil(rows / 160) M
//    tiles, so an expert of up to 160 rows streams its weights once.
//    Consecutive units are the M tiles of one N tile (else the N tiles of one
//    group) and run side by side on one XCD, so shared operands come from
//    that XCD's L2.
//  * A block is 8 waves, two per SIMD.  Waves 0-3 multiply: wave w owns
//    weight rows [32 w, 32 w + 32) of the gate half and of the up half of the
//    tile, as the M side of the MFMA, and multiplies them with token blocks
//    0-3 (the N side): each lane then holds one token's results, so its
//    activation scale is one value per token block and the block-scale
//    promotion is one FMA per accumulator.  Waves 4-7 move data -- load wave
//    4 + w brings wave w's 64 weight rows, token block w, 8 rows of token
//    block 4 and a share of the fp8 scales -- and, when the tile has rows
//    past 128, load wave 4 + w multiplies wave w's weight rows with token
//    block 4 (rows 128-159) on the same SIMD.  A load instruction holds the
//    CU's address path for many cycles once HBM pushes back, and a wave
//    cannot issue past it; kept out of the multiplying waves, those stalls no
//    longer idle the MFMA.
//  * Per K stage (128 bytes of every row: 64 bf16 or 128 e4m3 elements) the
//    256 weight rows and the token rows go to LDS by direct buffer->LDS
//    loads (16-byte pieces XOR-swizzled per row): weights (and fp8 scales)
//    in three slots, two stages in flight while one is multiplied; token
//    rows (from L2) in two slots, one stage ahead; one barrier per stage.  All
//    waves read LDS with ordinary loads, whose waits the compiler places.
//  * Lane l multiplies row l % 32 of a block and takes 64 of the stage's
//    bytes: pieces P(g, j) = 4 (j / 2) + 2 g + j % 2 for lane group g = l / 32,
//    j = 0..3.  MFMA step s uses piece j = s (bf16) or half s % 2 of piece
//    j = s / 2 (fp8); any split of K over the lanes gives the same product as
//    long as both operands use it, and this one makes the first half of a
//    bf16 stage (steps 0, 1) the first 32 K elements, so a half stage at the
//    end of K runs two steps.
//  * fp8: the accumulators hold the running sum over the 128-wide K blocks
//    divided by the current block's scale (activation row scale x weight
//    block scale) and are rescaled to the next block's scale before its
//    first MFMA; after the last block they are multiplied by its scale.  The fp8
//    MFMA itself is not used here: it drops product bits below ~2^-14 of the
//    largest of each eight products, enough to move SwiGLU outputs across the
//    fp8 rounding boundaries of h.
//  * Epilogue: SwiGLU from the gate and up accumulators (the same layout);
//    bf16 h, or fp8 h quantised per row per 128 columns (the unit's
//    columns: row amax across the four column waves through LDS).
#include "common.h"
#include "kernels.h"
#include "launch.h"
#include "lds.h"

namespace moe {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGuWaves = 4;        // multiplying waves (and as many load waves)
constexpr int kGuThreads = 2 * kGuWaves * kWave;
constexpr int kGuRowBytes = 128;   // bytes of a row per stage
constexpr int kGuWRows = 256;      // weight rows per unit (4 waves x (32 gate + 32 up))
constexpr int kGuMBlocks = 4;      // token blocks of the multiplying waves
constexpr int kGuTBlocks = 5;      // token blocks of 32 rows per unit (block 4 on the load waves)
constexpr int kGuTRows = 32 * kGuTBlocks;
constexpr int kGuDepth = 3;        // weight (and scale) slots
constexpr int kGuTDepth = 2;       // token slots
constexpr int kGuFewRounds = 4;    // unit rounds of the grid up to which a launch counts as short
constexpr int kGuFewChunk = 8;     // units per XCD chunk in a short launch

template <int DT>
struct GuCfg {
  static constexpr int ESZ = DT == kBF16 ? 2 : 1;
  static constexpr int SK = kGuRowBytes / ESZ;              // K elements per stage
  static constexpr int STEPS = SK / 16;                     // MFMA steps per stage
  static constexpr int W_BYTES = kGuWRows * kGuRowBytes;    // 32 KB
  // fp8 scales of two K blocks (this one, at 0, and the next, at 1024): the
  // 160 token rows' scales at 4 r (loaded by waves 4-6, 64 each) and the
  // gate / up weight-block scales at 768 / 772 (wave 7)
  static constexpr int S_BYTES = DT == kFP8 ? 2048 : 0;
  static constexpr int WS_SLOT = W_BYTES + S_BYTES;
  static constexpr int T_BYTES = kGuTRows * kGuRowBytes;    // 20 KB
  static constexpr int T_BASE = kGuDepth * WS_SLOT;         // token slots after the weight slots
  static constexpr int LDS = T_BASE + kGuTDepth * T_BYTES;
  // vector-memory operations per load wave per stage: 8 weight loads, 5
  // token loads, fp8: two 4-byte scale loads (this K block's and the next)
  static constexpr int NW = 8, NTL = 5, NS = DT == kFP8 ? 2 : 0;
  static constexpr int OPS = NW + NTL + NS;
  // left outstanding when a stage's loads have landed: the weight and scale
  // loads of the stage after it
  static constexpr int WAIT = NW + NS;
  static_assert(OPS < 16, "vmcnt range");
  static_assert(LDS <= 146 * 1024, "LDS (with the static arrays)");
};

struct GuArgs {
  Dims d;
  Inputs in;
  Work w;
  int ntile_r;   // N tiles of a routed expert (128 h columns each)
  int ntile_s;   // N tiles of the shared expert
};

// Position of logical 16-byte piece p in row r of a stage: the 16 rows read
// by one quarter of a wave's read instruction land in 16 distinct 16-byte
// bank groups (8 XOR values x the row's 128-byte parity).
__device__ __forceinline__ int gu_swz(int r) { return (r >> 1) & 7; }

// Logical piece of the lane's j-th 16 bytes (lane group g).
__device__ __forceinline__ int gu_piece(int g, int j) { return 4 * (j >> 1) + 2 * g + (j & 1); }

// The load waves' part of one unit.  Weight stage st (and its fp8 scales)
// goes to weight slot st % 3, token stage st to token slot st % 2.  A load
// wave issues weights 0, tokens 0 and weights 1, waits for stage 0, and at
// each stage's barrier (every wave is done with stage st - 1, whose weight
// slot stage st + 2 takes and whose token slot stage st + 1 takes) issues
// tokens st + 1 and weights st + 2 -- past the end the last stage again,
// into a free slot no one reads, so each step leaves exactly WAIT
// operations behind the ones awaited -- then runs work(st) (the fifth token
// block's MFMAs, or nothing) and waits until only the weights st + 2 are
// outstanding: stage st + 1 has landed by the next barrier (loads complete
// in order).  It passes exactly nstage barriers, as the multiplying waves do.
//
// The loads go through buffer resources (buffer_load ... lds): the compiler
// counts LDS reads exactly in a function that holds them (with the
// flat-encoded global_load_lds it falls back to waiting for all LDS reads),
// and an offset past a resource's extent reads zeros instead of faulting.
//
// Weight instruction q (0..7) moves rows 8 (q % 4) + drow of the gate (q < 4)
// or up block (wave-uniform offset (8 (q % 4) + (q >= 4 ? inter : 0)) *
// wstep; wstep = 0 for a wave past the columns: valid memory, never read)
// from lane offsets wl[q % 2]; token instruction q (0..4) from toff[q].
// whi / thi: the lane's piece lies in the second half of the stage's 128
// bytes (in a bf16 half stage -- the last one when K % 64 == 32 -- such
// pieces load the piece 64 bytes before instead: valid memory, and the steps
// that would use them are skipped).
template <int DT, typename F>
__device__ __forceinline__ void gu_load_unit(
    __amdgpu_buffer_rsrc_t rW, __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rS, const uint32_t (&wl)[2],
    const bool (&whi)[2], const uint32_t (&toff)[kGuTBlocks], const bool (&thi)[kGuTBlocks], uint32_t wstep,
    uint32_t inter, uint32_t kbytes, uint32_t soff, int nstage, int wave, uint32_t lds0, F &&work) {
  using C = GuCfg<DT>;
  auto kbs = [&](int st, uint32_t &kb, uint32_t &kb2) {
    kb = static_cast<uint32_t>(st) * kGuRowBytes;
    const bool half = DT == kBF16 && kb + kGuRowBytes > kbytes;
    kb2 = half ? kb - 64 : kb;
  };
  // weights (and scales) of stage st into the weight slot of stage slot_st
  auto issue_w = [&](int st, int slot_st) {
    const uint32_t sl = lds0 + static_cast<uint32_t>(slot_st % kGuDepth) * C::WS_SLOT;
    uint32_t kb, kb2;
    kbs(st, kb, kb2);
#pragma unroll
    for (int q = 0; q < C::NW; ++q) {
      const uint32_t wu = static_cast<uint32_t>(8 * (q & 3) + (q >= 4 ? inter : 0)) * wstep;
      buf16_to_lds(rW, wl[q & 1] + wu + (whi[q & 1] ? kb2 : kb), lds_ptr(sl + (8 * wave + q) * 1024));
    }
    if constexpr (C::NS) {
      // the next K block's scales too (past the last block: the last
      // block's again, unused)
      buf4_to_lds(rS, 4 * (soff + st), lds_ptr(sl + C::W_BYTES + 256 * wave));
      buf4_to_lds(rS, 4 * (soff + min(st + 1, nstage - 1)), lds_ptr(sl + C::W_BYTES + 1024 + 256 * wave));
    }
  };
  // token rows of stage st into the token slot of stage slot_st: block wave
  // (instructions 0-3), rows 128 + 8 wave .. + 8 of block 4 (instruction 4)
  auto issue_t = [&](int st, int slot_st) {
    const uint32_t tl = lds0 + C::T_BASE + static_cast<uint32_t>(slot_st % kGuTDepth) * C::T_BYTES;
    uint32_t kb, kb2;
    kbs(st, kb, kb2);
#pragma unroll
    for (int q = 0; q < C::NTL; ++q)
      buf16_to_lds(rA, toff[q] + (thi[q] ? kb2 : kb),
                   lds_ptr(tl + (q < 4 ? 4 * wave + q : 16 + wave) * 1024));
  };
  const int last = nstage - 1;
  issue_w(0, 0);
  issue_t(0, 0);
  issue_w(min(1, last), 1);
  wait_vm<C::WAIT>();
#pragma unroll 1
  for (int st = 0; st < nstage; ++st) {
    wait_lgkm<0>();   // work(st - 1)'s reads have landed
    __builtin_amdgcn_sched_barrier(0);
    ring_barrier();
    issue_t(min(st + 1, last), st + 1);
    issue_w(min(st + 2, last), st + 2);
    work(st);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<C::WAIT>();
  }
}

template <int DT>
__global__ __launch_bounds__(kGuThreads, 1) void gu_kernel(GuArgs a) {
  using C = GuCfg<DT>;
  extern __shared__ __align__(1024) uint8_t lds[];
  __shared__ int uoff[1026];             // unit prefix over the E + 1 groups
  __shared__ int wsum[2 * kGuWaves];
  __shared__ float amax_w[kGuWaves][kGuTRows];
  const Dims &d = a.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_id = uniform(tid >> 6);
  const bool loader = wave_id >= kGuWaves;                  // waves 4-7 load, 0-3 multiply
  const int wave = loader ? wave_id - kGuWaves : wave_id;   // the column wave served / itself
  const int G = d.E + (d.Is > 0 ? 1 : 0);
  const int *offsets = a.w.offsets;
  // this block's next ticket from its XCD's unit queue (the prefix's
  // barriers publish the first one)
  __shared__ int tk_next;
  int *const queue = a.w.queue + kQueueStride * (blockIdx.x & 7);
  if (tid == 0) tk_next = atomicAdd(queue, 1);

  // ---- unit prefix: units(g) = ceil(rows_g / 160) * ntile_g ----
  {
    constexpr int PER = (1025 + kGuThreads - 1) / kGuThreads;
    int loc[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid * PER + i;
      int u = 0;
      if (g < G) {
        const int rows = g < d.E ? offsets[g + 1] - offsets[g] : d.m;
        u = (rows + kGuTRows - 1) / kGuTRows * (g < d.E ? a.ntile_r : a.ntile_s);
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
    if (lane == 63) wsum[wave_id] = incl;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int i = 0; i < 2 * kGuWaves; ++i) base += i < wave_id ? wsum[i] : 0;
    int run = base + incl - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid * PER + i;
      if (g <= G) uoff[g] = run;
      run += loc[i];
    }
    __syncthreads();
  }
  const int total = uoff[G];
  const int P = gridDim.x;
  const int xcd = blockIdx.x & 7;
  // Units go to the XCDs in chunks of consecutive units (chunk c to XCD
  // c % 8: the M tiles of an N tile, or the N tiles of a group, run side by
  // side on one L2), and each XCD's blocks take its units in order, one
  // ticket of the XCD's counter each, so a block that finishes early takes
  // the next unit.  A short launch (units for at most kGuFewRounds rounds of
  // the grid) deals chunks of kGuFewChunk units, spreading heavy units over
  // the XCDs, and runs the shared expert's S units (last in group order,
  // the fullest tiles) first, so that lighter routed units come last.  (In
  // long launches shared-first measured neutral to slightly slower.)
  const bool few = total <= kGuFewRounds * P;
  const int chunk = few ? kGuFewChunk : P / 8;
  const int S = d.Is > 0 ? total - uoff[d.E] : 0;
  const bool shared_first = few && S > 0 && S < total;

  const int lg = lane >> 5, lr = lane & 31;   // lane group, row inside a block
  // the lane's read offsets inside a 32-row block, pieces j = 0..3
  uint32_t loff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) loff[j] = lr * kGuRowBytes + ((gu_piece(lg, j) ^ gu_swz(lr)) * 16);
  // a load instruction covers 8 rows: lane l writes piece l % 8 of row l / 8
  const int drow = lane >> 3, dpiece = lane & 7;

#pragma unroll 1
  for (;;) {
    __syncthreads();   // tk_next holds this block's ticket
    const int tk = tk_next;
    const int u = (tk / chunk) * (8 * chunk) + xcd * chunk + tk % chunk;   // increasing in tk
    if (u >= total) break;
    const int uu = shared_first ? (u < S ? total - S + u : u - S) : u;
    // ---- decode the unit (block-uniform) ----
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uoff[mid] <= uu) lo = mid; else hi = mid - 1;
    }
    const int g = uniform(lo);
    const bool shared = g == d.E;
    const int grows = uniform(shared ? d.m : offsets[g + 1] - offsets[g]);
    const int nmt = (grows + kGuTRows - 1) / kGuTRows;
    const int local = uu - uniform(uoff[g]);
    const int ntile = local / nmt;
    // the group's rows split evenly over its nmt M tiles (a 200-row expert
    // runs two tiles of 100 rows, not 160 + 40)
    const int trows = (grows + nmt - 1) / nmt;
    const int row0 = (local - ntile * nmt) * trows;
    const int rows = min(trows, grows - row0);
    const int ntb = (rows + 31) >> 5;                       // token blocks with rows (1..5)
    const int seg0 = shared ? 0 : uniform(offsets[g]);
    const int inter = shared ? d.Is : d.I;
    const int kbytes = d.H * C::ESZ;
    const int nstage = (kbytes + kGuRowBytes - 1) / kGuRowBytes;
    const int c0 = ntile * 128 + 32 * wave;                 // this wave's first h column
    const bool wave_on = c0 < inter;

    const uint8_t *Wb = static_cast<const uint8_t *>(shared ? a.in.sw13 : a.in.w13) +
                        (shared ? 0 : static_cast<size_t>(g) * 2 * d.I * d.H * C::ESZ);
    const uint8_t *Ab = DT == kFP8 ? static_cast<const uint8_t *>(a.w.xq)
                                   : static_cast<const uint8_t *>(a.in.x);

    // ---- accumulators: [weight block: 0 gate, 1 up][token block]; a load
    // wave keeps block 4 in [.][0] ----
    f32x16_t acc[2][kGuMBlocks];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < kGuMBlocks; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][t][i] = 0.f;

    // fp8: acc holds the running sum divided by the current K block's scale
    // s_k (activation row scale x weight block scale): after block k's last
    // MFMA, acc *= s_k / s_(k+1) (each stage's scale area holds both); the
    // MFMAs of block k + 1 then accumulate its products directly, and after
    // the last block acc *= s_last.  That is sum_k s_k P_k with one VALU
    // operation per accumulator and K block (as a separate partial sum would
    // take) but no registers for partials, and each accumulator block's
    // rescale sits between the last MFMAs of the others.
    // One stage: the lane's LDS reads of operand pieces (fp8: its token and
    // weight-block scales after piece 0), issued one piece ahead, the MFMAs of
    // each piece's steps in between; NT token blocks from block T0 (template
    // parameters keep the MFMA sequence free of branches).
    auto stage = [&](int st, auto ntc, auto t0c) {
      constexpr int NT = decltype(ntc)::value;
      constexpr int T0 = decltype(t0c)::value;
      const uint8_t *sw = lds + (st % kGuDepth) * C::WS_SLOT;
      const uint8_t *lw = sw + 64 * wave * kGuRowBytes;
      const uint8_t *lt = lds + C::T_BASE + (st % kGuTDepth) * C::T_BYTES + 32 * kGuRowBytes * T0;
      const bool half = DT == kBF16 && static_cast<uint32_t>(st + 1) * kGuRowBytes > static_cast<uint32_t>(kbytes);
      u32x4_t wr[4][2], tr[4][NT];
      uint32_t sxr[2][NT];     // [this K block, next][token block]
      u32x2_t swr[2];
      auto load_piece = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        wr[j][0] = lds_load<u32x4_t>(lw + loff[j]);
        wr[j][1] = lds_load<u32x4_t>(lw + loff[j] + 32 * kGuRowBytes);
        static_for<0, NT>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          tr[j][t] = lds_load<u32x4_t>(lt + loff[j] + 32 * kGuRowBytes * t);
        });
      };
      // piece 0 first: the scales are needed only after piece 3
      load_piece(std::integral_constant<int, 0>{});
      if constexpr (DT == kFP8) {
        const uint8_t *ls = sw + C::W_BYTES;
        static_for<0, NT>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          sxr[0][t] = lds_load<uint32_t>(ls + 4 * lr + 128 * (T0 + t));
          sxr[1][t] = lds_load<uint32_t>(ls + 4 * lr + 1024 + 128 * (T0 + t));
        });
        swr[0] = lds_load<u32x2_t>(ls + 768);
        swr[1] = lds_load<u32x2_t>(ls + 1024 + 768);
      }
      static_for<0, 4>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        // the reads of piece j + 1 go out before the MFMAs of piece j; the
        // compiler waits for piece j's values just before their first use
        if constexpr (j + 1 < 4) load_piece(std::integral_constant<int, j + 1>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DT == kBF16) {
          // step j: the piece as 8 bf16 values; a half stage runs steps 0, 1
          if (!(half && j >= 2)) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
              for (int b = 0; b < 2; ++b)
                acc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, wr[j][b]), __builtin_bit_cast(bf16x8_t, tr[j][t]),
                    acc[b][t], 0, 0, 0);
          }
        } else {
          // steps 2 j and 2 j + 1: the two 8-byte halves of the piece; the
          // rescale to this K block's scale before its first step
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            bf16x8_t wv[2], tv[NT];
#pragma unroll
            for (int b = 0; b < 2; ++b) wv[b] = e4m3x8_to_bf16(wr[j][b][2 * h], wr[j][b][2 * h + 1]);
#pragma unroll
            for (int t = 0; t < NT; ++t) tv[t] = e4m3x8_to_bf16(tr[j][t][2 * h], tr[j][t][2 * h + 1]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
              for (int b = 0; b < 2; ++b)
                acc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[b], tv[t], acc[b][t], 0, 0, 0);
          }
          if constexpr (j == 3) {
            // the K block is done: to the next block's scale (after the last
            // block, to its own scale: acc becomes the sum itself)
            const bool last = st + 1 == nstage;
            if constexpr (NT >= 2) {
              // ratio = (token ratio) x (weight-block ratio): NT + 2
              // reciprocals instead of 2 NT
              float tq[NT], wq[2];
#pragma unroll
              for (int t = 0; t < NT; ++t)
                tq[t] = __uint_as_float(sxr[0][t]) * __builtin_amdgcn_rcpf(last ? 1.0f : __uint_as_float(sxr[1][t]));
#pragma unroll
              for (int b = 0; b < 2; ++b)
                wq[b] = __uint_as_float(swr[0][b]) * __builtin_amdgcn_rcpf(last ? 1.0f : __uint_as_float(swr[1][b]));
#pragma unroll
              for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[b][t] *= tq[t] * wq[b];
            } else {
#pragma unroll
              for (int b = 0; b < 2; ++b) {
                const float s0 = __uint_as_float(sxr[0][0]) * __uint_as_float(swr[0][b]);
                const float s1 = __uint_as_float(sxr[1][0]) * __uint_as_float(swr[1][b]);
                acc[b][0] *= last ? s0 : s0 * __builtin_amdgcn_rcpf(s1);
              }
            }
          }
        }
      });
    };

    __syncthreads();   // every wave has read its ticket (tk_next is refilled at the unit's end)
    // the ticket after this one, fetched while the unit runs (issued after
    // the unit's own global loads above: loads complete in order)
    int tk_new = 0;
    if (tid == 0) tk_new = atomicAdd(queue, 1);
    // ---- the ring: stage st is multiplied from its slots while stages
    // st + 1 (tokens) and st + 2 (weights) load (gu_load_unit); both sides
    // take exactly nstage barriers per unit ----
    if (loader) {
      // ---- this wave's load sources (32-bit byte offsets; operands < 2 GiB) ----
      // Weight instruction q moves rows 8 (q % 4) + drow of the gate (q < 4)
      // or up block to LDS rows 64 wave + 8 q + drow; token instruction q
      // (0..3) token rows 32 wave + 8 q + drow, instruction 4 rows 128 +
      // 8 wave + drow (past the tile's rows: its last row again).  The lane
      // fetches logical piece dpiece ^ swz(row in its 32-row block): p0 ^ 4
      // (q % 2) for instructions 0-3 and weights, p0 ^ 4 (wave % 2) for
      // instruction 4, p0 = dpiece ^ (drow / 2).
      const int p0 = dpiece ^ (drow >> 1);
      const int wrow0 = wave_on ? c0 + drow : 0;           // out of range: read valid memory, store nothing
      const uint32_t wl[2] = {static_cast<uint32_t>(wrow0) * kbytes + p0 * 16,
                              static_cast<uint32_t>(wrow0) * kbytes + (p0 ^ 4) * 16};
      const bool whi[2] = {p0 >= 4, (p0 ^ 4) >= 4};
      uint32_t toff[kGuTBlocks];
      bool thi[kGuTBlocks];
#pragma unroll
      for (int q = 0; q < kGuTBlocks; ++q) {
        const int row = q < 4 ? 32 * wave + 8 * q + drow : 128 + 8 * wave + drow;
        const int rr = min(row, rows - 1);
        const int tok = shared ? row0 + rr : a.w.sorted_pair[seg0 + row0 + rr] / d.k;
        const int pc = p0 ^ (4 * ((q < 4 ? q : wave) & 1));
        toff[q] = static_cast<uint32_t>(tok) * kbytes + pc * 16;
        thi[q] = pc >= 4;
      }
      // fp8 scales: load waves 4-6 the token rows' (64 each, rows past the
      // tile's rows: its last row again), wave 7 the gate (even lanes) and up
      // (odd lanes) weight-block scales
      const float *sbase = a.w.sx;
      uint32_t soff = 0, sbytes = 4;
      if constexpr (DT == kFP8) {
        const int nkb = d.H / kQBlock;
        if (wave < 3) {
          const int rr = min(64 * wave + lane, rows - 1);
          const int tok = shared ? row0 + rr : a.w.sorted_pair[seg0 + row0 + rr] / d.k;
          soff = static_cast<uint32_t>(tok) * nkb;
          sbytes = static_cast<uint32_t>(d.m) * nkb * 4u;
        } else {
          sbase = shared ? a.in.sw13_scale
                         : a.in.w13_scale + static_cast<size_t>(g) * (2 * d.I / kQBlock) * nkb;
          const int srow = (lane & 1) ? inter / kQBlock + ntile : ntile;
          soff = static_cast<uint32_t>(srow) * nkb;
          sbytes = static_cast<uint32_t>(2 * inter / kQBlock) * nkb * 4u;
        }
      }
      // buffer extents: the group's w13 rows, the m token rows, the scale
      // table this wave reads
      const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(Wb, static_cast<uint32_t>(2 * inter) * kbytes);
      const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(Ab, static_cast<uint32_t>(d.m) * kbytes);
      const __amdgpu_buffer_rsrc_t rS = buffer_rsrc(sbase, sbytes);
      auto load = [&](auto work) {
        gu_load_unit<DT>(rW, rA, rS, wl, whi, toff, thi, wave_on ? static_cast<uint32_t>(kbytes) : 0u,
                         static_cast<uint32_t>(inter), static_cast<uint32_t>(kbytes), soff, nstage, wave,
                         lds_off(lds), work);
      };
      if (ntb == kGuTBlocks && wave_on)
        load([&](int st) {
          stage(st, std::integral_constant<int, 1>{}, std::integral_constant<int, kGuMBlocks>{});
        });
      else
        load([](int) {});
    } else {
      auto run = [&](auto ntc) {
#pragma unroll 1
        for (int st = 0; st < nstage; ++st) {
          // every read of the previous stage has landed before the barrier
          // that hands its slots to the loads
          wait_lgkm<0>();
          __builtin_amdgcn_sched_barrier(0);   // nothing moves across a stage boundary
          ring_barrier();
          if (wave_on) stage(st, ntc, std::integral_constant<int, 0>{});
        }
      };
      switch (ntb) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        default: run(std::integral_constant<int, 4>{}); break;
      }
    }
    // the trailing loads (the last stage again) land before the slots are
    // refilled: the next unit's first barrier waits for every load
    // ---- epilogue: a multiplying wave's block t (t < 4) and a load wave's
    // block 4 (in acc[.][0]); lane holds token row 32 t + lr, h columns
    // c0 + 8 (i / 4) + 4 lg + i % 4 for i = 0..15 ----
    const int nblk = loader ? (ntb == kGuTBlocks ? 1 : 0) : min(ntb, kGuMBlocks);
    auto row_of = [&](int t) { return loader ? 32 * kGuMBlocks + lr : 32 * t + lr; };
    if constexpr (DT == kBF16) {
      uint16_t *h = static_cast<uint16_t *>(shared ? a.w.h_sh : a.w.h);
#pragma unroll
      for (int t = 0; t < kGuMBlocks; ++t) {
        const int rr = row_of(t);
        if (t >= nblk || !wave_on || rr >= rows) continue;
        uint16_t *hr = h + static_cast<size_t>(seg0 + row0 + rr) * inter + c0 + 4 * lg;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w0 = f32_to_bf16(silu(acc[0][t][4 * q]) * acc[1][t][4 * q]) |
                        (static_cast<uint32_t>(f32_to_bf16(silu(acc[0][t][4 * q + 1]) * acc[1][t][4 * q + 1])) << 16);
          uint32_t w1 = f32_to_bf16(silu(acc[0][t][4 * q + 2]) * acc[1][t][4 * q + 2]) |
                        (static_cast<uint32_t>(f32_to_bf16(silu(acc[0][t][4 * q + 3]) * acc[1][t][4 * q + 3])) << 16);
          *reinterpret_cast<u32x2_t *>(hr + 8 * q) = u32x2_t{w0, w1};
        }
      }
    } else {
      // h per row per 128 columns (this unit's): amax across the 4 column
      // waves (rows 0-127: waves 0-3, rows 128-159: waves 4-7)
#pragma unroll
      for (int t = 0; t < kGuMBlocks; ++t) {
        if (t >= nblk) continue;
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float hv = wave_on ? silu(acc[0][t][i]) * acc[1][t][i] : 0.f;
          acc[0][t][i] = hv;
          am = fmaxf(am, fabsf(hv));
        }
        am = fmaxf(am, __shfl_xor(am, 32));
        if (lg == 0) amax_w[wave][row_of(t)] = am;
      }
      __syncthreads();
      uint8_t *h = static_cast<uint8_t *>(shared ? a.w.h_sh : a.w.h);
      float *hs = shared ? a.w.h_sh_scale : a.w.h_scale;
#pragma unroll
      for (int t = 0; t < kGuMBlocks; ++t) {
        const int rr = row_of(t);
        if (t >= nblk || rr >= rows) continue;
        float amax = 0.f;
#pragma unroll
        for (int w = 0; w < kGuWaves; ++w) amax = fmaxf(amax, amax_w[w][rr]);
        const float sc = amax > 0.f ? amax / kE4M3Max : 1.0f;
        const size_t row = static_cast<size_t>(seg0 + row0 + rr);
        if (wave == 0 && lg == 0) hs[row * (inter / kQBlock) + ntile] = sc;
        if (!wave_on) continue;
        uint8_t *hr = h + row * inter + c0 + 4 * lg;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = static_cast<uint32_t>(fp8_pack2(acc[0][t][4 * q] / sc, acc[0][t][4 * q + 1] / sc)) & 0xffffu;
          const uint32_t hi2 = static_cast<uint32_t>(fp8_pack2(acc[0][t][4 * q + 2] / sc, acc[0][t][4 * q + 3] / sc)) & 0xffffu;
          *reinterpret_cast<uint32_t *>(hr + 8 * q) = lo | (hi2 << 16);
        }
      }
    }
    // every wave has read tk_next (the barrier before the ring)
    if (tid == 0) tk_next = tk_new;
  }
}

template <int DT>
hipError_t gu_launch(const Dims &d, const Inputs &in, const Work &w, hipStream_t s) {
  using C = GuCfg<DT>;
  auto kern = gu_kernel<DT>;
  static const KernelSetup su = kernel_setup(reinterpret_cast<const void *>(kern), kGuThreads, C::LDS);
  if (su.err != hipSuccess) return su.err;
  GuArgs ga{d, in, w, (d.I + 127) / 128, (d.Is + 127) / 128};
  const int grid = (device_cus() * su.blocks_per_cu + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGuThreads), C::LDS, s, ga);
  return hipGetLastError();
}

bool gu_supported(const Dims &d) {
  if (d.wdt == kFP8) return d.H % kQBlock == 0 && d.I % kQBlock == 0 && d.Is % kQBlock == 0;
  if (d.wdt == kBF16) return d.H % 32 == 0 && d.I % 32 == 0 && d.Is % 32 == 0;
  return false;
}

}  // namespace

hipError_t launch_gu(const Dims &d, const Inputs &in, const Work &w, hipStream_t s) {
  if (!gu_supported(d)) return hipErrorInvalidValue;
  return d.wdt == kFP8 ? gu_launch<kFP8>(d, in, w, s) : gu_launch<kBF16>(d, in, w, s);
}

}  // namespace moe
