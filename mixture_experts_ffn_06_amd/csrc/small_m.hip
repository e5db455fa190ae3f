// Weight-streaming expert path: stream each selected expert's weights once
// per block of 16 of its rows (bf16 weights up to 256 tokens, MX weights at
// every batch size; an expert of r rows takes ceil(r / 16) blocks).
//
// With at most 16 tokens every expert holds at most 16 rows, so the work is
// a bandwidth-bound GEMV over the selected experts' weights (forward.rs,
// page 1: rows <= 16 take the decode kernels; forward.rs, page 2: the
// single-token arm runs gate/up as one launch and down as another over all
// selected experts; forward_layer.rs, page 4: one dispatch covers all
// selected experts of a decode step).
//
// Work item = (16-row block of a slot, column group): a slot is a routed
// expert with >= 1 row (or the shared expert, whose rows are the m tokens),
// cut into ceil(rows / 16) row blocks (the permute scan leaves each active
// slot's first block in rboff); a column group is NBLK weight blocks of 16
// rows (gate/up: NBLK/2 blocks of w1 and the matching NBLK/2 of w3; down:
// NBLK blocks of w2).  One wave (or KS waves splitting K, their partial sums
// met in LDS) owns an item.
//
// HBM efficiency decides this kernel, and the MFMA operand layout (a load
// instruction touching 16 weight rows, 64 bytes each) streams markedly slower
// than row-contiguous loads.  So the weights move in stages of RUN bytes per
// row: each direct global->LDS load covers 1024/RUN whole rows of RUN
// contiguous bytes, into a per-wave ring of DEPTH stages, and the MFMA B
// fragments are read back from LDS (16-byte pieces XOR-swizzled per row so
// those reads are bank-conflict free).  The item's <= 16 token rows (A, read
// from L2) go straight to registers, one stage ahead like the weights.  The
// grid covers the largest item count the routing allows (the live count is
// only known on the device; waves past it exit at once).
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "launch.h"
#include "lds.h"

namespace moe {

constexpr int kSmBlockWaves = 4;

enum : int { kSmGateUp = 0, kSmDown = 1 };

template <int NBLK, int RUN, int DEPTH>
struct SmCfg {
  static constexpr int NPR = RUN / 16;            // 16-byte pieces per row per stage
  static constexpr int RPI = 64 / NPR;            // rows per load instruction
  static constexpr int NI = NBLK * 16 / RPI;      // load instructions per stage
  static constexpr int SSTEPS = RUN / 64;         // 32-wide bf16 MFMA steps per stage
  static constexpr int STAGE = NBLK * 16 * RUN;   // bytes per stage
  static constexpr int WAVE_LDS = DEPTH * STAGE;
  static constexpr int LDS = kSmBlockWaves * WAVE_LDS;
  static_assert(RUN == 64 || RUN == 128 || RUN == 256, "swizzle covers 64- to 256-byte runs");
  static_assert(DEPTH == 2, "one stage in flight");
  static_assert(NI + SSTEPS < 64, "vmcnt range");
  static_assert(WAVE_LDS >= NBLK * kWave * 16, "partial sums fit the ring");
};

// Position of logical 16-byte piece p of row r inside the row's run: the
// 16 rows of a block read the same logical piece in one MFMA step, and the
// XOR puts them in 16 distinct 16-byte bank groups of each 256-byte window.
template <int RUN>
__device__ __forceinline__ int sm_swz(int p, int r) {
  return p ^ ((r / (256 / RUN)) % (RUN / 16));
}

// An item: a 16-row block of a slot and a column group.  Routed items come
// first: row block sr of all the active slots' blocks (the permute scan
// leaves each active slot's first block in rboff), column groups fastest,
// the slot found as the last one whose first block is <= sr; then the
// shared expert's ceil(m / 16) row blocks of the tokens.  Items past those
// have no rows (rows = 0).
struct SmItem {
  int e, seg0, rows, inter, cg;
  bool shared;
};
__device__ __forceinline__ SmItem sm_item(const Dims &d, const Work &w, int item, int ipr, int ips) {
  SmItem it{0, 0, 0, 0, 0, false};
  const int na = uniform(*w.nactive);
  const int nrb_r = uniform(w.rboff[na]);
  const int nrb_s = (d.m + 15) >> 4;
  if (item < nrb_r * ipr) {
    const int sr = item / ipr;
    it.cg = item - sr * ipr;
    int lo = 0, hi = na - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uniform(w.rboff[mid]) <= sr) lo = mid;
      else hi = mid - 1;
    }
    const int rb = sr - uniform(w.rboff[lo]);
    it.e = uniform(w.active[lo]);
    const int s0 = uniform(w.offsets[it.e]);
    const int r = uniform(w.offsets[it.e + 1]) - s0;
    it.seg0 = s0 + 16 * rb;
    it.rows = min(16, r - 16 * rb);
    it.inter = d.I;
  } else if (item < nrb_r * ipr + ips * nrb_s) {
    const int t = item - nrb_r * ipr;
    const int rb = t / ips;
    it.cg = t - rb * ips;
    it.shared = true;
    it.e = d.E;
    it.seg0 = 16 * rb;
    it.rows = min(16, d.m - 16 * rb);   // the shared expert's rows are the tokens
    it.inter = d.Is;
  }
  return it;
}

template <int MODE, int NBLK, int RUN, int DEPTH>
__global__ __launch_bounds__(kSmBlockWaves * kWave) void sm_kernel(Dims d, Inputs in, Work w, int ks) {
  using C = SmCfg<NBLK, RUN, DEPTH>;
  constexpr int CW = MODE == kSmGateUp ? 16 * NBLK / 2 : 16 * NBLK;   // output columns per item
  extern __shared__ __align__(1024) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  uint8_t *ring = lds + wave * C::WAVE_LDS;
  const int item = uniform(blockIdx.x * (kSmBlockWaves / ks) + wave / ks);
  const int kp = uniform(wave % ks);

  // ---- the item: slot, block of 16 rows and column group ----
  const int ncol_r = MODE == kSmGateUp ? d.I : d.H;
  const int ipr = (ncol_r + CW - 1) / CW;                  // items per routed slot
  const int ips = d.Is > 0 ? ((MODE == kSmGateUp ? d.Is : d.H) + CW - 1) / CW : 0;

  f32x4_t acc[NBLK];
#pragma unroll
  for (int j = 0; j < NBLK; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const SmItem it = sm_item(d, w, item, ipr, ips);
  const bool shared = it.shared;
  const int e = it.e, seg0 = uniform(it.seg0), rows = uniform(it.rows), inter = it.inter, cg = it.cg;
  int c0 = 0, ncol = 0;
  const bool live = rows > 0;
  if (live) {
    c0 = cg * CW;
    ncol = MODE == kSmGateUp ? inter : d.H;
    const int K = MODE == kSmGateUp ? d.H : inter;
    const int kbytes = K * 2;

    // Operand bases (wave-uniform) and 32-bit byte offsets from them (the
    // plan keeps every operand below 2 GiB).
    const int r = lane & 15;
    const int ar = min(r, rows - 1);   // rows past the slot's end repeat its last row
    const uint8_t *Ab, *Wb;
    uint32_t aoff;
    if (MODE == kSmGateUp) {
      const int tok = shared ? seg0 + ar : w.sorted_pair[seg0 + ar] / d.k;
      Ab = static_cast<const uint8_t *>(in.x);
      aoff = static_cast<uint32_t>(tok) * kbytes;
      Wb = shared ? static_cast<const uint8_t *>(in.sw13)
                  : static_cast<const uint8_t *>(in.w13) + static_cast<size_t>(e) * 2 * d.I * d.H * 2;
    } else {
      Ab = static_cast<const uint8_t *>(shared ? w.h_sh : w.h);
      aoff = static_cast<uint32_t>(seg0 + ar) * kbytes;
      Wb = shared ? static_cast<const uint8_t *>(in.sw2)
                  : static_cast<const uint8_t *>(in.w2) + static_cast<size_t>(e) * d.H * d.I * 2;
    }
    aoff += (lane >> 4) * 16;   // the lane's 8 K elements of each step
    // First weight row of block j (blocks past the last column read row 0
    // and store nothing).
    auto wrow = [&](int j) -> int {
      if (MODE == kSmGateUp) {
        const int c = c0 + 16 * (j % (NBLK / 2));
        return c < ncol ? (j < NBLK / 2 ? c : inter + c) : 0;
      }
      const int c = c0 + 16 * j;
      return c < ncol ? c : 0;
    };
    // Load instruction q covers block q / (16/RPI), rows (q % (16/RPI)) * RPI
    // + lane / NPR; the lane fetches logical piece sm_swz(lane % NPR, row) of
    // its row, so LDS position lane % NPR holds that piece.
    uint32_t qoff[C::NI];
#pragma unroll
    for (int q = 0; q < C::NI; ++q) {
      const int j = q / (16 / C::RPI);
      const int row = (q % (16 / C::RPI)) * C::RPI + lane / C::NPR;
      qoff[q] = static_cast<uint32_t>(wrow(j) + row) * kbytes + sm_swz<RUN>(lane % C::NPR, row) * 16;
    }

    // ---- K range of this wave, in stages of RUN bytes per row ----
    const int nst_all = kbytes / RUN;
    const int st0 = uniform(nst_all * kp / ks), st1 = uniform(nst_all * (kp + 1) / ks);
    uint4 aA[C::SSTEPS], aB[C::SSTEPS];
    // Loads of stage st into ring slot sl (K bytes are a multiple of RUN:
    // every stage is whole).
    auto issue = [&](int st, int sl, uint4 (&A)[C::SSTEPS]) {
      const uint32_t kb = static_cast<uint32_t>(st) * RUN;
      uint8_t *slot = ring + sl * C::STAGE;
#pragma unroll
      for (int q = 0; q < C::NI; ++q) dma16_to_lds(Wb + (qoff[q] + kb), slot + q * 1024);
#pragma unroll
      for (int i = 0; i < C::SSTEPS; ++i) A[i] = *reinterpret_cast<const uint4 *>(Ab + (aoff + kb) + i * 64);
    };
    // lane reads row r, logical piece 4 i + lane / 16 of step i
    const int g = lane >> 4;
    auto compute = [&](int st, int sl, const uint4 (&A)[C::SSTEPS]) {
      const uint8_t *slot = ring + sl * C::STAGE;
#pragma unroll
      for (int i = 0; i < C::SSTEPS; ++i) {
        const uint32_t rb = lds_off(slot + r * RUN + sm_swz<RUN>(4 * i + g, r) * 16);
        u32x4_t b[NBLK];
        if constexpr (NBLK == 2) {
          lds_read2<0, 16 * RUN>(rb, rb, b[0], b[1]);
        } else {
          static_assert(NBLK == 4, "2 or 4 blocks");
          lds_read4<0, 16 * RUN, 32 * RUN, 48 * RUN>(rb, rb, rb, rb, b[0], b[1], b[2], b[3]);
        }
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, A[i]);
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, b[j]), acc[j], 0, 0, 0);
      }
    };
    // Ring of two slots, walked two stages per iteration so that each
    // register buffer has a fixed slot; every wait counts exactly the LPS
    // operations of the stage issued after the one it waits for.  The
    // issue after the last stage repeats it into the idle slot (never read).
    constexpr int LPS = C::NI + C::SSTEPS;   // vector-memory ops per stage
    const int n = st1 - st0;
    if (n > 0) {
      issue(st0, 0, aA);
      int st = st0;
      for (int p = 0; p < n / 2; ++p, st += 2) {
        issue(st + 1, 1, aB);
        wait_vm<LPS>();
        compute(st, 0, aA);
        issue(min(st + 2, st1 - 1), 0, aA);
        wait_vm<LPS>();
        compute(st + 1, 1, aB);
      }
      wait_vm<0>();
      if (n & 1) compute(st, 0, aA);
    }
  }

  // ---- partial sums of the KS waves of an item meet in LDS (each wave's
  // own ring: all of its loads have landed) ----
  if (ks > 1) {
    f32x4_t *part = reinterpret_cast<f32x4_t *>(ring);
#pragma unroll
    for (int j = 0; j < NBLK; ++j) part[j * kWave + lane] = acc[j];
    __syncthreads();
    if (kp != 0) return;
    for (int q = 1; q < ks; ++q) {
      const f32x4_t *other = reinterpret_cast<const f32x4_t *>(lds + (wave + q) * C::WAVE_LDS);
#pragma unroll
      for (int j = 0; j < NBLK; ++j) acc[j] += other[j * kWave + lane];
    }
  }
  if (!live) return;

  // ---- epilogue: lane holds rows 4*(lane/16) + i, column lane % 16 ----
  const int cl = lane & 15;
  if (MODE == kSmGateUp) {
    uint16_t *h = static_cast<uint16_t *>(shared ? w.h_sh : w.h) + static_cast<size_t>(seg0) * inter;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 4) * 4 + i;
      if (row < rows) {
#pragma unroll
        for (int j = 0; j < NBLK / 2; ++j)
          if (c0 + 16 * j < ncol)
            h[static_cast<size_t>(row) * inter + c0 + 16 * j + cl] =
                f32_to_bf16(silu(acc[j][i]) * acc[j + NBLK / 2][i]);
      }
    }
  } else {
    float *y = (shared ? w.y_sh : w.y) + static_cast<size_t>(seg0) * d.H;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 4) * 4 + i;
      if (row < rows) {
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
          if (c0 + 16 * j < ncol)
            y[static_cast<size_t>(row) * d.H + c0 + 16 * j + cl] = acc[j][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MX weights (OCP Microscaling: FP4 E2M1 or FP8 E4M3 elements, one E8M0
// scale per 32 elements of a row along K; tokens and h stay bf16).  Same
// items, K split and two-slot ring as sm_kernel, with NB = 2 or 4 blocks of
// 16 weight rows per item; a stage is 128 bytes of each of the item's 16 NB
// weight rows (256 K elements of FP4, 128 of FP8; 2 NB 1 KB direct loads of 8
// whole rows each, pieces swizzled per row) plus the rows' scale bytes for
// those K elements (8 or 4 per row, 4-byte direct loads).  In MFMA step i of a stage, lane group g = lane / 16
// takes K elements [32 i + 8 g, 32 i + 8 g + 8): each token-row load then
// covers 64 contiguous bytes of every token (the four groups side by side,
// as in the bf16 kernel), the lane's weight bytes for the step are 4-byte
// word g of 16-byte piece i of its row (FP4) or the 8 bytes at 8 (g % 2) in
// piece 2 i + g / 2 (FP8), read from LDS, and all 32 K elements of a step
// share one E8M0 scale byte of the row (any split of K over the lanes gives
// the same product when A and B share it).  Giving each lane 32 contiguous
// weight bytes instead made every token-row load touch 64 separate cache
// lines, which cost about 15 % of the kernel time.
// The weights become bf16 in registers by gfx950's scaled conversions, which
// multiply by 2 to the power of the scale operand's exponent: with the scale
// 2^(e - 127) built from the E8M0 byte that is exact.  The MFMA is the bf16
// 16x16x32 of the bf16 path.
constexpr int kMxRun = 128;   // weight bytes per row per stage

// NB blocks of 16 weight rows per item (gate/up: NB/2 of w1 and the matching
// NB/2 of w3).
template <int FMT, int NB>
struct MxCfg {
  static constexpr bool F4 = FMT == kMXFP4;
  static constexpr int KPS = F4 ? 2 * kMxRun : kMxRun;   // K elements per stage
  static constexpr int SSTEPS = KPS / 32;                 // MFMA steps per stage
  static constexpr int SPR = KPS / 32;                    // scale bytes per row per stage
  static constexpr int ROWS = 16 * NB;                    // weight rows per item
  static constexpr int WBYTES = ROWS * kMxRun;            // weight bytes per stage
  static constexpr int SBYTES = ROWS * 8;                 // scale area per stage (FP8 fills half)
  static constexpr int STAGE = WBYTES + SBYTES;
  static constexpr int WAVE_LDS = 2 * STAGE;
  static constexpr int LDS = kSmBlockWaves * WAVE_LDS;
  static constexpr int NSD = F4 ? NB / 2 : 1;             // 4-byte scale loads per lane per stage
  static_assert(FMT == kMXFP4 || FMT == kMXFP8, "MX formats");
  static_assert(NB == 2 || NB == 4, "items of 2 or 4 blocks");
  static_assert(WAVE_LDS >= NB * kWave * 16, "partial sums fit the ring");
};

// One stage's weight and scale reads of an MX item from its ring slot, all
// issued and then waited for in one statement (NB blocks of 16 rows, block j
// 16 * kMxRun bytes after block j - 1; its scale bytes 16 * 8 (FP4) or
// 16 * 4 (FP8) bytes after).  a[i]: the lane's address of step i's weight
// bytes in block 0; as: of its scale bytes in block 0.
#define MX_RW(OP, J, I) OP " %[w" #J #I "], %[a" #I "] offset:%[o" #J "]\n\t"
#define MX_RS(OP, J) OP " %[q" #J "], %[as] offset:%[s" #J "]\n\t"
#define MX_F4_BLK(J)                                                                                   \
  MX_RW("ds_read_b32", J, 0) MX_RW("ds_read_b32", J, 1) MX_RW("ds_read_b32", J, 2)                     \
  MX_RW("ds_read_b32", J, 3) MX_RW("ds_read_b32", J, 4) MX_RW("ds_read_b32", J, 5)                     \
  MX_RW("ds_read_b32", J, 6) MX_RW("ds_read_b32", J, 7) MX_RS("ds_read_b64", J)
#define MX_F8_BLK(J)                                                                                   \
  MX_RW("ds_read_b64", J, 0) MX_RW("ds_read_b64", J, 1) MX_RW("ds_read_b64", J, 2)                     \
  MX_RW("ds_read_b64", J, 3) MX_RS("ds_read_b32", J)
#define MX_F4_OUT(J)                                                                                   \
  [w##J##0] "=&v"(wv[J][0]), [w##J##1] "=&v"(wv[J][1]), [w##J##2] "=&v"(wv[J][2]),                     \
  [w##J##3] "=&v"(wv[J][3]), [w##J##4] "=&v"(wv[J][4]), [w##J##5] "=&v"(wv[J][5]),                     \
  [w##J##6] "=&v"(wv[J][6]), [w##J##7] "=&v"(wv[J][7]), [q##J] "=&v"(q[J])
#define MX_F8_OUT(J)                                                                                   \
  [w##J##0] "=&v"(wv[J][0]), [w##J##1] "=&v"(wv[J][1]), [w##J##2] "=&v"(wv[J][2]),                     \
  [w##J##3] "=&v"(wv[J][3]), [q##J] "=&v"(q[J])
#define MX_A8 [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), \
              [a4] "v"(a[4]), [a5] "v"(a[5]), [a6] "v"(a[6]), [a7] "v"(a[7])
#define MX_A4 [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3])
#define MX_OFFS(SB) [o0] "i"(0), [o1] "i"(16 * kMxRun), [o2] "i"(32 * kMxRun), [o3] "i"(48 * kMxRun), \
                    [s0] "i"(0), [s1] "i"(16 * (SB)), [s2] "i"(32 * (SB)), [s3] "i"(48 * (SB))

__device__ __forceinline__ void mx_read(const uint32_t (&a)[8], uint32_t as, uint32_t (&wv)[2][8], u32x2_t (&q)[2]) {
  asm volatile(MX_F4_BLK(0) MX_F4_BLK(1) "s_waitcnt lgkmcnt(0)"
               : MX_F4_OUT(0), MX_F4_OUT(1)
               : MX_A8, [as] "v"(as), MX_OFFS(8)
               : "memory");
}
__device__ __forceinline__ void mx_read(const uint32_t (&a)[8], uint32_t as, uint32_t (&wv)[4][8], u32x2_t (&q)[4]) {
  asm volatile(MX_F4_BLK(0) MX_F4_BLK(1) MX_F4_BLK(2) MX_F4_BLK(3) "s_waitcnt lgkmcnt(0)"
               : MX_F4_OUT(0), MX_F4_OUT(1), MX_F4_OUT(2), MX_F4_OUT(3)
               : MX_A8, [as] "v"(as), MX_OFFS(8)
               : "memory");
}
__device__ __forceinline__ void mx_read(const uint32_t (&a)[4], uint32_t as, u32x2_t (&wv)[2][4], uint32_t (&q)[2]) {
  asm volatile(MX_F8_BLK(0) MX_F8_BLK(1) "s_waitcnt lgkmcnt(0)"
               : MX_F8_OUT(0), MX_F8_OUT(1)
               : MX_A4, [as] "v"(as), MX_OFFS(4)
               : "memory");
}
__device__ __forceinline__ void mx_read(const uint32_t (&a)[4], uint32_t as, u32x2_t (&wv)[4][4], uint32_t (&q)[4]) {
  asm volatile(MX_F8_BLK(0) MX_F8_BLK(1) MX_F8_BLK(2) MX_F8_BLK(3) "s_waitcnt lgkmcnt(0)"
               : MX_F8_OUT(0), MX_F8_OUT(1), MX_F8_OUT(2), MX_F8_OUT(3)
               : MX_A4, [as] "v"(as), MX_OFFS(4)
               : "memory");
}
#undef MX_RW
#undef MX_RS
#undef MX_F4_BLK
#undef MX_F8_BLK
#undef MX_F4_OUT
#undef MX_F8_OUT
#undef MX_A8
#undef MX_A4
#undef MX_OFFS

// Eight e2m1 codes (one 32-bit word, the even element in the low nibble of
// each byte) times 2^(e - 127), as bf16.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t word, uint32_t e) {
  const float sc = __uint_as_float(e << 23);
  const bf16x2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0);
  const bf16x2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1);
  const bf16x2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2);
  const bf16x2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3);
  return bf16x8_t{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
}

// Eight e4m3 codes (two 32-bit words, lowest byte first) times 2^(e - 127),
// as bf16.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi, uint32_t e) {
  const float sc = __uint_as_float(e << 23);
  const bf16x2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false);
  const bf16x2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true);
  const bf16x2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false);
  const bf16x2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true);
  return bf16x8_t{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
}

// Waves per SIMD that the LDS allows (NB = 2: four blocks per CU, NB = 4:
// two); without the bound the NB = 2 FP4 kernels took 163 registers (three
// waves).
template <int MODE, int FMT, int NB>
__global__ __launch_bounds__(kSmBlockWaves * kWave, NB == 2 ? 4 : 2) void sm_mx_kernel(Dims d, Inputs in, Work w, int ks) {
  using C = MxCfg<FMT, NB>;
  constexpr int CW = MODE == kSmGateUp ? 8 * NB : 16 * NB;   // output columns per item
  extern __shared__ __align__(1024) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  uint8_t *ring = lds + wave * C::WAVE_LDS;
  const int item = uniform(blockIdx.x * (kSmBlockWaves / ks) + wave / ks);
  const int kp = uniform(wave % ks);

  // ---- the item: slot, block of 16 rows and column group ----
  const int ncol_r = MODE == kSmGateUp ? d.I : d.H;
  const int ipr = (ncol_r + CW - 1) / CW;
  const int ips = d.Is > 0 ? ((MODE == kSmGateUp ? d.Is : d.H) + CW - 1) / CW : 0;

  f32x4_t acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const SmItem it = sm_item(d, w, item, ipr, ips);
  const bool shared = it.shared;
  const int e = it.e, seg0 = uniform(it.seg0), rows = uniform(it.rows), inter = it.inter, cg = it.cg;
  int c0 = 0, ncol = 0;
  const bool live = rows > 0;
  if (live) {
    c0 = cg * CW;
    ncol = MODE == kSmGateUp ? inter : d.H;
    const int K = MODE == kSmGateUp ? d.H : inter;
    // bytes per token / weight / scale row
    const int abytes = K * 2, wbytes = C::F4 ? K / 2 : K, sbytes = K / 32;

    const int r = lane & 15, g = lane >> 4;
    const int ar = min(r, rows - 1);   // rows past the slot's end repeat its last row
    const uint8_t *Ab, *Wb, *Sb;
    uint32_t aoff;
    const uint8_t *s13 = reinterpret_cast<const uint8_t *>(shared ? in.sw13_scale : in.w13_scale);
    const uint8_t *s2 = reinterpret_cast<const uint8_t *>(shared ? in.sw2_scale : in.w2_scale);
    if (MODE == kSmGateUp) {
      const int tok = shared ? seg0 + ar : w.sorted_pair[seg0 + ar] / d.k;
      Ab = static_cast<const uint8_t *>(in.x);
      aoff = static_cast<uint32_t>(tok) * abytes;
      const size_t eo = shared ? 0 : static_cast<size_t>(e) * 2 * d.I;   // first weight row
      Wb = static_cast<const uint8_t *>(shared ? in.sw13 : in.w13) + eo * (C::F4 ? d.H / 2 : d.H);
      Sb = s13 + eo * (d.H / 32);
    } else {
      Ab = static_cast<const uint8_t *>(shared ? w.h_sh : w.h);
      aoff = static_cast<uint32_t>(seg0 + ar) * abytes;
      const size_t eo = shared ? 0 : static_cast<size_t>(e) * d.H;
      Wb = static_cast<const uint8_t *>(shared ? in.sw2 : in.w2) + eo * (C::F4 ? d.I / 2 : d.I);
      Sb = s2 + eo * (d.I / 32);
    }
    aoff += g * 16;   // the lane group's 8 K elements of each step, in bf16
    // First weight row of block j (blocks past the last column read row 0
    // and store nothing).
    auto wrow = [&](int j) -> int {
      if (MODE == kSmGateUp) {
        const int c = c0 + 16 * (j % (NB / 2));
        return c < ncol ? (j < NB / 2 ? c : inter + c) : 0;
      }
      const int c = c0 + 16 * j;
      return c < ncol ? c : 0;
    };
    // Direct load q covers item rows 8 q .. 8 q + 7 (block q / 2); the lane
    // fetches logical piece sm_swz(lane % 8, row) of its row.
    uint32_t qoff[2 * NB];
#pragma unroll
    for (int q = 0; q < 2 * NB; ++q) {
      const int row = (q % 2) * 8 + lane / 8;
      qoff[q] = static_cast<uint32_t>(wrow(q / 2) + row) * wbytes + sm_swz<kMxRun>(lane % 8, row) * 16;
    }
    // scales, item row s at byte SPR s of the scale area: FP4 load q has lane
    // l fetch 4 of the 8 bytes of item row 32 q + l / 2; FP8 lane l the 4
    // bytes of item row l % ROWS (with 32 rows, lanes 32-63 repeat rows 0-31
    // into the unused upper half of the area)
    uint32_t soff[C::NSD];
#pragma unroll
    for (int q = 0; q < C::NSD; ++q) {
      const int srow = C::F4 ? 32 * q + (lane >> 1) : lane % C::ROWS;
      soff[q] = static_cast<uint32_t>(wrow(srow / 16) + srow % 16) * sbytes + (C::F4 ? (lane & 1) * 4 : 0);
    }

    const int nst_all = K / C::KPS;
    const int st0 = uniform(nst_all * kp / ks), st1 = uniform(nst_all * (kp + 1) / ks);
    uint4 aA[C::SSTEPS], aB[C::SSTEPS];
    auto issue = [&](int st, int sl, uint4 (&A)[C::SSTEPS]) {
      uint8_t *slot = ring + sl * C::STAGE;
      const uint32_t kw = static_cast<uint32_t>(st) * kMxRun;
#pragma unroll
      for (int q = 0; q < 2 * NB; ++q) dma16_to_lds(Wb + (qoff[q] + kw), slot + q * 1024);
#pragma unroll
      for (int q = 0; q < C::NSD; ++q)
        dma4_to_lds(Sb + (soff[q] + static_cast<uint32_t>(st) * C::SPR), slot + C::WBYTES + q * 256);
      const uint32_t ka = static_cast<uint32_t>(st) * C::KPS * 2;
#pragma unroll
      for (int i = 0; i < C::SSTEPS; ++i) A[i] = *reinterpret_cast<const uint4 *>(Ab + (aoff + ka) + i * 64);
    };
    // the lane's weight bytes of step i: FP4 word g of logical piece i of row
    // r, FP8 the 8 bytes at 8 (g % 2) of logical piece 2 i + g / 2 (block j
    // is 16 j rows further on); its scale bytes: the row's SPR bytes
    uint32_t boff[C::SSTEPS];
#pragma unroll
    for (int i = 0; i < C::SSTEPS; ++i)
      boff[i] = C::F4 ? static_cast<uint32_t>(r * kMxRun + sm_swz<kMxRun>(i, r) * 16 + 4 * g)
                      : static_cast<uint32_t>(r * kMxRun + sm_swz<kMxRun>(2 * i + g / 2, r) * 16 + 8 * (g % 2));
    const uint32_t srd = static_cast<uint32_t>(C::WBYTES + r * C::SPR);
    auto compute = [&](int sl, const uint4 (&A)[C::SSTEPS]) {
      const uint32_t base = lds_off(ring + sl * C::STAGE);
      if constexpr (C::F4) {
        uint32_t wv[NB][8];
        u32x2_t q[NB];
        uint32_t ad[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ad[i] = base + boff[i];
        mx_read(ad, base + srd, wv, q);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, A[i]);
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            // scale byte i of the row's 8 covers step i
            const uint32_t e = ((i < 4 ? q[j].x : q[j].y) >> (8 * (i % 4))) & 0xffu;
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_to_bf16(wv[j][i], e), acc[j], 0, 0, 0);
          }
        }
      } else {
        u32x2_t wv[NB][4];
        uint32_t q[NB];
        uint32_t ad[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ad[i] = base + boff[i];
        mx_read(ad, base + srd, wv, q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, A[i]);
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            // scale byte i of the row's 4 covers step i
            const uint32_t e = (q[j] >> (8 * i)) & 0xffu;
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp8x8_to_bf16(wv[j][i].x, wv[j][i].y, e), acc[j], 0, 0, 0);
          }
        }
      }
    };
    constexpr int LPS = 2 * NB + C::NSD + C::SSTEPS;   // vector-memory ops per stage
    const int n = st1 - st0;
    if (n > 0) {
      issue(st0, 0, aA);
      int st = st0;
      for (int p = 0; p < n / 2; ++p, st += 2) {
        issue(st + 1, 1, aB);
        wait_vm<LPS>();
        compute(0, aA);
        issue(min(st + 2, st1 - 1), 0, aA);
        wait_vm<LPS>();
        compute(1, aB);
      }
      wait_vm<0>();
      if (n & 1) compute(0, aA);
    }
  }

  // ---- partial sums of the KS waves of an item meet in LDS ----
  if (ks > 1) {
    f32x4_t *part = reinterpret_cast<f32x4_t *>(ring);
#pragma unroll
    for (int j = 0; j < NB; ++j) part[j * kWave + lane] = acc[j];
    __syncthreads();
    if (kp != 0) return;
    for (int q = 1; q < ks; ++q) {
      const f32x4_t *other = reinterpret_cast<const f32x4_t *>(lds + (wave + q) * C::WAVE_LDS);
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] += other[j * kWave + lane];
    }
  }
  if (!live) return;

  // ---- epilogue: lane holds rows 4*(lane/16) + i, column lane % 16 ----
  const int cl = lane & 15;
  if (MODE == kSmGateUp) {
    uint16_t *h = static_cast<uint16_t *>(shared ? w.h_sh : w.h) + static_cast<size_t>(seg0) * inter;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 4) * 4 + i;
      if (row < rows) {
#pragma unroll
        for (int j = 0; j < NB / 2; ++j)
          if (c0 + 16 * j < ncol)
            h[static_cast<size_t>(row) * inter + c0 + 16 * j + cl] =
                f32_to_bf16(silu(acc[j][i]) * acc[j + NB / 2][i]);
      }
    }
  } else {
    float *y = (shared ? w.y_sh : w.y) + static_cast<size_t>(seg0) * d.H;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 4) * 4 + i;
      if (row < rows) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
          if (c0 + 16 * j < ncol)
            y[static_cast<size_t>(row) * d.H + c0 + 16 * j + cl] = acc[j][i];
      }
    }
  }
}

// The largest item count the routing allows (the row blocks are only known
// on the device): the routed slots hold at most sum ceil(r_e / 16) <=
// (te + 15 slots) / 16 blocks (and at most ceil(m / 16) each), the shared
// expert ceil(m / 16).
static long sm_items_max(const Dims &d, int slots, int ipr, int ips) {
  const long nrb = (d.m + 15) / 16;
  const long rb_routed = std::min(static_cast<long>(slots) * nrb, (static_cast<long>(d.te) + 15L * slots) / 16);
  return rb_routed * ipr + static_cast<long>(ips) * nrb;
}

// Grid for the largest possible item count (items past the actual count exit
// at once).  KS, the waves per item
// (each streams 1/KS of K, partial sums meet in LDS), is at least 2 whenever
// every wave keeps three stages, then the largest of 2, 4 that keeps the wave
// tasks within three rounds of what fits at once and leaves every wave at
// least three stages: smaller tasks shorten the tail of a launch that would
// otherwise leave CUs idle (m = 4 gate/up: 46 -> 37 us; m = 16 gate/up with
// 2 rather than 1: 96 -> 84 us), while tasks of one or two stages cost more
// than they balance.
static int sm_pick_ks(long items, long cap, int nst) {
  int ks = nst >= 6 ? 2 : 1;
  while (ks < kSmBlockWaves && items * ks * 2 <= 3 * cap && nst / (ks * 2) >= 3) ks *= 2;
  return ks;
}
template <int MODE, int NBLK, int RUN, int DEPTH>
static hipError_t sm_launch(const Dims &d, const Inputs &in, const Work &w, hipStream_t s) {
  using C = SmCfg<NBLK, RUN, DEPTH>;
  constexpr int CW = MODE == kSmGateUp ? 16 * NBLK / 2 : 16 * NBLK;
  auto kern = sm_kernel<MODE, NBLK, RUN, DEPTH>;
  static const KernelSetup su = kernel_setup(reinterpret_cast<const void *>(kern), kSmBlockWaves * kWave, C::LDS);
  if (su.err != hipSuccess) return su.err;
  const int blocks_per_cu = su.blocks_per_cu;
  const int slots = d.te < d.E ? d.te : d.E;
  const int ncol_r = MODE == kSmGateUp ? d.I : d.H;
  const int ipr = (ncol_r + CW - 1) / CW;
  const int ips = d.Is > 0 ? ((MODE == kSmGateUp ? d.Is : d.H) + CW - 1) / CW : 0;
  const long items = sm_items_max(d, slots, ipr, ips);
  const long cap = static_cast<long>(device_cus()) * blocks_per_cu * kSmBlockWaves;
  // K stages of the shortest item (the shared expert's down K is I_s)
  const int kmin = MODE == kSmGateUp ? d.H : (d.Is > 0 && d.Is < d.I ? d.Is : d.I);
  const int nst = kmin * 2 / RUN;
  const int ks = sm_pick_ks(items, cap, nst);
  const long per_block = kSmBlockWaves / ks;
  const long grid = (items + per_block - 1) / per_block;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kSmBlockWaves * kWave), C::LDS, s,
                     d, in, w, ks);
  return hipGetLastError();
}

// Blocks of 16 weight rows per MX item.  Four halve the token-row loads per
// weight byte, which helps where they are heaviest, the MXFP4 gate/up (8 KB
// of token rows per 4 KB weight stage with two blocks; 16 tokens: 33.1-33.4
// against 34.6-35.6 us); with two blocks per CU instead of four the MXFP4
// down (19.3-19.7 -> 20.8-21.1 us) and both MXFP8 kernels were slower.
template <int MODE, int FMT>
constexpr int mx_blocks() { return MODE == kSmGateUp && FMT == kMXFP4 ? 4 : 2; }

// MX launch: the item count and grid of sm_launch; the K split of sm_launch
// except for short gate/up items.
template <int MODE, int FMT, int NB>
static hipError_t sm_mx_launch(const Dims &d, const Inputs &in, const Work &w, hipStream_t s) {
  using C = MxCfg<FMT, NB>;
  constexpr int CW = MODE == kSmGateUp ? 8 * NB : 16 * NB;
  auto kern = sm_mx_kernel<MODE, FMT, NB>;
  static const KernelSetup su = kernel_setup(reinterpret_cast<const void *>(kern), kSmBlockWaves * kWave, C::LDS);
  if (su.err != hipSuccess) return su.err;
  const int blocks_per_cu = su.blocks_per_cu;
  const int slots = d.te < d.E ? d.te : d.E;
  const int ncol_r = MODE == kSmGateUp ? d.I : d.H;
  const int ipr = (ncol_r + CW - 1) / CW;
  const int ips = d.Is > 0 ? ((MODE == kSmGateUp ? d.Is : d.H) + CW - 1) / CW : 0;
  const long items = sm_items_max(d, slots, ipr, ips);
  const long cap = static_cast<long>(device_cus()) * blocks_per_cu * kSmBlockWaves;
  const int kmin = MODE == kSmGateUp ? d.H : (d.Is > 0 && d.Is < d.I ? d.Is : d.I);
  const int nst = kmin / C::KPS;
  // gate/up items of at most 8 stages (MXFP4 at K = 2048) keep one wave:
  // splitting them left each wave four stages (34.6-34.9 against 35.1-35.6 us
  // at 16 tokens)
  const int ks = MODE == kSmGateUp && nst <= 8 ? 1 : sm_pick_ks(items, cap, nst);
  const long per_block = kSmBlockWaves / ks;
  const long grid = (items + per_block - 1) / per_block;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kSmBlockWaves * kWave), C::LDS, s,
                     d, in, w, ks);
  return hipGetLastError();
}

// H, I multiples of 32 and m <= 16 are checked by the caller (MX formats: H,
// I and I_s multiples of one stage's K, 256 for FP4 and 128 for FP8).  A stage moves
// RUN contiguous bytes of each row: 256 when K is a multiple of 128 (longer
// runs stream faster), else 128 or 64.
template <int MODE, int NBLK>
static hipError_t sm_dispatch(const Dims &d, const Inputs &in, const Work &w, hipStream_t s, int kgcd) {
  if (kgcd % 128 == 0) return sm_launch<MODE, NBLK, 256, 2>(d, in, w, s);
  if (kgcd % 64 == 0) return sm_launch<MODE, NBLK, 128, 2>(d, in, w, s);
  return sm_launch<MODE, NBLK, 64, 2>(d, in, w, s);
}

hipError_t launch_small_m_gateup(const Dims &d, const Inputs &in, const Work &w,
                                 hipStream_t s) {
  if (d.wdt == kMXFP4) return sm_mx_launch<kSmGateUp, kMXFP4, mx_blocks<kSmGateUp, kMXFP4>()>(d, in, w, s);
  if (d.wdt == kMXFP8) return sm_mx_launch<kSmGateUp, kMXFP8, mx_blocks<kSmGateUp, kMXFP8>()>(d, in, w, s);
  return sm_dispatch<kSmGateUp, 2>(d, in, w, s, d.H);   // 16 h columns per item
}

hipError_t launch_small_m_down(const Dims &d, const Inputs &in, const Work &w,
                               hipStream_t s) {
  if (d.wdt == kMXFP4) return sm_mx_launch<kSmDown, kMXFP4, mx_blocks<kSmDown, kMXFP4>()>(d, in, w, s);
  if (d.wdt == kMXFP8) return sm_mx_launch<kSmDown, kMXFP8, mx_blocks<kSmDown, kMXFP8>()>(d, in, w, s);
  // K is I for routed slots and I_s for the shared one: stages fit both
  const int kg = d.Is > 0 ? (d.I % 128 == 0 && d.Is % 128 == 0 ? 128 : (d.I % 64 == 0 && d.Is % 64 == 0 ? 64 : 32))
                          : d.I;
  return sm_dispatch<kSmDown, 2>(d, in, w, s, kg);      // 32 output columns per item
}

}  // namespace moe
