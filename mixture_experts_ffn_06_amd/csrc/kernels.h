// Internal launch interface between the C-ABI layer (moe_api.cpp) and the
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Shape and options of one forward call.
struct Dims {
  int m;        // tokens
  int H;        // hidden
  int E;        // routed experts
  int I;        // routed intermediate
  int Is;       // shared intermediate (0 = none)
  int k;        // top-k
  int te;       // m * k
  int wdt;      // weight storage: kF32 / kBF16 / kFP8 / kMXFP4 / kMXFP8
  int gating;   // 0 softmax, 1 sigmoid, 2 sqrtsoftplus
  int renorm;   // 1: renormalise the selected weights
  float scale;  // routed scaling factor
};

// Layer inputs (device pointers, caller-owned).
struct Inputs {
  const void *x;           // [m,H] f32 or bf16
  const void *router_w;    // [E,H]
  const void *w13;         // [E,2I,H]
  const void *w2;          // [E,H,I]
  const float *w13_scale;  // fp8: [E,2I/128,H/128] floats; MX: [E,2I,H/32] E8M0 bytes
  const float *w2_scale;   // fp8: [E,H/128,I/128] floats;  MX: [E,H,I/32] E8M0 bytes
  const float *bias;       // [E] or null
  const void *sw13;        // shared [2Is,H]
  const void *sw2;         // shared [H,Is]
  const float *sw13_scale; // [2Is/128,H/128] (MX: [2Is,H/32] bytes)
  const float *sw2_scale;  // [H/128,Is/128]  (MX: [H,Is/32] bytes)
  const void *sgate;       // [H] shared-expert gate vector (format of x) or null
};

// Device regions carved from the caller's workspace.
struct Work {
  float *logits;        // [m,E]
  float *rpart;         // [kRouterMaxSplits][m,E] router partial tiles (m <= 16)
  int *counts;          // [E]
  int *offsets;         // [E+1]
  int *sorted_pair;     // [te]
  int *slot_of_pair;    // [te]
  int *lrank;           // [te] rank of a pair among same-expert pairs of its run
  int *active;          // [E] experts with >= 1 pair, ascending
  int *nactive;         // [1]
  int *rboff;           // [E+1] per active slot: its first 16-row block (prefix of ceil(rows/16)); [nactive] = total
  int *perm_blk;        // [chunks][E] per-chunk counts, then starts (many pairs)
  uint8_t *xq;          // [m,H] fp8 codes of x
  float *sx;            // [m,H/128]
  void *h;              // [te,I]  routed SwiGLU output (sorted rows)
  float *h_scale;       // [te,I/128]
  void *h_sh;           // [m,Is]  shared SwiGLU output
  float *h_sh_scale;    // [m,Is/128]
  float *y;             // [te,H]  routed down output (sorted rows), fp32
  float *y_sh;          // [m,H]   shared down output, fp32
  int *queue;           // [kQueueInts] per-XCD unit tickets of the persistent
                        // GEMMs (gate/up: XCD x at kQueueStride x, down: at
                        // kQueueStride (8 + x)), zeroed by the routing sort
};

// Unit queues: one counter per XCD and GEMM, each on its own 128-byte line.
constexpr int kQueueStride = 32;
constexpr int kQueueInts = 16 * kQueueStride;

// permute.hip: one block below kPermMultiMin pairs, else chunks of
// perm_chunk(te) pairs, about eight of them (needs Work::perm_blk of
// permute_chunks(te) * E ints)
constexpr int kPermMultiMin = 8192;
__host__ __device__ inline int perm_chunk(long te) { return te >= 32768 ? 4096 : (te >= 16384 ? 2048 : 1024); }
__host__ __device__ inline int permute_chunks(long te) {
  return te >= kPermMultiMin ? static_cast<int>((te + perm_chunk(te) - 1) / perm_chunk(te)) : 0;
}
hipError_t launch_permute(const Dims &d, const int *topk_idx, const Work &w,
                          hipStream_t s);

// router.hip
// m <= 16 (route_fused_ok): the router writes kRouterMaxSplits-bounded K-split
// partial tiles to Work::rpart, and one kernel sums them, runs gating + top-k
// and the sort by expert
constexpr int kRouterMaxSplits = 8;
bool route_fused_ok(const Dims &d);
// fp8 layers with m > 16 and H a multiple of 512: the router kernel also
// writes xq and sx (no quantisation launch)
bool router_quant_fused(const Dims &d);
int router_splits(const Dims &d);
hipError_t launch_topk_permute(const Dims &d, const Inputs &in, const Work &w, int *topk_idx,
                               float *topk_w, hipStream_t s);
hipError_t launch_router(const Dims &d, const Inputs &in, const Work &w,
                         hipStream_t s);
hipError_t launch_topk(const Dims &d, const Inputs &in, const Work &w,
                       int *topk_idx, float *topk_w, hipStream_t s);

// quant.hip
hipError_t launch_quant_x(const Dims &d, const Inputs &in, const Work &w,
                          hipStream_t s);

// Expert paths: gate/up (+ SwiGLU) and down, routed and shared rows.
// simple.hip (fp32 VALU, any storage format)
hipError_t launch_simple_gateup(const Dims &d, const Inputs &in, const Work &w, hipStream_t s);
hipError_t launch_simple_down(const Dims &d, const Inputs &in, const Work &w, hipStream_t s);
// grouped.hip (MFMA grouped down GEMM, bf16 / fp8 weights)
hipError_t launch_grouped_down(const Dims &d, const Inputs &in, const Work &w, hipStream_t s);
// gateup.hip (grouped gate/up + SwiGLU on the bf16 32x32x16 MFMA; bf16 weights
// with H, I and I_s multiples of 32, fp8 weights with multiples of 128: the
// plan's own conditions; anything else returns hipErrorInvalidValue)
hipError_t launch_gu(const Dims &d, const Inputs &in, const Work &w, hipStream_t s);
// small_m.hip (weight streaming in 16-row blocks; bf16, MXFP4 and MXFP8 weights)
hipError_t launch_small_m_gateup(const Dims &d, const Inputs &in, const Work &w, hipStream_t s);
hipError_t launch_small_m_down(const Dims &d, const Inputs &in, const Work &w, hipStream_t s);

// combine.hip
hipError_t launch_combine(const Dims &d, const Inputs &in, const Work &w, const int *topk_idx,
                          const float *topk_w, void *out, hipStream_t s);

}  // namespace moe
