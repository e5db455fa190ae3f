// C ABI of libmoe (declared in include/moe.h): plan validation, workspace
// layout, argument checks and the launch sequence of one layer forward.
//
// Launch order on the caller's stream (forward_prefill.rs, page 3,
// MoeLayer::forward_prefill "Pipeline"):
//   router logits -> gating + top-k -> sort by expert [-> fp8 activation
//   quantisation] -> experts (gate/up + SwiGLU, down; routed and shared)
//   -> unpermute + weighted reduce + shared blend.
// No host synchronisation, no allocation, no host<->device copies.
#include <algorithm>
#include <limits>
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"

struct moe_plan_s {
  moe_config_t cfg;
};

namespace {

thread_local char g_err[256] = "";

int hip_fail(hipError_t e, const char *what) {
  std::snprintf(g_err, sizeof(g_err), "%s: %s", what, hipGetErrorString(e));
  return MOE_ERR_HIP;
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

bool aligned(const void *p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Most tokens the weight-streaming path takes with bf16 weights (an expert's
// rows in blocks of 16, each streaming its expert's weights once; the blocks
// of one expert run side by side, so the repeats are mostly served from
// cache): kBf16StreamMaxTokens, where the grouped MFMA path takes over (bf16
// layer of 128 experts, 2048 x 768, steps of 20: 64 tokens 269 K against
// 219 K tokens/s, 128 tokens 510 K against 423 K, 256 tokens 915 K against
// 828 K; 384 tokens 1.11 M against 1.21 M, the repeated streams cost more than
// they save).  MX weights take it at every batch size: an expert's weights
// (1.5 MB of MXFP4 w13 at that shape) stay in its XCD's L2 while its blocks
// run, and the alternative is the VALU path (MXFP4, 64 tokens: 59.5 ms against
// 0.14 ms); MXFP4 runs at 2.71 M tokens/s at 1024 tokens, 3.12 M at 2048,
// 3.53 M at 4096 and 3.72 M at 8192 (MXFP8 1.91 M, 2.10 M, 2.31 M, 2.38 M).
bool is_mx(int weight_dtype) { return weight_dtype == MOE_MXFP4 || weight_dtype == MOE_MXFP8; }

constexpr int kBf16StreamMaxTokens = 256;

int small_m_limit(const moe_config_t &c) {
  return is_mx(c.weight_dtype) ? std::numeric_limits<int>::max() : kBf16StreamMaxTokens;
}

int resolve_path(const moe_config_t &c, int m) {
  if (c.path != MOE_PATH_AUTO) return c.path;
  if (c.weight_dtype == MOE_F32) return MOE_PATH_SIMPLE;
  if ((c.weight_dtype == MOE_BF16 || is_mx(c.weight_dtype)) && m <= small_m_limit(c))
    return MOE_PATH_SMALL_M;
  return MOE_PATH_GROUPED;
}

// Byte sizes of every workspace region for m tokens.
struct Layout {
  enum {
    kLogits, kRpart, kCounts, kOffsets, kSorted, kSlot, kLrank, kActive, kNactive, kRbOff, kPermBlk, kXq,
    kSx, kH, kHs, kHsh, kHshs, kY, kYsh, kQueue, kN
  };
  size_t size[kN];
  size_t off[kN];
  size_t total;
};

Layout layout(const moe_plan_s &p, int m) {
  const moe_config_t &c = p.cfg;
  const size_t E = c.num_experts, H = c.hidden, I = c.inter, Is = c.shared_inter;
  const size_t te = static_cast<size_t>(m) * c.topk;
  const bool fp8 = c.weight_dtype == MOE_FP8_E4M3;
  const size_t hb = c.weight_dtype == MOE_F32 ? 4 : (fp8 ? 1 : 2);
  const size_t yb = 4;   // expert down outputs reach the combine in fp32
  Layout L;
  L.size[Layout::kLogits] = m * E * 4;
  L.size[Layout::kRpart] = m <= 16 ? static_cast<size_t>(moe::kRouterMaxSplits) * m * E * 4 : 0;
  L.size[Layout::kCounts] = E * 4;
  L.size[Layout::kOffsets] = (E + 1) * 4;
  L.size[Layout::kSorted] = te * 4;
  L.size[Layout::kSlot] = te * 4;
  L.size[Layout::kLrank] = te * 4;
  L.size[Layout::kActive] = E * 4;
  L.size[Layout::kNactive] = 4;
  L.size[Layout::kRbOff] = (E + 1) * 4;
  L.size[Layout::kPermBlk] = static_cast<size_t>(moe::permute_chunks(static_cast<long>(te))) * E * 4;
  L.size[Layout::kXq] = fp8 ? m * H : 0;
  L.size[Layout::kSx] = fp8 ? m * (H / 128) * 4 : 0;
  L.size[Layout::kH] = te * I * hb;
  L.size[Layout::kHs] = fp8 ? te * (I / 128) * 4 : 0;
  L.size[Layout::kHsh] = m * Is * hb;
  L.size[Layout::kHshs] = fp8 ? m * (Is / 128) * 4 : 0;
  L.size[Layout::kY] = te * H * yb;
  L.size[Layout::kYsh] = Is > 0 ? m * H * yb : 0;
  L.size[Layout::kQueue] = moe::kQueueInts * 4;
  size_t o = 0;
  for (int i = 0; i < Layout::kN; ++i) {
    L.off[i] = o;
    o += align256(L.size[i]);
  }
  L.total = o;
  return L;
}

moe::Work carve(const Layout &L, void *ws) {
  char *b = static_cast<char *>(ws);
  auto at = [&](int i) { return static_cast<void *>(b + L.off[i]); };
  moe::Work w;
  w.logits = static_cast<float *>(at(Layout::kLogits));
  w.rpart = static_cast<float *>(at(Layout::kRpart));
  w.counts = static_cast<int *>(at(Layout::kCounts));
  w.offsets = static_cast<int *>(at(Layout::kOffsets));
  w.sorted_pair = static_cast<int *>(at(Layout::kSorted));
  w.slot_of_pair = static_cast<int *>(at(Layout::kSlot));
  w.lrank = static_cast<int *>(at(Layout::kLrank));
  w.active = static_cast<int *>(at(Layout::kActive));
  w.nactive = static_cast<int *>(at(Layout::kNactive));
  w.rboff = static_cast<int *>(at(Layout::kRbOff));
  w.perm_blk = static_cast<int *>(at(Layout::kPermBlk));
  w.xq = static_cast<uint8_t *>(at(Layout::kXq));
  w.sx = static_cast<float *>(at(Layout::kSx));
  w.h = at(Layout::kH);
  w.h_scale = static_cast<float *>(at(Layout::kHs));
  w.h_sh = at(Layout::kHsh);
  w.h_sh_scale = static_cast<float *>(at(Layout::kHshs));
  w.y = static_cast<float *>(at(Layout::kY));
  w.y_sh = static_cast<float *>(at(Layout::kYsh));
  w.queue = static_cast<int *>(at(Layout::kQueue));
  return w;
}

int check_cfg(const moe_config_t &c) {
  if (c.hidden <= 0 || c.num_experts <= 0 || c.inter <= 0 || c.topk <= 0 ||
      c.max_tokens < 0 || c.shared_inter < 0)
    return MOE_ERR_INVALID_ARG;
  if (c.num_experts > 1024) return MOE_ERR_INVALID_ARG;
  if (c.topk > c.num_experts || c.topk > 32) return MOE_ERR_INVALID_ARG;
  if (c.gating < MOE_GATE_SOFTMAX || c.gating > MOE_GATE_SQRTSOFTPLUS) return MOE_ERR_INVALID_ARG;
  if (c.weight_dtype < MOE_F32 || c.weight_dtype > MOE_MXFP8) return MOE_ERR_INVALID_ARG;
  if (c.path < MOE_PATH_AUTO || c.path > MOE_PATH_SMALL_M) return MOE_ERR_INVALID_ARG;
  if (!(c.routed_scale == c.routed_scale)) return MOE_ERR_INVALID_ARG;  // NaN
  if (c.hidden % 8) return MOE_ERR_UNSUPPORTED;
  if (c.weight_dtype == MOE_FP8_E4M3 &&
      (c.hidden % 128 || c.inter % 128 || c.shared_inter % 128))
    return MOE_ERR_UNSUPPORTED;
  if (c.weight_dtype == MOE_BF16 &&
      (c.hidden % 32 || c.inter % 32 || c.shared_inter % 32))
    return MOE_ERR_UNSUPPORTED;
  if (c.weight_dtype == MOE_F32 && c.path != MOE_PATH_AUTO && c.path != MOE_PATH_SIMPLE)
    return MOE_ERR_UNSUPPORTED;
  const bool mx = c.weight_dtype == MOE_MXFP4 || c.weight_dtype == MOE_MXFP8;
  if (c.path == MOE_PATH_SMALL_M && c.weight_dtype != MOE_BF16 && !mx) return MOE_ERR_UNSUPPORTED;
  // the MX formats run on the weight-streaming path (one stage is 256 (FP4)
  // or 128 (FP8) K elements; the VALU path when forced); there is no grouped
  // MX GEMM
  const int mx_k = c.weight_dtype == MOE_MXFP4 ? 256 : 128;
  if (mx && (c.hidden % mx_k || c.inter % mx_k || c.shared_inter % mx_k || c.path == MOE_PATH_GROUPED))
    return MOE_ERR_UNSUPPORTED;
  // the expert kernels address each operand (token rows, the sorted h / y
  // rows, one expert's weight matrix) with 32-bit byte offsets
  const int64_t esz = c.weight_dtype == MOE_F32 ? 4 : 2;
  const int64_t widest = std::max<int64_t>({c.hidden, c.inter, c.shared_inter});
  const int64_t lim = int64_t(1) << 31;
  if (int64_t(c.max_tokens) * c.topk * widest * esz >= lim ||
      int64_t(2) * std::max(c.inter, c.shared_inter) * c.hidden * esz >= lim)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int run_forward(moe_plan_t plan, int32_t m, const void *x, const void *router_w,
                const void *w13, const void *w2, const moe_shared_t *shared,
                int32_t topk, void *out, int32_t *topk_idx, float *topk_w,
                const float *bias, const void *w13_scale,
                const void *w2_scale, void *ws, size_t ws_bytes,
                void *stream, const moe_debug_t *dbg) {
  if (!plan) return MOE_ERR_INVALID_ARG;
  const moe_config_t &c = plan->cfg;
  if (m < 0 || m > c.max_tokens || topk != c.topk) return MOE_ERR_INVALID_ARG;
  if (m == 0) return MOE_OK;
  const bool fp8 = c.weight_dtype == MOE_FP8_E4M3;
  const bool mx = c.weight_dtype == MOE_MXFP4 || c.weight_dtype == MOE_MXFP8;
  const bool scaled = fp8 || mx;   // block scales given
  const void *need[] = {x, router_w, w13, w2, out, topk_idx, topk_w, ws};
  for (const void *q : need)
    if (!q || !aligned(q, 16)) return MOE_ERR_INVALID_ARG;
  if (!aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
  if (scaled) {
    if (!w13_scale || !w2_scale || !aligned(w13_scale, 16) || !aligned(w2_scale, 16))
      return MOE_ERR_INVALID_ARG;
  } else if (w13_scale || w2_scale) {
    return MOE_ERR_INVALID_ARG;
  }
  if (bias && !aligned(bias, 16)) return MOE_ERR_INVALID_ARG;
  if ((c.shared_inter > 0) != (shared != nullptr)) return MOE_ERR_INVALID_ARG;
  if (shared) {
    if (!shared->w13 || !shared->w2 || !aligned(shared->w13, 16) || !aligned(shared->w2, 16))
      return MOE_ERR_INVALID_ARG;
    if (scaled && (!shared->w13_scale || !shared->w2_scale || !aligned(shared->w13_scale, 16) ||
                   !aligned(shared->w2_scale, 16)))
      return MOE_ERR_INVALID_ARG;
    if (!scaled && (shared->w13_scale || shared->w2_scale)) return MOE_ERR_INVALID_ARG;
    if (shared->gate && !aligned(shared->gate, 16)) return MOE_ERR_INVALID_ARG;
  }
  const int path = resolve_path(c, m);
  if (path == MOE_PATH_SMALL_M && m > small_m_limit(c)) return MOE_ERR_UNSUPPORTED;
  const Layout L = layout(*plan, m);
  if (ws_bytes < L.total) {
    std::snprintf(g_err, sizeof(g_err), "%d tokens need %zu bytes, %zu given", m, L.total, ws_bytes);
    return MOE_ERR_WORKSPACE;
  }

  moe::Dims d;
  d.m = m; d.H = c.hidden; d.E = c.num_experts; d.I = c.inter;
  d.Is = c.shared_inter; d.k = c.topk; d.te = m * c.topk;
  d.wdt = c.weight_dtype == MOE_F32 ? moe::kF32
        : fp8 ? moe::kFP8
        : c.weight_dtype == MOE_MXFP4 ? moe::kMXFP4
        : c.weight_dtype == MOE_MXFP8 ? moe::kMXFP8 : moe::kBF16;
  d.gating = c.gating; d.renorm = c.renormalize ? 1 : 0; d.scale = c.routed_scale;
  moe::Inputs in;
  in.x = x; in.router_w = router_w; in.w13 = w13; in.w2 = w2;
  in.w13_scale = static_cast<const float *>(w13_scale);   // E8M0 bytes for MXFP4
  in.w2_scale = static_cast<const float *>(w2_scale);
  in.bias = bias;
  in.sw13 = shared ? shared->w13 : nullptr;
  in.sw2 = shared ? shared->w2 : nullptr;
  in.sw13_scale = shared ? static_cast<const float *>(shared->w13_scale) : nullptr;
  in.sw2_scale = shared ? static_cast<const float *>(shared->w2_scale) : nullptr;
  in.sgate = shared ? shared->gate : nullptr;
  const moe::Work w = carve(L, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);

  // Stage sequence; with dbg->events set, an event is recorded before each
  // stage and after the last.
  auto mark = [&](int i) -> hipError_t {
    if (dbg && dbg->events[i])
      return hipEventRecord(static_cast<hipEvent_t>(dbg->events[i]), s);
    return hipSuccess;
  };
  hipError_t e;
  const char *what = "";
  const bool fused = moe::route_fused_ok(d);
  auto stage = [&](int i, const char *name, auto &&launch) -> bool {
    what = name;
    if ((e = mark(i)) != hipSuccess) return false;
    e = launch();
    return e == hipSuccess;
  };
  const bool ok =
      // m <= 16: top-k and sort in one kernel (the permute stage is empty)
      stage(MOE_STAGE_ROUTER, "router", [&] { return moe::launch_router(d, in, w, s); }) &&
      stage(MOE_STAGE_TOPK, "topk", [&] {
        return fused ? moe::launch_topk_permute(d, in, w, topk_idx, topk_w, s)
                     : moe::launch_topk(d, in, w, topk_idx, topk_w, s);
      }) &&
      stage(MOE_STAGE_PERMUTE, "permute", [&] {
        return fused ? hipSuccess : moe::launch_permute(d, topk_idx, w, s);
      }) &&
      // fp8: the router kernel quantised x already where it could
      stage(MOE_STAGE_QUANT, "quant_x", [&] {
        return fp8 && !moe::router_quant_fused(d) ? moe::launch_quant_x(d, in, w, s) : hipSuccess;
      }) &&
      stage(MOE_STAGE_GATEUP, "gate/up", [&] {
        switch (path) {
          case MOE_PATH_SIMPLE: return moe::launch_simple_gateup(d, in, w, s);
          case MOE_PATH_SMALL_M: return moe::launch_small_m_gateup(d, in, w, s);
          default: return moe::launch_gu(d, in, w, s);
        }
      }) &&
      stage(MOE_STAGE_DOWN, "down", [&] {
        switch (path) {
          case MOE_PATH_SIMPLE: return moe::launch_simple_down(d, in, w, s);
          case MOE_PATH_SMALL_M: return moe::launch_small_m_down(d, in, w, s);
          default: return moe::launch_grouped_down(d, in, w, s);
        }
      }) &&
      stage(MOE_STAGE_COMBINE, "combine", [&] { return moe::launch_combine(d, in, w, topk_idx, topk_w, out, s); }) &&
      stage(MOE_NUM_STAGES, "end event", [&] { return hipSuccess; });
  if (!ok) return hip_fail(e, what);

  if (dbg) {
    struct Copy { void *dst; int region; size_t bytes; };
    const size_t te = d.te;
    const Copy copies[] = {
        {dbg->logits, Layout::kLogits, L.size[Layout::kLogits]},
        {dbg->counts, Layout::kCounts, L.size[Layout::kCounts]},
        {dbg->offsets, Layout::kOffsets, L.size[Layout::kOffsets]},
        {dbg->sorted_pair, Layout::kSorted, te * 4},
        {dbg->slot_of_pair, Layout::kSlot, te * 4},
        {dbg->xq, Layout::kXq, L.size[Layout::kXq]},
        {dbg->sx, Layout::kSx, L.size[Layout::kSx]},
        {dbg->h, Layout::kH, L.size[Layout::kH]},
        {dbg->h_scale, Layout::kHs, L.size[Layout::kHs]},
        {dbg->h_shared, Layout::kHsh, L.size[Layout::kHsh]},
        {dbg->h_shared_scale, Layout::kHshs, L.size[Layout::kHshs]},
        {dbg->y, Layout::kY, L.size[Layout::kY]},
        {dbg->y_shared, Layout::kYsh, L.size[Layout::kYsh]},
    };
    for (const Copy &cp : copies) {
      if (!cp.dst || cp.bytes == 0) continue;
      e = hipMemcpyAsync(cp.dst, static_cast<char *>(ws) + L.off[cp.region],
                         cp.bytes, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "debug copy");
    }
  }
  return MOE_OK;
}

// ---- scratch of moe_forward_noalloc ----
// One copy of this array per GPU the library runs on, held until the process
// ends.  In host code its name is only a host-side stand-in: the device
// address comes from hipGetSymbolAddress, once per device with that device
// current, and only that address is ever handed to a kernel.
static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of this GPU's scratch (nullptr and the error on failure).
void *scratch_address(hipError_t *err) {
  static std::once_flag once[kMaxDevices];
  static void *addr[kMaxDevices];
  static hipError_t status[kMaxDevices];
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(once[dev], [dev] {
    void *p = nullptr;
    status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = status[dev] == hipSuccess ? p : nullptr;
  });
  *err = status[dev];
  return addr[dev];
}

}  // namespace

extern "C" {

int moe_plan(const moe_config_t *cfg, moe_plan_t *plan_out) {
  if (!cfg || !plan_out) return MOE_ERR_INVALID_ARG;
  const int st = check_cfg(*cfg);
  if (st != MOE_OK) return st;
  moe_plan_s *p = new (std::nothrow) moe_plan_s;
  if (!p) return MOE_ERR_NO_MEMORY;
  p->cfg = *cfg;
  *plan_out = p;
  return MOE_OK;
}

size_t moe_workspace_bytes(moe_plan_t plan, int32_t m) {
  if (!plan || m < 0) return 0;
  // enough for every call of up to m tokens: the regions grow with m, but
  // calls of <= 16 tokens also hold the router's partial sums, which larger
  // calls do without
  return std::max(layout(*plan, m).total, layout(*plan, std::min(m, 16)).total);
}

int moe_forward(moe_plan_t plan, int32_t m, const void *x, const void *router_w,
                const void *experts_w13, const void *experts_w2,
                const moe_shared_t *shared_w, int32_t topk, void *out,
                int32_t *topk_idx, float *topk_w, const float *router_bias,
                const void *w13_scale, const void *w2_scale, void *workspace,
                size_t workspace_bytes, void *stream) {
  return run_forward(plan, m, x, router_w, experts_w13, experts_w2, shared_w,
                     topk, out, topk_idx, topk_w, router_bias, w13_scale,
                     w2_scale, workspace, workspace_bytes, stream, nullptr);
}

int moe_forward_debug(moe_plan_t plan, int32_t m, const void *x,
                      const void *router_w, const void *experts_w13,
                      const void *experts_w2, const moe_shared_t *shared_w,
                      int32_t topk, void *out, int32_t *topk_idx, float *topk_w,
                      const float *router_bias, const void *w13_scale,
                      const void *w2_scale, void *workspace,
                      size_t workspace_bytes, void *stream,
                      const moe_debug_t *dbg) {
  return run_forward(plan, m, x, router_w, experts_w13, experts_w2, shared_w,
                     topk, out, topk_idx, topk_w, router_bias, w13_scale,
                     w2_scale, workspace, workspace_bytes, stream, dbg);
}

int moe_forward_noalloc(moe_plan_t plan, int32_t m, const void *x, const void *router_w,
                        const void *experts_w13, const void *experts_w2,
                        const moe_shared_t *shared_w, int32_t topk, void *out,
                        int32_t *topk_idx, float *topk_w, const float *router_bias,
                        const void *w13_scale, const void *w2_scale, void *stream) {
  if (!plan) return MOE_ERR_INVALID_ARG;
  if (m < 0 || m > plan->cfg.max_tokens) return MOE_ERR_INVALID_ARG;
  const size_t need = layout(*plan, m).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) {
    std::snprintf(g_err, sizeof(g_err),
                  "moe_forward_noalloc: %d tokens need %zu bytes of scratch, the static scratch "
                  "holds %zu", m, need, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
    return MOE_ERR_WORKSPACE;
  }
  if (m == 0) return run_forward(plan, 0, x, router_w, experts_w13, experts_w2, shared_w, topk,
                                 out, topk_idx, topk_w, router_bias, w13_scale, w2_scale,
                                 nullptr, 0, stream, nullptr);
  hipError_t e;
  void *ws = scratch_address(&e);
  if (!ws) return hip_fail(e, "moe_forward_noalloc: scratch address");
  return run_forward(plan, m, x, router_w, experts_w13, experts_w2, shared_w, topk, out,
                     topk_idx, topk_w, router_bias, w13_scale, w2_scale, ws,
                     MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_path_for(moe_plan_t plan, int32_t m) {
  if (!plan) return -1;
  return resolve_path(plan->cfg, m);
}

void moe_plan_destroy(moe_plan_t plan) { delete plan; }

const char *moe_strerror(int status) {
  thread_local char buf[320];
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE:
      std::snprintf(buf, sizeof(buf), "workspace too small (%s)", g_err);
      return buf;
    case MOE_ERR_NO_MEMORY: return "out of host memory";
    case MOE_ERR_HIP:
      std::snprintf(buf, sizeof(buf), "HIP error (%s)", g_err);
      return buf;
    default: return "unknown status";
  }
}

}  // extern "C"
