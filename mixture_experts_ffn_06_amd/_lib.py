"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every step of the layer runs in the HIP library; this module turns torch
tensors into device pointers and status codes into exceptions.  It fails
loudly when the library is missing -- there is no other implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

F32, BF16, FP8_E4M3, MXFP4, MXFP8 = 0, 1, 2, 3, 4
GATE_SOFTMAX, GATE_SIGMOID, GATE_SQRTSOFTPLUS = 0, 1, 2
PATHS = {"auto": 0, "simple": 1, "grouped": 2, "small_m": 3}
PATH_NAMES = {v: k for k, v in PATHS.items()}
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "mxfp4": MXFP4, "mxfp8": MXFP8}
GATINGS = {"softmax": GATE_SOFTMAX, "sigmoid": GATE_SIGMOID,
           "sqrtsoftplus": GATE_SQRTSOFTPLUS}

EXPORTS = ("moe_plan", "moe_workspace_bytes", "moe_forward", "moe_forward_debug",
           "moe_forward_noalloc", "moe_path_for", "moe_plan_destroy", "moe_strerror")
NOALLOC_SCRATCH_BYTES = 128 << 20      # MOE_NOALLOC_SCRATCH_BYTES


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("gating", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("weight_dtype", ctypes.c_int32),
                ("path", ctypes.c_int32)]


class MoeShared(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("gate", ctypes.c_void_p)]


NUM_STAGES = 7
STAGES = ("router", "topk", "permute", "quant", "gateup", "down", "combine")
DEBUG_BUFFERS = ("logits", "counts", "offsets", "sorted_pair", "slot_of_pair",
                 "xq", "sx", "h", "h_scale")


DEBUG_BUFFERS_2 = ("h_shared", "h_shared_scale", "y", "y_shared")


class MoeDebug(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_void_p) for n in DEBUG_BUFFERS] +
                [("events", ctypes.c_void_p * (NUM_STAGES + 1))] +
                [(n, ctypes.c_void_p) for n in DEBUG_BUFFERS_2])


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({strerror(status)})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by ``mixture_experts_ffn_06_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_ffn_06_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_plan.argtypes = [ctypes.POINTER(MoeConfig), ctypes.POINTER(vp)]
        L.moe_plan.restype = ctypes.c_int
        L.moe_workspace_bytes.argtypes = [vp, i32]
        L.moe_workspace_bytes.restype = sz
        fwd = [vp, i32, vp, vp, vp, vp, ctypes.POINTER(MoeShared), i32, vp, vp, vp,
               vp, vp, vp, vp, sz, vp]
        L.moe_forward.argtypes = fwd
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward_debug.argtypes = fwd + [ctypes.POINTER(MoeDebug)]
        L.moe_forward_debug.restype = ctypes.c_int
        L.moe_forward_noalloc.argtypes = fwd[:14] + [vp]
        L.moe_forward_noalloc.restype = ctypes.c_int
        L.moe_path_for.argtypes = [vp, i32]
        L.moe_path_for.restype = ctypes.c_int
        L.moe_plan_destroy.argtypes = [vp]
        L.moe_plan_destroy.restype = None
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().moe_strerror(status).decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _event_handle(ev) -> int:
    """hipEvent_t of a torch.cuda.Event (created on first use)."""
    h = ev.cuda_event
    if not h:
        ev.record()          # torch creates the HIP event lazily
        h = ev.cuda_event
    return h


class MoePlan:
    """A validated layer configuration (``moe_plan``)."""

    def __init__(self, hidden: int, num_experts: int, inter: int, topk: int,
                 max_tokens: int, shared_inter: int = 0, gating: str = "softmax",
                 renormalize: bool = True, routed_scale: float = 1.0,
                 weight_dtype: str = "bf16", path: str = "auto"):
        self.cfg = MoeConfig(hidden, num_experts, inter, shared_inter, topk,
                             max_tokens, GATINGS.get(gating, gating), int(renormalize),
                             float(routed_scale), DTYPES.get(weight_dtype, weight_dtype),
                             PATHS[path])
        self._h = ctypes.c_void_p()
        st = lib().moe_plan(ctypes.byref(self.cfg), ctypes.byref(self._h))
        if st != 0:
            raise MoeError(st, "moe_plan")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.moe_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def workspace_bytes(self, m: int) -> int:
        return int(lib().moe_workspace_bytes(self._h, m))

    def path_for(self, m: int) -> str:
        return PATH_NAMES[lib().moe_path_for(self._h, m)]

    def forward(self, x, router_w, w13, w2, out, topk_idx, topk_w, workspace,
                shared=None, bias=None, w13_scale=None, w2_scale=None,
                stream=None, debug=None, m: int | None = None,
                workspace_bytes: int | None = None, check: bool = True) -> int:
        """Enqueue one layer forward (``moe_forward``) on ``stream``.

        Tensors are torch device tensors (or raw device addresses).
        ``shared`` is None or a dict with ``w13, w2`` (+ ``w13_scale,
        w2_scale``, ``gate``); ``debug`` is None or a dict of stage tensors named as
        in ``moe_debug_t``, plus optionally ``events``: a sequence of
        ``NUM_STAGES + 1`` ``torch.cuda.Event`` (or None) recorded around the
        stages.  Returns the status; raises MoeError on failure when
        ``check``.
        """
        import torch
        if m is None:
            m = x.shape[0]
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        elif hasattr(stream, "cuda_stream"):
            stream = stream.cuda_stream
        if workspace_bytes is None:
            workspace_bytes = (workspace.numel() * workspace.element_size()
                               if hasattr(workspace, "numel") else 0)
        sh = None
        if shared is not None:
            sh = MoeShared(_ptr(shared["w13"]), _ptr(shared["w2"]),
                           _ptr(shared.get("w13_scale")), _ptr(shared.get("w2_scale")),
                           _ptr(shared.get("gate")))
        args = [self._h, m, _ptr(x), _ptr(router_w), _ptr(w13), _ptr(w2),
                ctypes.byref(sh) if sh is not None else None, self.cfg.topk,
                _ptr(out), _ptr(topk_idx), _ptr(topk_w), _ptr(bias),
                _ptr(w13_scale), _ptr(w2_scale), _ptr(workspace), workspace_bytes,
                stream]
        if debug is None:
            st = lib().moe_forward(*args)
        else:
            dbg = MoeDebug(*[_ptr(debug.get(n)) for n in DEBUG_BUFFERS])
            for n in DEBUG_BUFFERS_2:
                setattr(dbg, n, _ptr(debug.get(n)))
            for i, ev in enumerate(debug.get("events") or ()):
                dbg.events[i] = None if ev is None else _event_handle(ev)
            st = lib().moe_forward_debug(*args, ctypes.byref(dbg))
        if st != 0 and check:
            raise MoeError(st, "moe_forward")
        return st

    def forward_noalloc(self, x, router_w, w13, w2, out, topk_idx, topk_w,
                        shared=None, bias=None, w13_scale=None, w2_scale=None,
                        stream=None, m: int | None = None, check: bool = True) -> int:
        """Enqueue one layer forward through ``moe_forward_noalloc`` (the
        library's static per-GPU scratch instead of a workspace)."""
        import torch
        if m is None:
            m = x.shape[0]
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        elif hasattr(stream, "cuda_stream"):
            stream = stream.cuda_stream
        sh = None
        if shared is not None:
            sh = MoeShared(_ptr(shared["w13"]), _ptr(shared["w2"]),
                           _ptr(shared.get("w13_scale")), _ptr(shared.get("w2_scale")),
                           _ptr(shared.get("gate")))
        st = lib().moe_forward_noalloc(
            self._h, m, _ptr(x), _ptr(router_w), _ptr(w13), _ptr(w2),
            ctypes.byref(sh) if sh is not None else None, self.cfg.topk,
            _ptr(out), _ptr(topk_idx), _ptr(topk_w), _ptr(bias),
            _ptr(w13_scale), _ptr(w2_scale), stream)
        if st != 0 and check:
            raise MoeError(st, "moe_forward_noalloc")
        return st
