"""Thin ctypes binding of ``libmoe_mi355x.so`` (the C ABI in ``include/moe.h``).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch provides device memory and the current stream.  Importing this module
fails loudly when the library has not been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

from .configs import MoEConfig

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m mixture_experts_layer_27_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
MOE_WS_ROUTE, MOE_WS_ROUND, MOE_WS_EXPERTS, MOE_WS_BACKWARD, MOE_WS_EXPERTS_COMBINE = 0, 1, 2, 3, 4
STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_ENOTSUP", 3: "MOE_EWORKSPACE", 4: "MOE_EHIP"}
EXPORTS = ("moe_max_rows", "moe_plan_bytes", "moe_plan_init", "moe_workspace_bytes", "moe_route",
           "moe_round_tokens", "moe_permute", "moe_grouped_gemm_swiglu", "moe_grouped_gemm_swiglu_gather",
           "moe_grouped_gemm_swiglu_traced", "moe_grouped_gemm_swiglu_gather_traced",
           "moe_grouped_gemm_swiglu_noalloc", "moe_grouped_gemm_swiglu_combine", "moe_quantize_weights_mx",
           "moe_grouped_gemm_swiglu_wcodes",
           "moe_unpermute_combine", "moe_backward", "moe_backward_traced",
           "moe_quantize_mx", "moe_ref_stream", "moe_status_str")
TRACE_MAX_KERNELS = 48
NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("act", ctypes.c_int32), ("gemm", ctypes.c_int32),
                ("round_tile", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
                ("capacity_factor", ctypes.c_float), ("lb_coef", ctypes.c_float), ("z_coef", ctypes.c_float)]


_PLAN_FIELDS = ("logits", "probs_t", "topk_idx", "topk_gate", "counts_raw", "counts", "offsets",
                "token_of_row", "expert_of_row", "gate_of_row", "row_of_slot", "tok_ptr", "tok_rows",
                "keep_bits", "aux", "sched")


class MoePlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _PLAN_FIELDS]


class MoeTrace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("capacity", ctypes.c_int32),
                ("count", ctypes.c_int32), ("names", ctypes.c_char_p * TRACE_MAX_KERNELS)]


_vp, _sz, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
_P_SHAPE, _P_PLAN, _P_TRACE = ctypes.POINTER(MoeShape), ctypes.POINTER(MoePlan), ctypes.POINTER(MoeTrace)
for name, res, args in [
    ("moe_max_rows", _i64, [_P_SHAPE]),
    ("moe_plan_bytes", _sz, [_P_SHAPE]),
    ("moe_plan_init", ctypes.c_int, [_P_SHAPE, _vp, _sz, _P_PLAN]),
    ("moe_workspace_bytes", _sz, [_P_SHAPE, ctypes.c_int]),
    ("moe_route", ctypes.c_int, [_P_SHAPE, _vp, _vp, _vp, _vp, _P_PLAN, _vp, _sz, _vp]),
    ("moe_round_tokens", ctypes.c_int, [_P_SHAPE, _P_PLAN, _vp, _sz, _vp]),
    ("moe_permute", ctypes.c_int, [_P_SHAPE, _vp, _P_PLAN, _vp, _vp]),
    ("moe_grouped_gemm_swiglu", ctypes.c_int, [_P_SHAPE, _vp, _vp, _vp, _P_PLAN, _vp, _vp, _vp, _sz, _vp]),
    ("moe_grouped_gemm_swiglu_gather", ctypes.c_int, [_P_SHAPE, _vp, _vp, _vp, _P_PLAN, _vp, _vp, _vp, _sz, _vp]),
    ("moe_grouped_gemm_swiglu_noalloc", ctypes.c_int, [_P_SHAPE, _vp, _vp, _vp, _P_PLAN, _vp, _vp, _vp]),
    ("moe_grouped_gemm_swiglu_combine", ctypes.c_int,
     [_P_SHAPE, _vp, ctypes.c_int, _vp, _vp, _P_PLAN, _vp, _vp, _vp, _sz, _vp, _P_TRACE]),
    ("moe_quantize_weights_mx", ctypes.c_int, [_P_SHAPE, _vp, _vp, _vp, _sz, _vp]),
    ("moe_grouped_gemm_swiglu_wcodes", ctypes.c_int,
     [_P_SHAPE, _vp, ctypes.c_int, _P_PLAN, _vp, _vp, _vp, _sz, _vp, _P_TRACE]),
    ("moe_unpermute_combine", ctypes.c_int, [_P_SHAPE, _vp, _P_PLAN, _vp, _vp]),
    ("moe_grouped_gemm_swiglu_traced", ctypes.c_int,
     [_P_SHAPE, _vp, _vp, _vp, _P_PLAN, _vp, _vp, _vp, _sz, _vp, _P_TRACE]),
    ("moe_grouped_gemm_swiglu_gather_traced", ctypes.c_int,
     [_P_SHAPE, _vp, _vp, _vp, _P_PLAN, _vp, _vp, _vp, _sz, _vp, _P_TRACE]),
    ("moe_backward", ctypes.c_int, [_P_SHAPE, _vp, _vp, _vp, _vp, _P_PLAN, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _sz, _vp]),
    ("moe_backward_traced", ctypes.c_int, [_P_SHAPE, _vp, _vp, _vp, _vp, _P_PLAN, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _sz, _vp, _P_TRACE]),
    ("moe_quantize_mx", ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, _vp, _vp, _vp]),
    ("moe_ref_stream", ctypes.c_int, [_vp, _vp, _i64, ctypes.c_int, _vp]),
    ("moe_status_str", ctypes.c_char_p, [ctypes.c_int]),
]:
    fn = getattr(_lib, name)
    fn.restype, fn.argtypes = res, args


class MoEError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({_lib.moe_status_str(code).decode()})")
        self.code = code


def _check(fn: str, code: int):
    if code != 0:
        raise MoEError(fn, code)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


MOE_GATE_TOPK, MOE_GATE_ALL = 0, 1


def make_shape(T, d, E, k, d_ff, act=MOE_BF16, gemm=None, round_tile=0, gate_mode=MOE_GATE_TOPK,
               capacity_factor=0.0, lb_coef=0.0, z_coef=0.0) -> MoeShape:
    if gemm is None:
        gemm = act
    return MoeShape(T, d, E, k, d_ff, act, gemm, round_tile, gate_mode, capacity_factor, lb_coef, z_coef)


def shape_of(cfg: MoEConfig) -> MoeShape:
    act = MOE_BF16 if cfg.act == "bf16" else MOE_F32
    gemm = {"bf16": MOE_BF16, "f32": MOE_F32, "mxfp8": MOE_MXFP8}[cfg.gemm]
    gate_mode = {"topk": MOE_GATE_TOPK, "all": MOE_GATE_ALL}[cfg.gate]
    return make_shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, act, gemm, cfg.round_tile, gate_mode,
                      cfg.capacity_factor, cfg.lb_coef, cfg.z_coef)


def max_rows(s: MoeShape) -> int:
    return int(_lib.moe_max_rows(ctypes.byref(s)))


def plan_bytes(s: MoeShape) -> int:
    return int(_lib.moe_plan_bytes(ctypes.byref(s)))


def workspace_bytes(s: MoeShape, which: int) -> int:
    return int(_lib.moe_workspace_bytes(ctypes.byref(s), which))


class Plan:
    """A plan blob on the device plus the pointer table the C ABI fills in."""

    def __init__(self, s: MoeShape, device="cuda"):
        self.shape = s
        nbytes = plan_bytes(s)
        if nbytes == 0:
            raise MoEError("moe_plan_bytes", 2)
        self.blob = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.blob.data_ptr()) % 256
        self.blob = self.blob[off:off + nbytes]
        self.c = MoePlan()
        _check("moe_plan_init", _lib.moe_plan_init(ctypes.byref(s), _ptr(self.blob), nbytes, ctypes.byref(self.c)))

    def view(self, field: str, n: int, dtype=torch.int32) -> torch.Tensor:
        """A tensor view of one plan array (n elements)."""
        p = getattr(self.c, field)
        if p is None:
            raise ValueError(f"plan field {field} is not allocated for this shape")
        off = p - self.blob.data_ptr()
        esz = torch.tensor([], dtype=dtype).element_size()
        return self.blob[off:off + n * esz].view(dtype)

    def arrays(self) -> Dict[str, torch.Tensor]:
        s = self.shape
        N = max_rows(s)
        W = (s.E + 31) // 32
        out = {
            "logits": self.view("logits", s.T * s.E, torch.float32).view(s.T, s.E),
            "topk_idx": self.view("topk_idx", s.T * s.k).view(s.T, s.k),
            "topk_gate": self.view("topk_gate", s.T * s.k, torch.float32).view(s.T, s.k),
            "counts_raw": self.view("counts_raw", s.E),
            "counts": self.view("counts", s.E),
            "offsets": self.view("offsets", s.E + 1),
            "token_of_row": self.view("token_of_row", N),
            "expert_of_row": self.view("expert_of_row", N),
            "gate_of_row": self.view("gate_of_row", N, torch.float32),
            "row_of_slot": self.view("row_of_slot", s.T * s.k).view(s.T, s.k),
            "tok_ptr": self.view("tok_ptr", s.T + 1),
            "tok_rows": self.view("tok_rows", N),
            "keep_bits": self.view("keep_bits", s.T * W).view(s.T, W),
            "aux": self.view("aux", 4 + s.E, torch.float32),
        }
        if s.round_tile:
            out["probs_t"] = self.view("probs_t", s.E * s.T, torch.float32).view(s.E, s.T)
        return out


def _aligned_ws(nbytes: int, device="cuda") -> torch.Tensor:
    t = torch.empty(max(nbytes, 1) + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + max(nbytes, 1)]


# ----------------------------------------------------------------- entry points


def route(s: MoeShape, x, w_gate, bias, plan: Plan, ws=None, stream=None, noise=None):
    _check("moe_route", _lib.moe_route(ctypes.byref(s), _ptr(x), _ptr(w_gate), _ptr(bias), _ptr(noise),
                                       ctypes.byref(plan.c), _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(stream)))


def round_tokens(s: MoeShape, plan: Plan, ws=None, stream=None):
    _check("moe_round_tokens", _lib.moe_round_tokens(ctypes.byref(s), ctypes.byref(plan.c), _ptr(ws),
                                                     0 if ws is None else ws.numel(), _stream(stream)))


def permute(s: MoeShape, src, plan: Plan, dst, stream=None):
    _check("moe_permute", _lib.moe_permute(ctypes.byref(s), _ptr(src), ctypes.byref(plan.c), _ptr(dst),
                                           _stream(stream)))


class Trace:
    """Timing events between the kernels of one traced call (moe_trace).  The
    events are torch CUDA events with timing, recorded once here so their HIP
    handles exist; after the call, ``durations_ms()`` gives (kernel name, device
    time) in launch order (valid once the stream has passed the call)."""

    def __init__(self, capacity=TRACE_MAX_KERNELS + 1, stream=None):
        st = stream if stream is not None else torch.cuda.current_stream()
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        for ev in self.events:
            ev.record(st)
        self._handles = (ctypes.c_void_p * capacity)(*[ev.cuda_event for ev in self.events])
        self.c = MoeTrace(ctypes.cast(self._handles, ctypes.POINTER(ctypes.c_void_p)), capacity, 0)

    def durations_ms(self):
        n = self.c.count
        return [(self.c.names[i].decode(), self.events[i].elapsed_time(self.events[i + 1])) for i in range(n - 1)]


def grouped_gemm_swiglu(s: MoeShape, x_perm, w1, w2, plan: Plan, h_saved, y, ws, stream=None, trace=None):
    if trace is not None:
        _check("moe_grouped_gemm_swiglu_traced",
               _lib.moe_grouped_gemm_swiglu_traced(ctypes.byref(s), _ptr(x_perm), _ptr(w1), _ptr(w2),
                                                   ctypes.byref(plan.c), _ptr(h_saved), _ptr(y), _ptr(ws), ws.numel(),
                                                   _stream(stream), ctypes.byref(trace.c)))
        return
    _check("moe_grouped_gemm_swiglu",
           _lib.moe_grouped_gemm_swiglu(ctypes.byref(s), _ptr(x_perm), _ptr(w1), _ptr(w2), ctypes.byref(plan.c),
                                        _ptr(h_saved), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))


def grouped_gemm_swiglu_gather(s: MoeShape, x, w1, w2, plan: Plan, h_saved, y, ws, stream=None, trace=None):
    """The expert FFN reading the rows of x through the plan (no permuted copy)."""
    if trace is not None:
        _check("moe_grouped_gemm_swiglu_gather_traced",
               _lib.moe_grouped_gemm_swiglu_gather_traced(ctypes.byref(s), _ptr(x), _ptr(w1), _ptr(w2),
                                                          ctypes.byref(plan.c), _ptr(h_saved), _ptr(y), _ptr(ws),
                                                          ws.numel(), _stream(stream), ctypes.byref(trace.c)))
        return
    _check("moe_grouped_gemm_swiglu_gather",
           _lib.moe_grouped_gemm_swiglu_gather(ctypes.byref(s), _ptr(x), _ptr(w1), _ptr(w2), ctypes.byref(plan.c),
                                               _ptr(h_saved), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))


def grouped_gemm_swiglu_noalloc(s: MoeShape, x_perm, w1, w2, plan: Plan, h_saved, y, stream=None):
    """The expert FFN with the library's own device scratch (no workspace, no allocation)."""
    _check("moe_grouped_gemm_swiglu_noalloc",
           _lib.moe_grouped_gemm_swiglu_noalloc(ctypes.byref(s), _ptr(x_perm), _ptr(w1), _ptr(w2),
                                                ctypes.byref(plan.c), _ptr(h_saved), _ptr(y), _stream(stream)))


def grouped_gemm_swiglu_combine(s: MoeShape, x, w1, w2, plan: Plan, h_saved, out, ws, gathered=True, stream=None,
                                trace=None):
    """Expert FFN + combine with the gate and the scatter to token order in GEMM2's epilogue
    (out [T, d]; ws of workspace_bytes(s, MOE_WS_EXPERTS_COMBINE) bytes)."""
    _check("moe_grouped_gemm_swiglu_combine",
           _lib.moe_grouped_gemm_swiglu_combine(ctypes.byref(s), _ptr(x), int(bool(gathered)), _ptr(w1), _ptr(w2),
                                                ctypes.byref(plan.c), _ptr(h_saved), _ptr(out), _ptr(ws), ws.numel(),
                                                _stream(stream), None if trace is None else ctypes.byref(trace.c)))


def quantize_weights_mx(s: MoeShape, w1, w2, ws, stream=None):
    """MXFP8 codes of w1 and w2 (both orientations) into the expert workspace ws,
    for the micro-batches of one optimizer step (grouped_gemm_swiglu_wcodes)."""
    _check("moe_quantize_weights_mx", _lib.moe_quantize_weights_mx(ctypes.byref(s), _ptr(w1), _ptr(w2), _ptr(ws),
                                                                   ws.numel(), _stream(stream)))


def grouped_gemm_swiglu_wcodes(s: MoeShape, x, plan: Plan, h_saved, y, ws, gathered=True, stream=None, trace=None):
    """The MXFP8 expert FFN with the weight codes already in ws (quantize_weights_mx);
    x [T, d] read through the plan (gathered) or x_perm [N_max, d]."""
    _check("moe_grouped_gemm_swiglu_wcodes",
           _lib.moe_grouped_gemm_swiglu_wcodes(ctypes.byref(s), _ptr(x), int(bool(gathered)), ctypes.byref(plan.c),
                                               _ptr(h_saved), _ptr(y), _ptr(ws), ws.numel(), _stream(stream),
                                               None if trace is None else ctypes.byref(trace.c)))


def unpermute_combine(s: MoeShape, y, plan: Plan, out, stream=None):
    _check("moe_unpermute_combine", _lib.moe_unpermute_combine(ctypes.byref(s), _ptr(y), ctypes.byref(plan.c),
                                                               _ptr(out), _stream(stream)))


def backward(s: MoeShape, x, w_gate, w1, w2, plan: Plan, h_saved, dout, dx, dw_gate, dw1, dw2, ws,
             dlogits=None, ds=None, stream=None, x_perm=None, fwd_ws=None, trace=None):
    args = (ctypes.byref(s), _ptr(x), _ptr(w_gate), _ptr(w1), _ptr(w2), ctypes.byref(plan.c), _ptr(h_saved),
            _ptr(x_perm), _ptr(fwd_ws), _ptr(dout), _ptr(dx), _ptr(dw_gate), _ptr(dw1), _ptr(dw2), _ptr(dlogits),
            _ptr(ds), _ptr(ws), ws.numel(), _stream(stream))
    if trace is not None:
        _check("moe_backward_traced", _lib.moe_backward_traced(*args, ctypes.byref(trace.c)))
        return
    _check("moe_backward", _lib.moe_backward(*args))


def quantize_mx(src, codes, scales, k_axis=1, stream=None):
    """MXFP8 codes/scales of src [rows, cols] bf16 along k_axis (1: rows, 0: columns,
    written transposed [cols, rows])."""
    rows, cols = src.shape
    _check("moe_quantize_mx", _lib.moe_quantize_mx(_ptr(src), rows, cols, k_axis, _ptr(codes), _ptr(scales),
                                                   _stream(stream)))


REF_READ, REF_WRITE, REF_COPY_NT_LOAD, REF_COPY_NT_BOTH = 0, 1, 2, 3


def ref_stream(src, dst, nbytes, mode, stream=None):
    """Reference streaming kernel (measurement only): read, write or copy nbytes."""
    _check("moe_ref_stream", _lib.moe_ref_stream(_ptr(src), _ptr(dst), nbytes, mode, _stream(stream)))


# ----------------------------------------------------------------- one layer


class LayerRun:
    """Device buffers for one layer problem and the call sequence of a training step.

    ``forward()`` = route [+ round] + permute + grouped GEMMs + combine;
    ``backward()`` = the backward entry point.  Inputs must already be on the device.
    ``fused_gather``: the forward reads x through the plan inside the expert GEMMs
    (no x_perm) and the backward gathers x and dout the same way."""

    def __init__(self, cfg: MoEConfig, inputs: Dict[str, torch.Tensor], device="cuda", fused_gather=False):
        self.cfg = cfg
        self.fused_gather = bool(fused_gather)
        self.s = shape_of(cfg)
        s = self.s
        dt = torch.bfloat16 if cfg.act == "bf16" else torch.float32
        self.inp = {k: v.to(device).contiguous() for k, v in inputs.items()}
        self.N = max_rows(s)
        self.plan = Plan(s, device)
        self.x_perm = torch.empty((self.N, s.d), dtype=dt, device=device)
        self.h = torch.empty((self.N, 2 * s.d_ff), dtype=dt, device=device)
        self.y = torch.empty((self.N, s.d), dtype=dt, device=device)
        self.out = torch.empty((s.T, s.d), dtype=dt, device=device)
        self.ws_fwd = _aligned_ws(workspace_bytes(s, MOE_WS_EXPERTS), device)
        self.has_bwd = "dout" in self.inp
        if self.has_bwd:
            self.dx = torch.empty((s.T, s.d), dtype=dt, device=device)
            self.dw_gate = torch.empty((s.E, s.d), dtype=torch.float32, device=device)
            self.dw1 = torch.empty((s.E, 2 * s.d_ff, s.d), dtype=torch.float32, device=device)
            self.dw2 = torch.empty((s.E, s.d, s.d_ff), dtype=torch.float32, device=device)
            self.dlogits = torch.empty((s.T, s.E), dtype=torch.float32, device=device)
            self.ds = torch.empty((self.N,), dtype=torch.float32, device=device)
            self.ws_bwd = _aligned_ws(workspace_bytes(s, MOE_WS_BACKWARD), device)

    def route(self, stream=None):
        route(self.s, self.inp["x"], self.inp["w_gate"], self.inp.get("bias"), self.plan, stream=stream,
              noise=self.inp.get("noise"))
        if self.s.round_tile:
            round_tokens(self.s, self.plan, stream=stream)

    def forward(self, stream=None):
        self.route(stream)
        self.experts(stream)
        unpermute_combine(self.s, self.y, self.plan, self.out, stream)
        return self.out

    def experts(self, stream=None):
        """Permute + expert FFN, or (fused_gather) the expert FFN reading x through the plan."""
        if self.fused_gather:
            grouped_gemm_swiglu_gather(self.s, self.inp["x"], self.inp["w1"], self.inp["w2"], self.plan, self.h,
                                       self.y, self.ws_fwd, stream)
        else:
            permute(self.s, self.inp["x"], self.plan, self.x_perm, stream)
            grouped_gemm_swiglu(self.s, self.x_perm, self.inp["w1"], self.inp["w2"], self.plan, self.h, self.y,
                                self.ws_fwd, stream)

    def backward(self, stream=None, with_optional=True, reuse_x_perm=True, reuse_fwd_ws=True, trace=None):
        """reuse_x_perm: hand the forward's permuted x to the backward (else its dW1 reads x
        through the plan, or permutes x again where row gathers are not possible);
        reuse_fwd_ws: hand it the forward's workspace (MXFP8: the backward-orientation codes of
        W1, W2 and x_perm), else it quantises them again."""
        backward(self.s, self.inp["x"], self.inp["w_gate"], self.inp["w1"], self.inp["w2"], self.plan, self.h,
                 self.inp["dout"], self.dx, self.dw_gate, self.dw1, self.dw2, self.ws_bwd,
                 self.dlogits if with_optional else None, self.ds if with_optional else None, stream,
                 self.x_perm if (reuse_x_perm and not self.fused_gather) else None,
                 self.ws_fwd if reuse_fwd_ws else None, trace)

    def step(self, stream=None):
        self.forward(stream)
        if self.has_bwd:
            self.backward(stream)
