"""MI355X-native gradient compression with error feedback.

A thin ctypes binding over the C ABI of ``libgc.so`` (declared in
``include/gc.h``).  Every function here has the name of the C entry point it
marshals arguments for; all computation runs in the library's gfx950 kernels.
PyTorch supplies device memory and the stream only.

Importing this package loads ``libgc.so`` and raises ``ImportError`` if it has
not been built (``python -m gradient_compression_error_amd.build``).  There is
no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgc.so")

GC_OK, GC_ERR_ARG, GC_ERR_DTYPE, GC_ERR_WORKSPACE, GC_ERR_HIP = 0, 1, 2, 3, 4
GC_F32, GC_BF16 = 0, 1
GC_LEVEL_LOW, GC_LEVEL_HIGH = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m gradient_compression_error_amd.build` "
                      "(or __graft_entry__.build()); there is no fallback path")

lib = C.CDLL(LIB_PATH)


class gc_mat(C.Structure):
    _fields_ = [("grad", C.c_void_p), ("mem", C.c_void_p), ("q", C.c_void_p), ("p", C.c_void_p),
                ("out", C.c_void_p), ("n", C.c_int32), ("m", C.c_int32), ("rank", C.c_int32)]


class gc_span(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("len", C.c_int64)]


class gc_vec(C.Structure):
    _fields_ = [("grad", C.c_void_p), ("out", C.c_void_p), ("len", C.c_int64)]


def _sig(name, res, *args):
    f = getattr(lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_vp, _i64, _i32, _f32, _sz = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t
_sig("gc_status_str", C.c_char_p, _i32)
_sig("gc_last_error", C.c_char_p)
_sig("gc_topk_workspace_bytes", _sz, _i64, _i64)
_sig("gc_topk_ef_encode", _i32, _vp, _i32, _vp, _i64, _f32, _i64, _vp, _vp, _vp, _sz, _vp)
_sig("gc_topk_decode", _i32, _vp, _vp, _i64, _vp, _i64, _i32, _vp)
_sig("gc_topk_ef_encode_deferred", _i32, _vp, _i32, _vp, _i64, _f32, _i64, _vp, _vp, _vp, _i32, _vp, _sz, _vp)
_sig("gc_topk_materialize", _i32, _vp, _i64, _vp, _vp)
_sig("gc_randk_ef_encode", _i32, _vp, _i32, _vp, _i64, _f32, _vp, _i64, _vp, _vp)
_sig("gc_powersgd_workspace_bytes", _sz, C.POINTER(gc_mat), _i32)
_sig("gc_powersgd_ef_step", _i32, C.POINTER(gc_mat), _i32, _i32, _f32, _vp, _sz, _vp)
_sig("gc_powersgd_ef_step_deferred", _i32, C.POINTER(gc_mat), C.POINTER(C.c_int32), _i32, _i32, _f32, _vp, _sz, _vp)
_sig("gc_powersgd_materialize", _i32, C.POINTER(gc_mat), C.POINTER(C.c_int32), _i32, _vp, _sz, _vp)
_sig("gc_powersgd_plan_bytes", _sz, C.POINTER(gc_mat), _i32)
_sig("gc_powersgd_plan", _i32, C.POINTER(gc_mat), C.POINTER(C.c_int32), _i32, _i32, _vp, _sz, _vp, _sz, _vp)
_sig("gc_powersgd_run", _i32, _vp, _sz, _f32, _vp, _vp)
_sig("gc_powersgd_run_phases", _i32, _vp, _sz, _f32, _vp, _i32, _vp)
_sig("gc_grad_norm_workspace_bytes", _sz, C.POINTER(gc_span), _i32)
_sig("gc_grad_norm", _i32, C.POINTER(gc_span), _i32, _i32, _vp, _vp, _sz, _vp)
_sig("gc_grad_norm_noalloc", _i32, C.POINTER(gc_span), _i32, _i32, _vp, _vp)
_sig("gc_passthrough", _i32, C.POINTER(gc_vec), _i32, _i32, _f32, _vp)
_sig("gc_accordion_select", _i32, C.POINTER(C.c_float), C.POINTER(C.c_float), _i32, _f32, _i32,
     C.POINTER(C.c_int))
_sig("gc_timing_enable", _i32, C.c_char_p)
_sig("gc_timing_read", _i32, C.POINTER(C.c_double), C.POINTER(C.c_int64))
_sig("gc_kernel_names", C.c_char_p)

EXPORTED = ["gc_status_str", "gc_last_error", "gc_topk_workspace_bytes", "gc_topk_ef_encode",
            "gc_topk_ef_encode_deferred", "gc_topk_materialize",
            "gc_topk_decode", "gc_randk_ef_encode", "gc_powersgd_workspace_bytes", "gc_powersgd_ef_step",
            "gc_powersgd_ef_step_deferred", "gc_powersgd_materialize",
            "gc_powersgd_plan_bytes", "gc_powersgd_plan", "gc_powersgd_run", "gc_powersgd_run_phases",
            "gc_grad_norm_workspace_bytes", "gc_grad_norm", "gc_grad_norm_noalloc", "gc_passthrough",
            "gc_accordion_select",
            "gc_timing_enable", "gc_timing_read", "gc_kernel_names"]


class GCError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gc_status_str(status)} ({gc_last_error()})")


def _check(status: int, where: str):
    if status != GC_OK:
        raise GCError(status, where)


def gc_status_str(status: int) -> str:
    return lib.gc_status_str(status).decode()


def gc_last_error() -> str:
    return lib.gc_last_error().decode()


def gc_kernel_names() -> list[str]:
    return lib.gc_kernel_names().decode().split(",")


# ------------------------------------------------------------------ tensor helpers

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return GC_F32
    if t.dtype == torch.bfloat16:
        return GC_BF16
    raise TypeError(f"gradient dtype {t.dtype} not supported (float32 or bfloat16)")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


# The C ABI sees pointers and one length per call, so the sizes and dtypes of
# the tensors behind them are checked here, before any pointer is passed on.

def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dtype_is(t, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


# ------------------------------------------------------------------ top-k

def gc_topk_workspace_bytes(d: int, k: int) -> int:
    return int(lib.gc_topk_workspace_bytes(d, k))


def gc_topk_ef_encode(grad, mem, eta: float, k: int, out_idx, out_val, ws, stream=None) -> None:
    """Mem-SGD top-k encode: mem <- acc - top_k(acc), (out_idx, out_val) <- top_k(acc)."""
    import torch
    _dtype_is(mem, torch.float32, "mem")
    _dtype_is(out_idx, torch.int32, "out_idx")
    _dtype_is(out_val, torch.float32, "out_val")
    _need(grad.numel() == mem.numel(), "grad and mem must have the same number of entries")
    _need(out_idx.numel() >= k and out_val.numel() >= k, "out_idx and out_val need room for k entries")
    _check(lib.gc_topk_ef_encode(_ptr(grad), _dtype_code(grad), _ptr(mem), mem.numel(), float(eta), int(k),
                                 _ptr(out_idx), _ptr(out_val), _ptr(ws), _nbytes(ws), _stream(stream)),
           "gc_topk_ef_encode")


def gc_topk_ef_encode_deferred(grad, mem, eta: float, k: int, out_idx, out_val, sel, has_prev: bool, ws,
                               stream=None) -> None:
    """Top-k encode with the memory in deferred form: mem keeps acc and sel
    (int32 device tensor of 4 entries) records the selection, whose entries
    the next deferred call takes as +0.0."""
    import torch
    _dtype_is(mem, torch.float32, "mem")
    _dtype_is(out_idx, torch.int32, "out_idx")
    _dtype_is(out_val, torch.float32, "out_val")
    _dtype_is(sel, torch.int32, "sel")
    _need(sel.numel() >= 4, "sel needs 4 entries")
    _need(grad.numel() == mem.numel(), "grad and mem must have the same number of entries")
    _need(out_idx.numel() >= k and out_val.numel() >= k, "out_idx and out_val need room for k entries")
    _check(lib.gc_topk_ef_encode_deferred(_ptr(grad), _dtype_code(grad), _ptr(mem), mem.numel(), float(eta), int(k),
                                          _ptr(out_idx), _ptr(out_val), _ptr(sel), 1 if has_prev else 0, _ptr(ws),
                                          _nbytes(ws), _stream(stream)), "gc_topk_ef_encode_deferred")


def gc_topk_materialize(mem, sel, stream=None) -> None:
    """Writes a deferred top-k memory out (the selected entries become +0.0)."""
    import torch
    _dtype_is(mem, torch.float32, "mem")
    _dtype_is(sel, torch.int32, "sel")
    _need(sel.numel() >= 4, "sel needs 4 entries")
    _check(lib.gc_topk_materialize(_ptr(mem), mem.numel(), _ptr(sel), _stream(stream)), "gc_topk_materialize")


def gc_randk_ef_encode(grad, mem, eta: float, idx, out_val, stream=None) -> None:
    """Rand-k EF step on the given ascending index subset; k = idx.numel()."""
    import torch
    _dtype_is(mem, torch.float32, "mem")
    _dtype_is(idx, torch.int32, "idx")
    _dtype_is(out_val, torch.float32, "out_val")
    _need(grad.numel() == mem.numel(), "grad and mem must have the same number of entries")
    _need(out_val.numel() >= idx.numel(), "out_val needs room for idx.numel() entries")
    _check(lib.gc_randk_ef_encode(_ptr(grad), _dtype_code(grad), _ptr(mem), mem.numel(), float(eta), _ptr(idx),
                                  idx.numel(), _ptr(out_val), _stream(stream)), "gc_randk_ef_encode")


def gc_topk_decode(idx, val, out, accumulate: bool = False, stream=None) -> None:
    import torch
    _dtype_is(idx, torch.int32, "idx")
    _dtype_is(val, torch.float32, "val")
    _dtype_is(out, torch.float32, "out")
    _need(val.numel() == idx.numel(), "idx and val must have the same number of entries")
    k = idx.numel()
    _check(lib.gc_topk_decode(_ptr(idx) if k else None, _ptr(val) if k else None, k, _ptr(out), out.numel(),
                              1 if accumulate else 0, _stream(stream)), "gc_topk_decode")


# ------------------------------------------------------------------ PowerSGD

@dataclass
class Mat:
    """One PowerSGD matrix: grad/mem n x m, q (rank cols, m) column-major, p (rank cols, n), out n x m."""
    grad: object
    mem: object
    q: object
    rank: int
    p: object = None
    out: object = None


def _mats(mats: Sequence[Mat], prev=None, need_grad: bool = True):
    """ctypes array of the matrices; prev: the previous ranks of a deferred
    or materialize call (q and p must then hold max(rank, prev) columns)."""
    import torch
    _need(len(mats) >= 1, "need at least one matrix")
    g0 = next((a.grad for a in mats if a.grad is not None), None)
    arr = (gc_mat * len(mats))()
    for i, a in enumerate(mats):
        _need(a.mem.dim() == 2, f"mats[{i}].mem must be 2-D (n, m)")
        n, m = a.mem.shape
        r = max(int(a.rank), int(prev[i])) if prev is not None else int(a.rank)
        _dtype_is(a.mem, torch.float32, f"mats[{i}].mem")
        _dtype_is(a.q, torch.float32, f"mats[{i}].q")
        if a.grad is None:
            _need(not need_grad, f"mats[{i}].grad is required")
        else:
            _need(a.grad.dtype == g0.dtype, "every gradient must have the first one's dtype")
            _need(a.grad.numel() == n * m, f"mats[{i}].grad must have n*m entries")
        _need(a.q.numel() >= r * m, f"mats[{i}].q needs rank*m entries")
        if a.p is not None:
            _dtype_is(a.p, torch.float32, f"mats[{i}].p")
            _need(a.p.numel() >= r * n, f"mats[{i}].p needs rank*n entries")
        if a.out is not None:
            _dtype_is(a.out, torch.float32, f"mats[{i}].out")
            _need(a.out.numel() == n * m, f"mats[{i}].out must have n*m entries")
    for i, a in enumerate(mats):
        n, m = a.mem.shape
        arr[i] = gc_mat(_ptr(a.grad), _ptr(a.mem), _ptr(a.q), _ptr(a.p), _ptr(a.out), n, m, int(a.rank))
    return arr


class MatArray:
    """The matrices of a PowerSGD call marshalled once: checked and turned into
    the C array a single time, then passed to every step that uses the same
    buffers (the tensors must stay alive and in place).  For sets of hundreds
    of matrices this takes the per-call host work from about a millisecond to
    a few microseconds."""

    def __init__(self, mats: Sequence[Mat]):
        self.mats = list(mats)
        self.arr = _mats(self.mats)
        self.count = len(self.mats)
        self.dtype = _dtype_code(self.mats[0].grad)
        # columns of q and p each matrix has room for (bounds prev_rank)
        self.qcols = np.array([a.q.numel() // a.mem.shape[1] for a in self.mats], np.int64)
        self.pcols = np.array([a.p.numel() // a.mem.shape[0] if a.p is not None else 0 for a in self.mats], np.int64)


def gc_powersgd_workspace_bytes(mats: Sequence[Mat]) -> int:
    # the query reads the shapes only
    return int(lib.gc_powersgd_workspace_bytes(_mats(mats, need_grad=False), len(mats)))


def gc_powersgd_ef_step(mats, eta: float, ws, stream=None) -> None:
    """mats: a list of Mat, or a MatArray built from one."""
    if isinstance(mats, MatArray):
        arr, count, dt = mats.arr, mats.count, mats.dtype
    else:
        arr, count, dt = _mats(mats), len(mats), _dtype_code(mats[0].grad)
    _check(lib.gc_powersgd_ef_step(arr, count, dt, float(eta), _ptr(ws), _nbytes(ws), _stream(stream)),
           "gc_powersgd_ef_step")


def _prev_ranks(mats, prev_rank):
    prev = np.ascontiguousarray(prev_rank, np.int32)
    _need(prev.ndim == 1 and prev.size == len(mats), "prev_rank needs one entry per matrix")
    for i, a in enumerate(mats):
        _need(a.p is not None, f"mats[{i}].p is required: it keeps P^ for the deferred memory")
    return prev


def gc_powersgd_ef_step_deferred(mats, prev_rank, eta: float, ws, stream=None) -> None:
    """PowerSGD step with the memory kept as (M, P^, Q); prev_rank[i] = 0 when
    mem holds the memory itself, else the rank of the previous deferred call.
    mats: a list of Mat, or a MatArray built from one."""
    if isinstance(mats, MatArray):
        prev = np.ascontiguousarray(prev_rank, np.int32)
        _need(prev.ndim == 1 and prev.size == mats.count, "prev_rank needs one entry per matrix")
        _need(bool(np.all(mats.pcols > 0)), "every matrix needs p: it keeps P^ for the deferred memory")
        _need(bool(np.all((prev <= mats.qcols) & (prev <= mats.pcols))), "q and p need prev_rank columns")
        arr, count, dt = mats.arr, mats.count, mats.dtype
    else:
        prev = _prev_ranks(mats, prev_rank)
        arr, count, dt = _mats(mats, prev), len(mats), _dtype_code(mats[0].grad)
    _check(lib.gc_powersgd_ef_step_deferred(arr, prev.ctypes.data_as(C.POINTER(C.c_int32)), count, dt, float(eta),
                                            _ptr(ws), _nbytes(ws), _stream(stream)), "gc_powersgd_ef_step_deferred")


def gc_powersgd_plan_bytes(mats) -> int:
    arr = mats.arr if isinstance(mats, MatArray) else _mats(mats, need_grad=False)
    return int(lib.gc_powersgd_plan_bytes(arr, len(arr)))


def gc_powersgd_plan(mats, prev_rank, ws, stream=None) -> np.ndarray:
    """Records a PowerSGD step (prev_rank None: explicit memory; else the
    deferred form with these previous ranks).  Returns the host plan.
    mats: a list of Mat, or a MatArray built from one."""
    prev = None
    if isinstance(mats, MatArray):
        arr, count, dt = mats.arr, mats.count, mats.dtype
        if prev_rank is not None:
            prev = np.ascontiguousarray(prev_rank, np.int32)
            _need(prev.ndim == 1 and prev.size == count, "prev_rank needs one entry per matrix")
            _need(bool(np.all(mats.pcols > 0)), "every matrix needs p: it keeps P^ for the deferred memory")
            _need(bool(np.all((prev <= mats.qcols) & (prev <= mats.pcols))), "q and p need prev_rank columns")
    else:
        if prev_rank is not None:
            prev = _prev_ranks(mats, prev_rank)
        arr, count, dt = _mats(mats, prev), len(mats), _dtype_code(mats[0].grad)
    plan = np.zeros(int(lib.gc_powersgd_plan_bytes(arr, count)), np.uint8)
    pp = None if prev is None else prev.ctypes.data_as(C.POINTER(C.c_int32))
    _check(lib.gc_powersgd_plan(arr, pp, count, dt, plan.ctypes.data, plan.nbytes, _ptr(ws), _nbytes(ws),
                                _stream(stream)), "gc_powersgd_plan")
    return plan


def gc_powersgd_run(plan: np.ndarray, eta: float, ws, stream=None) -> None:
    """Launches a recorded PowerSGD step (kernels only)."""
    _need(isinstance(plan, np.ndarray) and plan.dtype == np.uint8, "plan must come from gc_powersgd_plan")
    _check(lib.gc_powersgd_run(plan.ctypes.data, plan.nbytes, float(eta), _ptr(ws), _stream(stream)),
           "gc_powersgd_run")


PHASE_ENCODE, PHASE_DECODE = 1, 2


def gc_powersgd_run_phases(plan: np.ndarray, eta: float, ws, phases: int, stream=None) -> None:
    """Launches the encode (1), the decode (2) or both (3) of a recorded step."""
    _need(isinstance(plan, np.ndarray) and plan.dtype == np.uint8, "plan must come from gc_powersgd_plan")
    _check(lib.gc_powersgd_run_phases(plan.ctypes.data, plan.nbytes, float(eta), _ptr(ws), int(phases),
                                      _stream(stream)), "gc_powersgd_run_phases")


def gc_powersgd_materialize(mats: Sequence[Mat], prev_rank, ws, stream=None) -> None:
    """Writes the deferred memory out: mem = M - P^ Q^T where prev_rank[i] > 0."""
    prev = _prev_ranks(mats, prev_rank)
    arr = _mats([Mat(grad=None, mem=a.mem, q=a.q, rank=a.rank, p=a.p) for a in mats], prev, need_grad=False)
    _check(lib.gc_powersgd_materialize(arr, prev.ctypes.data_as(C.POINTER(C.c_int32)), len(mats), _ptr(ws),
                                       _nbytes(ws), _stream(stream)), "gc_powersgd_materialize")


# ------------------------------------------------------------------ uncompressed tensors

def _vec_array(grads, outs):
    import torch
    _need(len(grads) >= 1 and len(grads) == len(outs), "need one out per gradient, at least one")
    arr = (gc_vec * len(grads))()
    for i, (g, o) in enumerate(zip(grads, outs)):
        _dtype_is(o, torch.float32, f"outs[{i}]")
        _need(g.dtype == grads[0].dtype, "every gradient must have the first one's dtype")
        _need(g.numel() == o.numel(), f"grads[{i}] and outs[{i}] must have the same number of entries")
        arr[i] = gc_vec(_ptr(g), _ptr(o), g.numel())
    return arr


def gc_passthrough(grads, outs, eta: float, stream=None) -> None:
    """Vectors sent uncompressed: outs[i] = eta * grads[i] (float32, one rounding)."""
    arr = _vec_array(grads, outs)
    _check(lib.gc_passthrough(arr, len(grads), _dtype_code(grads[0]), float(eta), _stream(stream)),
           "gc_passthrough")


class PreparedVecs:
    """gc_passthrough's argument array built once, for a set of vectors that is
    sent every step: calling it costs one library call and no per-vector
    marshalling.  It keeps the tensors alive; they must stay in place (their
    device addresses are in the array)."""

    def __init__(self, grads, outs):
        self.arr = _vec_array(grads, outs)
        self.n = len(grads)
        self.dtype = _dtype_code(grads[0])
        self._keep = (list(grads), list(outs))

    def __call__(self, eta: float, stream=None) -> None:
        _check(lib.gc_passthrough(self.arr, self.n, self.dtype, float(eta), _stream(stream)), "gc_passthrough")


def gc_passthrough_prepare(grads, outs) -> PreparedVecs:
    """The argument array of gc_passthrough(grads, outs, ...) for repeated calls."""
    return PreparedVecs(grads, outs)


# ------------------------------------------------------------------ norms / Accordion

def _spans(layers):
    arr = (gc_span * len(layers))()
    for i, t in enumerate(layers):
        arr[i] = gc_span(_ptr(t), t.numel())
    return arr


def gc_grad_norm_workspace_bytes(layers) -> int:
    return int(lib.gc_grad_norm_workspace_bytes(_spans(layers), len(layers)))


def gc_grad_norm(layers, norms, ws, stream=None) -> None:
    import torch
    _dtype_is(norms, torch.float32, "norms")
    _need(norms.numel() >= len(layers), "norms needs one entry per layer")
    _need(all(t.dtype == layers[0].dtype for t in layers), "every layer must have the first one's dtype")
    _check(lib.gc_grad_norm(_spans(layers), len(layers), _dtype_code(layers[0]), _ptr(norms), _ptr(ws), _nbytes(ws),
                            _stream(stream)), "gc_grad_norm")


GC_NORM_SCRATCH_TILES = 65536


def gc_grad_norm_noalloc(layers, norms, stream=None) -> None:
    """gc_grad_norm with the library's fixed per-device scratch instead of a workspace."""
    import torch
    _dtype_is(norms, torch.float32, "norms")
    _need(norms.numel() >= len(layers), "norms needs one entry per layer")
    _need(all(t.dtype == layers[0].dtype for t in layers), "every layer must have the first one's dtype")
    _check(lib.gc_grad_norm_noalloc(_spans(layers), len(layers), _dtype_code(layers[0]), _ptr(norms),
                                    _stream(stream)), "gc_grad_norm_noalloc")


def gc_accordion_select(norm_now, norm_prev, threshold: float, has_prev: bool):
    """Host call.  Returns (levels int32[n], new norm_prev float32[n])."""
    now = np.ascontiguousarray(norm_now, np.float32)
    prev = np.ascontiguousarray(norm_prev, np.float32).copy()
    _need(prev.size == now.size, "norm_now and norm_prev must have the same length")
    lv = np.zeros(now.size, np.int32)
    _check(lib.gc_accordion_select(now.ctypes.data_as(C.POINTER(C.c_float)), prev.ctypes.data_as(C.POINTER(C.c_float)),
                                   now.size, float(threshold), 1 if has_prev else 0,
                                   lv.ctypes.data_as(C.POINTER(C.c_int))), "gc_accordion_select")
    return lv, prev


# ------------------------------------------------------------------ timing hooks

def gc_timing_enable(kernel_name: Optional[str]) -> None:
    _check(lib.gc_timing_enable(kernel_name.encode() if kernel_name else None), "gc_timing_enable")


def gc_timing_read():
    ms, n = C.c_double(), C.c_int64()
    _check(lib.gc_timing_read(C.byref(ms), C.byref(n)), "gc_timing_read")
    return ms.value, n.value
