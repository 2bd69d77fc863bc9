"""Thin ctypes binding of libbakron.so (declared in include/bakron.h).

Argument marshalling only: tensors are allocated with torch on the current
device, their pointers and torch's current HIP stream are passed to the C ABI,
and every step of the computation runs in the library's HIP kernels.  There
is no fallback: without the built library or a GPU the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbakron.so")

Q_SYM, Q_ASYM, Q_UNIT = 0, 1, 2
ORDER_AUTO, ORDER_LA_FIRST, ORDER_LB_FIRST = 0, 1, 2
FLAG_PHASE_TIMING = 4
FLAG_NO_GRAPH = 8
FLAG_MSE_SCALE = 16
FLAG_SPLIT_COLS = 32
FLAG_SPLIT_ROWS = 64
DEV_NONFINITE, DEV_NOT_PD = 1, 2

EXPORTS = (
    "bakron_hessian_workspace_size", "bakron_hessian",
    "bakron_factor_workspace_size", "bakron_factor",
    "bakron_quantize_workspace_size", "bakron_quantize", "bakron_quantize_noalloc",
    "bakron_quantize_antidiag_workspace_size", "bakron_quantize_antidiag",
    "bakron_schedule_info", "bakron_schedule_plan", "bakron_last_phase_ms",
    "bakron_status_string", "bakron_last_error",
)

_lib = None


class BakronError(RuntimeError):
    pass


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbakron.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise BakronError(f"{path} is missing; build it with `python -m two_sided_gptq_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F, D = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                             ctypes.c_float, ctypes.c_double)
    lib.bakron_hessian_workspace_size.argtypes = [I64, I64]
    lib.bakron_hessian_workspace_size.restype = SZ
    lib.bakron_hessian.argtypes = [P, I64, I64, F, P, P, SZ, P]
    lib.bakron_hessian.restype = I32
    lib.bakron_factor_workspace_size.argtypes = [I64]
    lib.bakron_factor_workspace_size.restype = SZ
    lib.bakron_factor.argtypes = [P, I64, P, P, P, SZ, P]
    lib.bakron_factor.restype = I32
    lib.bakron_quantize_workspace_size.argtypes = [I64, I64, I32, I32]
    lib.bakron_quantize_workspace_size.restype = SZ
    lib.bakron_quantize.argtypes = [P, I64, I64, P, P, I32, I32, P, P, P, P, P, P, P, I32, P, SZ, P]
    lib.bakron_quantize.restype = I32
    lib.bakron_quantize_noalloc.argtypes = [P, I64, I64, P, P, I32, I32, P, P, P, P, P, P, P, I32, P]
    lib.bakron_quantize_noalloc.restype = I32
    lib.bakron_quantize_antidiag_workspace_size.argtypes = [I64, I64, I32, I32]
    lib.bakron_quantize_antidiag_workspace_size.restype = SZ
    lib.bakron_quantize_antidiag.argtypes = [P, I64, I64, P, P, I32, I32, P, P, P, P, P, P, P, SZ, P]
    lib.bakron_quantize_antidiag.restype = I32
    lib.bakron_schedule_info.argtypes = [I64, I64, I32, ctypes.POINTER(D)]
    lib.bakron_schedule_info.restype = I32
    lib.bakron_schedule_plan.argtypes = [I64, I64, I32, ctypes.POINTER(I32), I64,
                                         ctypes.POINTER(I64)]
    lib.bakron_schedule_plan.restype = I32
    lib.bakron_last_phase_ms.argtypes = [ctypes.POINTER(D)]
    lib.bakron_last_phase_ms.restype = I32
    lib.bakron_status_string.argtypes = [I32]
    lib.bakron_status_string.restype = ctypes.c_char_p
    lib.bakron_last_error.argtypes = []
    lib.bakron_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        lib = load()
        raise BakronError(f"{what}: {lib.bakron_status_string(rc).decode()} "
                          f"({lib.bakron_last_error().decode()})")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _f32_dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
        raise BakronError(f"{name} must be a contiguous float32 GPU tensor")
    return t


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def hessian(X: torch.Tensor, damp_rel: float, stream=None) -> torch.Tensor:
    """H = X^T X / N + damp_rel * mean(diag) * I (bakron_hessian)."""
    lib = load()
    X = _f32_dev(X, "X")
    N, d = X.shape
    H = torch.empty((d, d), dtype=torch.float32, device=X.device)
    ws = _workspace(lib.bakron_hessian_workspace_size(N, d), X.device)
    _check(lib.bakron_hessian(_ptr(X), N, d, float(damp_rel), _ptr(H), _ptr(ws), ws.numel(),
                              _stream(stream)), "bakron_hessian")
    return H


def factor(H: torch.Tensor, dev_status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """L with L L^T = H^-1, lower (bakron_factor)."""
    lib = load()
    H = _f32_dev(H, "H")
    d = H.shape[0]
    L = torch.empty((d, d), dtype=torch.float32, device=H.device)
    ws = _workspace(lib.bakron_factor_workspace_size(d), H.device)
    _check(lib.bakron_factor(_ptr(H), d, _ptr(L), _ptr(dev_status), _ptr(ws), ws.numel(),
                             _stream(stream)), "bakron_factor")
    return L


def quantize_workspace_size(m: int, n: int, kind: int, bits: int) -> int:
    return int(load().bakron_quantize_workspace_size(m, n, kind, bits))


def quantize(W, LA, LB, kind=Q_SYM, bits=4, order=ORDER_AUTO, want_V=True, want_E=False,
             want_sum=False, dev_status=None, timing=False, graph=True, workspace=None, out=None,
             stream=None, mse=False, split=None):
    """Run bakron_quantize.  Returns a dict with codes (int8), scales, zeros
    (None unless asymmetric), V, E, sum_e2 (device tensors or None).  split:
    None, "cols" or "rows" (the hybrid schedule, BAKRON_FLAG_SPLIT_*)."""
    lib = load()
    W = _f32_dev(W, "W")
    LA = _f32_dev(LA, "LA")
    LB = _f32_dev(LB, "LB")
    m, n = W.shape
    dev = W.device
    if out is None:
        out = dict(
            codes=torch.empty((m, n), dtype=torch.int8, device=dev),
            scales=torch.empty(m, dtype=torch.float32, device=dev),
            zeros=torch.empty(m, dtype=torch.float32, device=dev) if kind == Q_ASYM else None,
            V=torch.empty((m, n), dtype=torch.float32, device=dev) if want_V else None,
            E=torch.empty((m, n), dtype=torch.float32, device=dev) if want_E else None,
            sum_e2=torch.empty(1, dtype=torch.float64, device=dev) if want_sum else None,
        )
    if workspace is None:
        workspace = _workspace(quantize_workspace_size(m, n, kind, bits), dev)
    if split not in (None, "cols", "rows"):
        raise ValueError(f"split must be None, 'cols' or 'rows', not {split!r}")
    flags = (int(order) | (FLAG_PHASE_TIMING if timing else 0) | (0 if graph else FLAG_NO_GRAPH) |
             (FLAG_MSE_SCALE if mse else 0) | (FLAG_SPLIT_COLS if split == "cols" else 0) |
             (FLAG_SPLIT_ROWS if split == "rows" else 0))
    rc = lib.bakron_quantize(_ptr(W), m, n, _ptr(LA), _ptr(LB), kind, bits, _ptr(out["codes"]),
                             _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["V"]),
                             _ptr(out["E"]), _ptr(out["sum_e2"]), _ptr(dev_status), flags,
                             _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "bakron_quantize")
    return out


NOALLOC_SCRATCH_BYTES = 256 << 20  # BAKRON_NOALLOC_SCRATCH_BYTES


def quantize_noalloc(W, LA, LB, kind=Q_SYM, bits=4, order=ORDER_AUTO, want_V=True, want_E=False,
                     want_sum=False, dev_status=None, out=None, stream=None, mse=False, split=None):
    """Run bakron_quantize_noalloc (no workspace: the library's fixed scratch
    array; the plan in order on one stream).  Outputs as for quantize(); pass
    ``out`` to reuse preallocated output tensors."""
    lib = load()
    W = _f32_dev(W, "W")
    LA = _f32_dev(LA, "LA")
    LB = _f32_dev(LB, "LB")
    m, n = W.shape
    dev = W.device
    if out is None:
        out = dict(
            codes=torch.empty((m, n), dtype=torch.int8, device=dev),
            scales=torch.empty(m, dtype=torch.float32, device=dev),
            zeros=torch.empty(m, dtype=torch.float32, device=dev) if kind == Q_ASYM else None,
            V=torch.empty((m, n), dtype=torch.float32, device=dev) if want_V else None,
            E=torch.empty((m, n), dtype=torch.float32, device=dev) if want_E else None,
            sum_e2=torch.empty(1, dtype=torch.float64, device=dev) if want_sum else None,
        )
    if split not in (None, "cols", "rows"):
        raise ValueError(f"split must be None, 'cols' or 'rows', not {split!r}")
    flags = (int(order) | (FLAG_MSE_SCALE if mse else 0) | (FLAG_SPLIT_COLS if split == "cols" else 0) |
             (FLAG_SPLIT_ROWS if split == "rows" else 0))
    rc = lib.bakron_quantize_noalloc(_ptr(W), m, n, _ptr(LA), _ptr(LB), kind, bits, _ptr(out["codes"]),
                                     _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["V"]),
                                     _ptr(out["E"]), _ptr(out["sum_e2"]), _ptr(dev_status), flags,
                                     _stream(stream))
    _check(rc, "bakron_quantize_noalloc")
    return out


def quantize_antidiag(W, LA, LB, kind=Q_SYM, bits=4, want_V=True, want_E=False, dev_status=None,
                      stream=None):
    """Run bakron_quantize_antidiag (BaKron-antidiagonal).  Returns a dict with
    codes, scales, zeros (None unless asymmetric), V, E (device tensors or None)."""
    lib = load()
    W = _f32_dev(W, "W")
    LA = _f32_dev(LA, "LA")
    LB = _f32_dev(LB, "LB")
    m, n = W.shape
    dev = W.device
    out = dict(
        codes=torch.empty((m, n), dtype=torch.int8, device=dev),
        scales=torch.empty(m, dtype=torch.float32, device=dev),
        zeros=torch.empty(m, dtype=torch.float32, device=dev) if kind == Q_ASYM else None,
        V=torch.empty((m, n), dtype=torch.float32, device=dev) if want_V else None,
        E=torch.empty((m, n), dtype=torch.float32, device=dev) if want_E else None,
    )
    size = int(lib.bakron_quantize_antidiag_workspace_size(m, n, kind, bits))
    workspace = _workspace(size, dev)
    rc = lib.bakron_quantize_antidiag(_ptr(W), m, n, _ptr(LA), _ptr(LB), kind, bits, _ptr(out["codes"]),
                                      _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["V"]),
                                      _ptr(out["E"]), _ptr(dev_status), _ptr(workspace),
                                      workspace.numel(), _stream(stream))
    _check(rc, "bakron_quantize_antidiag")
    return out


SCHEDULE_KEYS = ("tile", "leaf_launches", "band_launches", "leaf_steps", "order",
                 "alg_band_flops", "exec_band_flops", "F", "leaf_flops", "depth",
                 "useful_band_flops", "pull_flops", "pull_leaves", "side_launches",
                 "side_useful_flops")


def schedule_info(m: int, n: int, order: int = ORDER_AUTO) -> dict:
    lib = load()
    buf = (ctypes.c_double * len(SCHEDULE_KEYS))()
    _check(lib.bakron_schedule_info(m, n, order, buf), "bakron_schedule_info")
    return dict(zip(SCHEDULE_KEYS, list(buf)))


PLAN_FIELDS = ("kind", "side", "ev", "K", "flags", "L", "H", "depth", "prod", "lo", "hi",
               "mode", "olo", "cols", "rlo", "rows")


def schedule_plan(m: int, n: int, order: int = ORDER_AUTO) -> list:
    """The ordered steps of an m x n solve (bakron_schedule_plan), one dict each."""
    lib = load()
    count = ctypes.c_int64(0)
    _check(lib.bakron_schedule_plan(m, n, order, None, 0, ctypes.byref(count)), "bakron_schedule_plan")
    buf = (ctypes.c_int32 * (16 * count.value))()
    _check(lib.bakron_schedule_plan(m, n, order, buf, count.value, ctypes.byref(count)),
           "bakron_schedule_plan")
    vals = list(buf)
    return [dict(zip(PLAN_FIELDS, vals[16 * k:16 * k + 16])) for k in range(count.value)]


PHASE_KEYS = ("prep_ms", "leaf_ms", "band_ms", "final_ms", "leaf_launches", "band_launches",
              "side_ms", "side_launches", "band_replay_ms", "side_replay_ms")


def last_phase_ms() -> dict:
    lib = load()
    buf = (ctypes.c_double * len(PHASE_KEYS))()
    _check(lib.bakron_last_phase_ms(buf), "bakron_last_phase_ms")
    return dict(zip(PHASE_KEYS, list(buf)))
