"""ctypes binding of libspade.so (argument marshalling only).

Every function here forwards to the C entry point of the same name declared
in include/spade.h; all computation happens in the library's HIP kernels.
There is no fallback: if the shared library is missing the import of the
binding raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPADE_LIB names another build of the same library (the host-sanitizer
# build the CPU tests load); by default the in-tree libspade.so
LIB_PATH = os.environ.get("SPADE_LIB") or os.path.join(_PKG, "libspade.so")

SPADE_OK = 0
SPADE_ERR_INVALID_ARG = 1
SPADE_ERR_UNSUPPORTED = 2
SPADE_ERR_CAPACITY = 3
SPADE_ERR_DEVICE = 4

SPADE_STATIC_SCRATCH_BYTES = 8 << 20  # the header's static selection buffer, per device

SPADE_BF16 = 0
SPADE_F32 = 1

SPADE_KEEP_COUNT = 0
SPADE_KEEP_RATIO = 1
SPADE_KEEP_MASS = 2

MODES = {"count": SPADE_KEEP_COUNT, "ratio": SPADE_KEEP_RATIO, "mass": SPADE_KEEP_MASS}

SPADE_SUM_MEAN = 0
SPADE_SUM_MAX = 1
SPADE_SUM_MIN = 2

SUMMARIZERS = {"mean": SPADE_SUM_MEAN, "max": SPADE_SUM_MAX, "min": SPADE_SUM_MIN}


class SpadeError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
        ("T", ctypes.c_int32), ("Hh", ctypes.c_int32), ("W", ctypes.c_int32),
        ("bt", ctypes.c_int32), ("bh", ctypes.c_int32), ("bw", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("summarizer", ctypes.c_int32),
    ]


class _Budget(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("per_head", ctypes.POINTER(ctypes.c_float)),
                ("window_enable", ctypes.c_int32), ("window_t", ctypes.c_int32),
                ("window_h", ctypes.c_int32), ("window_w", ctypes.c_int32)]


@dataclass(frozen=True)
class Problem:
    B: int
    H: int
    N: int
    d: int
    T: int
    Hh: int
    W: int
    bt: int
    bh: int
    bw: int
    dtype: int = SPADE_BF16
    scale: float = 0.0
    summarizer: int = SPADE_SUM_MEAN

    def c(self) -> _Problem:
        return _Problem(self.B, self.H, self.N, self.d, self.T, self.Hh, self.W,
                        self.bt, self.bh, self.bw, self.dtype, self.scale, self.summarizer)


class _BlockShape(ctypes.Structure):
    _fields_ = [("bt", ctypes.c_int32), ("bh", ctypes.c_int32), ("bw", ctypes.c_int32)]


def block_shapes(candidates: Sequence[Sequence[int]]):
    """Host array of block shapes (bt, bh, bw) for the scheme entry points."""
    arr = (_BlockShape * max(1, len(candidates)))()
    for i, (bt, bh, bw) in enumerate(candidates):
        arr[i] = _BlockShape(int(bt), int(bh), int(bw))
    return arr


class Budget:
    """Per-head keep budget (host memory, kept alive with the object); window is
    None or the static window's radii (rt, rh, rw) in blocks."""

    def __init__(self, mode, per_head: Sequence[float], window: Optional[Sequence[int]] = None):
        self.mode = MODES[mode] if isinstance(mode, str) else int(mode)
        self.values = (ctypes.c_float * max(1, len(per_head)))(*[float(v) for v in per_head])
        self.window = None if window is None else tuple(int(r) for r in window)
        wt, wh, ww = self.window if self.window is not None else (0, 0, 0)
        self._c = _Budget(self.mode, ctypes.cast(self.values, ctypes.POINTER(ctypes.c_float)),
                          1 if self.window is not None else 0, wt, wh, ww)

    def c(self) -> _Budget:
        return self._c


def _load() -> ctypes.CDLL:
    # torch first: its HIP runtime is then the one libspade.so binds to, so
    # torch's streams, events and allocations are valid handles for the library
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python input_adaptive_block_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(_Problem)
    Bp = ctypes.POINTER(_Budget)
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    sz = ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "spade_num_blocks": (ctypes.c_int32, [P]),
        "spade_max_nnz": (i64, [P, Bp]),
        "spade_workspace_bytes": (sz, [P]),
        "spade_check": (st, [P, Bp, i64]),
        "spade_status_string": (ctypes.c_char_p, [st]),
        "spade_summarize": (st, [P, vp, vp, vp, vp, vp]),
        "spade_summarize_sics": (st, [P, vp, vp, vp, vp, vp, vp, vp]),
        "spade_estimate_select": (st, [P, vp, vp, Bp, vp, vp, i64, vp, sz, vp]),
        "spade_estimate_select_static": (st, [P, vp, vp, Bp, vp, vp, i64, vp]),
        "spade_block_sparse_attn": (st, [P, vp, vp, vp, vp, vp, i64, vp, vp, sz, vp]),
        "spade_attn": (st, [P, vp, vp, vp, Bp, vp, vp, vp, i64, vp, sz, vp]),
        "spade_debug_scores": (st, [P, vp, vp, vp, vp]),
        "spade_debug_dense_walk": (ctypes.c_int32, [P]),
        "spade_schemes_workspace_bytes": (sz, [P, vp, ctypes.c_int32, Bp]),
        "spade_scheme_select": (st, [P, vp, vp, vp, ctypes.c_int32, vp, vp, vp, sz, vp]),
        "spade_attn_schemes": (st, [P, vp, vp, vp, vp, ctypes.c_int32, Bp, vp, vp, vp, vp, sz, vp]),
        "spade_profile_events": (None, [vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = _load()

EXPORTED = (
    "spade_num_blocks", "spade_max_nnz", "spade_workspace_bytes", "spade_check",
    "spade_status_string", "spade_summarize", "spade_summarize_sics", "spade_estimate_select",
    "spade_estimate_select_static",
    "spade_block_sparse_attn", "spade_attn", "spade_debug_scores", "spade_debug_dense_walk",
    "spade_profile_events",
    "spade_schemes_workspace_bytes", "spade_scheme_select", "spade_attn_schemes",
)


def lib() -> ctypes.CDLL:
    return _LIB


def status_string(status: int) -> str:
    return _LIB.spade_status_string(int(status)).decode()


def _ref(x):
    return ctypes.byref(x) if x is not None else None


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != SPADE_OK:
        raise SpadeError(status, where)


def spade_num_blocks(problem: Problem) -> int:
    return _LIB.spade_num_blocks(ctypes.byref(problem.c()))


def spade_max_nnz(problem: Problem, budget: Budget) -> int:
    return _LIB.spade_max_nnz(ctypes.byref(problem.c()), _ref(budget.c()))


def spade_workspace_bytes(problem: Problem) -> int:
    return _LIB.spade_workspace_bytes(ctypes.byref(problem.c()))


def spade_check(problem: Problem, budget: Optional[Budget] = None, col_capacity: int = -1) -> int:
    return _LIB.spade_check(ctypes.byref(problem.c()), None if budget is None else ctypes.byref(budget.c()),
                            int(col_capacity))


def spade_summarize(problem: Problem, q, k, q_mean, k_mean, stream=None) -> None:
    _check(_LIB.spade_summarize(ctypes.byref(problem.c()), _ptr(q), _ptr(k), _ptr(q_mean), _ptr(k_mean),
                                _stream(stream)), "spade_summarize")


def spade_summarize_sics(problem: Problem, q, k, q_mean, k_mean, q_sics, k_sics, stream=None) -> None:
    _check(_LIB.spade_summarize_sics(ctypes.byref(problem.c()), _ptr(q), _ptr(k), _ptr(q_mean), _ptr(k_mean),
                                     _ptr(q_sics), _ptr(k_sics), _stream(stream)), "spade_summarize_sics")


def spade_estimate_select(problem: Problem, q_mean, k_mean, budget: Budget, row_ptr, col_idx,
                          col_capacity: int, workspace, ws_bytes: int, stream=None) -> None:
    _check(_LIB.spade_estimate_select(ctypes.byref(problem.c()), _ptr(q_mean), _ptr(k_mean),
                                      ctypes.byref(budget.c()), _ptr(row_ptr), _ptr(col_idx),
                                      int(col_capacity), _ptr(workspace), int(ws_bytes), _stream(stream)),
           "spade_estimate_select")


def spade_debug_dense_walk(problem: Problem) -> int:
    return int(_LIB.spade_debug_dense_walk(ctypes.byref(problem.c())))


def spade_estimate_select_static(problem: Problem, q_mean, k_mean, budget: Budget, row_ptr, col_idx,
                                 col_capacity: int, stream=None) -> None:
    _check(_LIB.spade_estimate_select_static(ctypes.byref(problem.c()), _ptr(q_mean), _ptr(k_mean),
                                             ctypes.byref(budget.c()), _ptr(row_ptr), _ptr(col_idx),
                                             int(col_capacity), _stream(stream)),
           "spade_estimate_select_static")


def spade_block_sparse_attn(problem: Problem, q, k, v, row_ptr, col_idx, col_capacity: int, o,
                            workspace, ws_bytes: int, stream=None) -> None:
    _check(_LIB.spade_block_sparse_attn(ctypes.byref(problem.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                        _ptr(col_idx), int(col_capacity), _ptr(o), _ptr(workspace),
                                        int(ws_bytes), _stream(stream)),
           "spade_block_sparse_attn")


def spade_attn(problem: Problem, q, k, v, budget: Budget, o, row_ptr, col_idx, col_capacity: int,
               workspace, ws_bytes: int, stream=None) -> None:
    _check(_LIB.spade_attn(ctypes.byref(problem.c()), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(budget.c()),
                           _ptr(o), _ptr(row_ptr), _ptr(col_idx), int(col_capacity), _ptr(workspace),
                           int(ws_bytes), _stream(stream)),
           "spade_attn")


def spade_debug_scores(problem: Problem, q_mean, k_mean, scores, stream=None) -> None:
    _check(_LIB.spade_debug_scores(ctypes.byref(problem.c()), _ptr(q_mean), _ptr(k_mean), _ptr(scores),
                                   _stream(stream)), "spade_debug_scores")


def spade_profile_events(start, stop) -> None:
    """Record hipEvent handles around every later attention kernel (None, None: off)."""
    _LIB.spade_profile_events(start, stop)


def spade_schemes_workspace_bytes(problem: Problem, candidates, budget: Optional[Budget] = None) -> int:
    arr = block_shapes(candidates)
    return int(_LIB.spade_schemes_workspace_bytes(ctypes.byref(problem.c()), ctypes.cast(arr, ctypes.c_void_p),
                                                  len(candidates), ctypes.byref(budget.c()) if budget else None))


def spade_scheme_select(problem: Problem, q, k, candidates, agg, scheme, workspace, ws_bytes, stream=None) -> None:
    arr = block_shapes(candidates)
    _check(_LIB.spade_scheme_select(ctypes.byref(problem.c()), _ptr(q), _ptr(k), ctypes.cast(arr, ctypes.c_void_p),
                                    len(candidates), _ptr(agg), _ptr(scheme), _ptr(workspace), ws_bytes,
                                    _stream(stream)), "spade_scheme_select")


def spade_attn_schemes(problem: Problem, q, k, v, candidates, budget: Budget, o, agg, scheme, workspace, ws_bytes,
                       stream=None) -> None:
    arr = block_shapes(candidates)
    _check(_LIB.spade_attn_schemes(ctypes.byref(problem.c()), _ptr(q), _ptr(k), _ptr(v),
                                   ctypes.cast(arr, ctypes.c_void_p), len(candidates), ctypes.byref(budget.c()),
                                   _ptr(o), _ptr(agg), _ptr(scheme), _ptr(workspace), ws_bytes, _stream(stream)),
           "spade_attn_schemes")

