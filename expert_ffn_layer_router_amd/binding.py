"""ctypes binding of ``libmoe.so`` (the C ABI in ``include/moe.h``).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
Torch supplies device memory and the current stream. The ``moe_*`` functions mirror the
C entry points one to one; :func:`forward` additionally allocates the outputs and the
workspace with torch and calls ``moe_forward``.

The library is loaded on first use. If it has not been built, the first call raises
``RuntimeError``; there is no other implementation to fall back to.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path
from typing import Optional

LIB_PATH = Path(__file__).resolve().with_name("libmoe.so")

(MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
 MOE_ERR_SCRATCH_LIMIT) = range(6)
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20
MOE_F32, MOE_BF16 = 0, 1
KINDS = {"linear": 0, "relu2": 1, "swiglu": 2}
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16}

# Every symbol include/moe.h declares.
EXPORTED = (
    "moe_status_string", "moe_check_problem", "moe_capacity", "moe_workspace_size",
    "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward",
    "moe_forward_timed", "moe_workspace_size_ex", "moe_route_ex", "moe_dispatch_padded",
    "moe_expert_ffn_ex", "moe_forward_ex", "moe_backward_workspace_size", "moe_backward",
    "moe_saved_size", "moe_forward_train", "moe_backward_saved", "moe_route_noalloc",
)
STAGES = ("route", "dispatch", "expert_up", "expert_down", "combine")


class MoeProblem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("D", ctypes.c_int64), ("DH", ctypes.c_int64),
        ("D_out", ctypes.c_int64), ("E", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double), ("dtype", ctypes.c_int32),
        ("kind", ctypes.c_int32),
    ]


class MoeOptions(ctypes.Structure):
    """``moe_options``: router noise, un-renormalised gates, the padded layout and the
    importance-loss output (device pointers; all zero = the plain layer)."""
    _fields_ = [
        ("w_noise", ctypes.c_void_p), ("noise", ctypes.c_void_p),
        ("no_renormalise", ctypes.c_int32), ("padded", ctypes.c_int32),
        ("importance_loss", ctypes.c_void_p),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None
_P = ctypes.c_void_p
_PP = ctypes.POINTER(MoeProblem)
_PO = ctypes.POINTER(MoeOptions)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "or python -m expert_ffn_layer_router_amd.build_lib")
        L = ctypes.CDLL(str(LIB_PATH))
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_check_problem.restype = ctypes.c_int
        L.moe_check_problem.argtypes = [_PP]
        L.moe_capacity.restype = ctypes.c_int64
        L.moe_capacity.argtypes = [_PP]
        L.moe_workspace_size.restype = ctypes.c_size_t
        L.moe_workspace_size.argtypes = [_PP]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                _P]
        L.moe_route_noalloc.restype = ctypes.c_int
        L.moe_route_noalloc.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [_PP, _P, _P, _P, _P, _P]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P]
        L.moe_forward_timed.restype = ctypes.c_int
        L.moe_forward_timed.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, ctypes.c_size_t, _P, _P]
        L.moe_workspace_size_ex.restype = ctypes.c_size_t
        L.moe_workspace_size_ex.argtypes = [_PP, _PO]
        L.moe_route_ex.restype = ctypes.c_int
        L.moe_route_ex.argtypes = [_PP, _PO, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]
        L.moe_dispatch_padded.restype = ctypes.c_int
        L.moe_dispatch_padded.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                          _P]
        L.moe_expert_ffn_ex.restype = ctypes.c_int
        L.moe_expert_ffn_ex.argtypes = [_PP, _PO, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                        _P]
        L.moe_backward_workspace_size.restype = ctypes.c_size_t
        L.moe_backward_workspace_size.argtypes = [_PP]
        L.moe_backward.restype = ctypes.c_int
        L.moe_backward.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                   _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_saved_size.restype = ctypes.c_size_t
        L.moe_saved_size.argtypes = [_PP]
        L.moe_forward_train.restype = ctypes.c_int
        L.moe_forward_train.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, ctypes.c_size_t, _P, ctypes.c_size_t, _P]
        L.moe_backward_saved.restype = ctypes.c_int
        L.moe_backward_saved.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P, ctypes.c_float, _P, _P, _P, _P, _P,
                                         _P, _P, ctypes.c_size_t, _P]
        L.moe_forward_ex.restype = ctypes.c_int
        L.moe_forward_ex.argtypes = [_PP, _PO, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, ctypes.c_size_t, _P, _P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


@dataclass(frozen=True)
class Problem:
    """The problem statement, as in ``moe_problem``; dtype "f32"/"bf16", kind
    "linear"/"relu2"/"swiglu"."""

    T: int
    D: int
    DH: int
    D_out: int
    E: int
    top_k: int
    capacity_factor: float = 0.0
    dtype: str = "bf16"
    kind: str = "swiglu"

    def c(self) -> MoeProblem:
        return MoeProblem(self.T, self.D, self.DH, self.D_out, self.E, self.top_k,
                          float(self.capacity_factor), DTYPES[self.dtype], KINDS[self.kind])

    @classmethod
    def from_spec(cls, sp, T: Optional[int] = None) -> "Problem":
        return cls(T=sp.T if T is None else T, D=sp.D, DH=sp.DH, D_out=sp.D_out, E=sp.E,
                   top_k=sp.top_k, capacity_factor=sp.capacity_factor, dtype=sp.dtype,
                   kind=sp.kind)


def _ptr(t) -> Optional[int]:
    """Device address of a torch tensor (None -> NULL). Refuses host tensors."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def check_problem(p: Problem) -> int:
    return lib().moe_check_problem(ctypes.byref(p.c()))


def capacity(p: Problem) -> int:
    return int(lib().moe_capacity(ctypes.byref(p.c())))


def workspace_size(p: Problem) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(p.c())))


@dataclass
class Options:
    """``moe_options`` with torch tensors: w_noise (D, E) and noise (T, E) float32 (both or
    neither), renormalise, padded, importance_loss (1,) float32 output."""

    w_noise: object = None
    noise: object = None
    renormalise: bool = True
    padded: bool = False
    importance_loss: object = None

    def c(self) -> MoeOptions:
        return MoeOptions(_ptr(self.w_noise), _ptr(self.noise), 0 if self.renormalise else 1,
                          1 if self.padded else 0, _ptr(self.importance_loss))


def _opts(o: Optional[Options]):
    return None if o is None else ctypes.byref(o.c())


def workspace_size_ex(p: Problem, o: Optional[Options] = None) -> int:
    return int(lib().moe_workspace_size_ex(ctypes.byref(p.c()), _opts(o)))


def moe_route_ex(p: Problem, o: Optional[Options], x, w_router, router_bias, expert_indices,
                 gates, aux_loss, expert_counts=None, logits_out=None, uncertified=None,
                 ws=None, stream=None):
    _check(lib().moe_route_ex(ctypes.byref(p.c()), _opts(o), _ptr(x), _ptr(w_router),
                              _ptr(router_bias), _ptr(expert_indices), _ptr(gates),
                              _ptr(aux_loss), _ptr(expert_counts), _ptr(logits_out),
                              _ptr(uncertified), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream)), "moe_route_ex")


def moe_dispatch_padded(p: Problem, expert_indices, x, expert_counts, expert_offsets, perm,
                        slot_row, x_pad=None, ws=None, stream=None):
    _check(lib().moe_dispatch_padded(ctypes.byref(p.c()), _ptr(expert_indices), _ptr(x),
                                     _ptr(expert_counts), _ptr(expert_offsets), _ptr(perm),
                                     _ptr(slot_row), _ptr(x_pad), _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream)), "moe_dispatch_padded")


def moe_expert_ffn_ex(p: Problem, o: Optional[Options], x_perm, expert_offsets, w1, w3, w2,
                      y_perm, ws=None, stream=None):
    _check(lib().moe_expert_ffn_ex(ctypes.byref(p.c()), _opts(o), _ptr(x_perm),
                                   _ptr(expert_offsets), _ptr(w1), _ptr(w3), _ptr(w2),
                                   _ptr(y_perm), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream)), "moe_expert_ffn_ex")


def moe_forward_ex(p: Problem, o: Optional[Options], x, w_router, router_bias, w1, w3, w2, out,
                   expert_indices, gates, aux_loss, expert_counts, expert_offsets, slot_row, ws,
                   stage_events=None, stream=None):
    """``stage_events``: as in moe_forward_timed, or None."""
    _check(lib().moe_forward_ex(ctypes.byref(p.c()), _opts(o), _ptr(x), _ptr(w_router),
                                _ptr(router_bias), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out),
                                _ptr(expert_indices), _ptr(gates), _ptr(aux_loss),
                                _ptr(expert_counts), _ptr(expert_offsets), _ptr(slot_row),
                                _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(stream), stage_events), "moe_forward_ex")


def backward_workspace_size(p: Problem) -> int:
    return int(lib().moe_backward_workspace_size(ctypes.byref(p.c())))


def moe_backward(p: Problem, x, w_router, router_bias, w1, w3, w2, dout, d_aux: float, dx,
                 dw_router, dbias, dw1, dw3, dw2, ws, stream=None):
    _check(lib().moe_backward(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(router_bias),
                              _ptr(w1), _ptr(w3), _ptr(w2), _ptr(dout), float(d_aux), _ptr(dx),
                              _ptr(dw_router), _ptr(dbias), _ptr(dw1), _ptr(dw3), _ptr(dw2),
                              _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream)), "moe_backward")


def saved_size(p: Problem) -> int:
    return int(lib().moe_saved_size(ctypes.byref(p.c())))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def moe_forward_train(p: Problem, x, w_router, router_bias, w1, w3, w2, out, expert_indices,
                      gates, aux_loss, expert_counts, expert_offsets, slot_row, saved, ws,
                      stream=None):
    _check(lib().moe_forward_train(ctypes.byref(p.c()), _ptr(x), _ptr(w_router),
                                   _ptr(router_bias), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out),
                                   _ptr(expert_indices), _ptr(gates), _ptr(aux_loss),
                                   _ptr(expert_counts), _ptr(expert_offsets), _ptr(slot_row),
                                   _ptr(saved), _nbytes(saved), _ptr(ws), _nbytes(ws),
                                   _stream(stream)), "moe_forward_train")


def moe_backward_saved(p: Problem, x, w_router, w1, w3, w2, expert_indices, gates,
                       expert_counts, expert_offsets, slot_row, saved, dout, d_aux: float, dx,
                       dw_router, dbias, dw1, dw3, dw2, ws, stream=None):
    _check(lib().moe_backward_saved(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(w1),
                                    _ptr(w3), _ptr(w2), _ptr(expert_indices), _ptr(gates),
                                    _ptr(expert_counts), _ptr(expert_offsets), _ptr(slot_row),
                                    _ptr(saved), _nbytes(saved), _ptr(dout), float(d_aux),
                                    _ptr(dx), _ptr(dw_router), _ptr(dbias), _ptr(dw1), _ptr(dw3),
                                    _ptr(dw2), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_backward_saved")


def moe_route(p: Problem, x, w_router, router_bias, expert_indices, gates, aux_loss,
              expert_counts=None, logits_out=None, uncertified=None, ws=None, stream=None):
    _check(lib().moe_route(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(router_bias),
                           _ptr(expert_indices), _ptr(gates), _ptr(aux_loss),
                           _ptr(expert_counts), _ptr(logits_out), _ptr(uncertified), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(),
                           _stream(stream)), "moe_route")


def moe_route_noalloc(p: Problem, x, w_router, router_bias, expert_indices, gates, aux_loss,
                      expert_counts=None, logits_out=None, uncertified=None, stream=None):
    _check(lib().moe_route_noalloc(ctypes.byref(p.c()), _ptr(x), _ptr(w_router),
                                   _ptr(router_bias), _ptr(expert_indices), _ptr(gates),
                                   _ptr(aux_loss), _ptr(expert_counts), _ptr(logits_out),
                                   _ptr(uncertified), _stream(stream)), "moe_route_noalloc")


def moe_dispatch(p: Problem, expert_indices, x, expert_counts, expert_offsets, perm, slot_row,
                 x_perm=None, ws=None, stream=None):
    _check(lib().moe_dispatch(ctypes.byref(p.c()), _ptr(expert_indices), _ptr(x),
                              _ptr(expert_counts), _ptr(expert_offsets), _ptr(perm),
                              _ptr(slot_row), _ptr(x_perm), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream)), "moe_dispatch")


def moe_expert_ffn(p: Problem, x_perm, expert_offsets, w1, w3, w2, y_perm, ws=None,
                   stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(p.c()), _ptr(x_perm), _ptr(expert_offsets),
                                _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y_perm), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(stream)), "moe_expert_ffn")


def moe_combine(p: Problem, y_perm, slot_row, gates, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(p.c()), _ptr(y_perm), _ptr(slot_row), _ptr(gates),
                             _ptr(out), _stream(stream)), "moe_combine")


def moe_forward(p: Problem, x, w_router, router_bias, w1, w3, w2, out, expert_indices, gates,
                aux_loss, expert_counts, expert_offsets, slot_row, ws, stream=None):
    _check(lib().moe_forward(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(router_bias),
                             _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out), _ptr(expert_indices),
                             _ptr(gates), _ptr(aux_loss), _ptr(expert_counts),
                             _ptr(expert_offsets), _ptr(slot_row), _ptr(ws),
                             0 if ws is None else ws.numel() * ws.element_size(),
                             _stream(stream)), "moe_forward")


def moe_forward_timed(p: Problem, x, w_router, router_bias, w1, w3, w2, out, expert_indices,
                      gates, aux_loss, expert_counts, expert_offsets, slot_row, ws, stage_events,
                      stream=None):
    """``stage_events``: a ctypes array of 2 * len(STAGES) hipEvent_t handles (or None)."""
    _check(lib().moe_forward_timed(ctypes.byref(p.c()), _ptr(x), _ptr(w_router),
                                   _ptr(router_bias), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out),
                                   _ptr(expert_indices), _ptr(gates), _ptr(aux_loss),
                                   _ptr(expert_counts), _ptr(expert_offsets), _ptr(slot_row),
                                   _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream), stage_events), "moe_forward_timed")


class StageEvents:
    """2 * len(STAGES) HIP event slots for moe_forward_timed, created with hipEventCreate for
    the stages named in `stages` (default: all) and left NULL for the others."""

    def __init__(self, stages=None):
        self.stages = tuple(STAGES if stages is None else stages)
        unknown = set(self.stages) - set(STAGES)
        if unknown:
            raise ValueError(f"unknown stages {sorted(unknown)}")
        # HIP entry points through libmoe.so's own dependency scope, i.e. the one HIP
        # runtime this process has loaded (never a second copy)
        self._hip = lib()
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        n = 2 * len(STAGES)
        self.events = (ctypes.c_void_p * n)()
        for s, name in enumerate(STAGES):
            if name not in self.stages:
                continue
            for i in (2 * s, 2 * s + 1):
                h = ctypes.c_void_p()
                if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                self.events[i] = h
        self._alive = True

    def elapsed_ms(self) -> dict:
        """Per-stage device milliseconds; call after the stream has been synchronised."""
        out = {}
        for s, name in enumerate(STAGES):
            if name not in self.stages:
                continue
            ms = ctypes.c_float()
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.events[2 * s],
                                             self.events[2 * s + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = ms.value
        return out

    def close(self):
        if self._alive:
            for h in self.events:
                if h:
                    self._hip.hipEventDestroy(h)
            self._alive = False

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# --- convenience: allocate with torch, then call the C entry points -----------------------

def torch_dtype(p: Problem):
    import torch
    return torch.bfloat16 if p.dtype == "bf16" else torch.float32


def alloc_workspace(p: Problem, device="cuda", o: Optional[Options] = None):
    import torch
    n = workspace_size(p) if o is None else workspace_size_ex(p, o)
    # torch's caching allocator hands out blocks aligned to at least 512 bytes
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def alloc_outputs(p: Problem, device="cuda") -> dict:
    import torch
    i32 = torch.int32
    return dict(
        out=torch.empty((p.T, p.D_out), dtype=torch_dtype(p), device=device),
        expert_indices=torch.empty((p.T, p.top_k), dtype=i32, device=device),
        gates=torch.empty((p.T, p.top_k), dtype=torch.float32, device=device),
        aux_loss=torch.empty((1,), dtype=torch.float32, device=device),
        expert_counts=torch.empty((p.E,), dtype=i32, device=device),
        expert_offsets=torch.empty((p.E + 1,), dtype=i32, device=device),
        slot_row=torch.empty((p.T * p.top_k,), dtype=i32, device=device),
    )


def forward(p: Problem, x, w_router, router_bias, w1, w3=None, w2=None, ws=None, outs=None,
            stream=None) -> dict:
    """The whole layer; returns the output tensors (device) in a dict."""
    if outs is None:
        outs = alloc_outputs(p, x.device)
    if ws is None:
        ws = alloc_workspace(p, x.device)
    moe_forward(p, x, w_router, router_bias, w1, w3, w2, outs["out"], outs["expert_indices"],
                outs["gates"], outs["aux_loss"], outs["expert_counts"], outs["expert_offsets"],
                outs["slot_row"], ws, stream)
    return outs
