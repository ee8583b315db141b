"""ctypes binding of libmtgr.so: the C ABI of include/mtgr.h, same names.

Argument marshalling only: tensors are passed as device pointers plus sizes,
every computation runs in the library's HIP kernels.  PyTorch provides device
memory and streams.  There is no fallback: if the library is missing or was
not built, loading raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmtgr.so")

MTGR_F32, MTGR_BF16, MTGR_F16 = 0, 1, 2
(OP_PREP, OP_GLN_FWD, OP_GLN_BWD, OP_ATTN_FWD, OP_ATTN_BWD, OP_LAYER_FWD, OP_LAYER_BWD, OP_STACK_FWD,
 OP_STOCHASTIC_LENGTH) = range(9)

_DT = {torch.float32: MTGR_F32, torch.bfloat16: MTGR_BF16, torch.float16: MTGR_F16}

EXPORTED = (
    "mtgr_version", "mtgr_status_string", "mtgr_workspace_size", "mtgr_jagged_prep",
    "mtgr_group_layernorm", "mtgr_group_layernorm_bwd", "mtgr_hstu_attn_fwd", "mtgr_hstu_attn_bwd",
    "mtgr_hstu_layer_fwd", "mtgr_hstu_layer_bwd", "mtgr_hstu_stack_fwd", "mtgr_stack_graph_create",
    "mtgr_stack_graph_launch", "mtgr_stack_graph_destroy", "mtgr_stochastic_length",
    "mtgr_head_workspace_size", "mtgr_candidate_head_fwd", "mtgr_candidate_head_loss", "mtgr_serving_graph_create",
    "mtgr_set_validate", "mtgr_hstu_attn_fwd_noalloc",
)


class MtgrError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({_status_text(status)})")


class LayerParams(ctypes.Structure):
    _fields_ = [("W_uqkv", ctypes.c_void_p), ("b_uqkv", ctypes.c_void_p),
                ("gamma1", ctypes.c_void_p), ("beta1", ctypes.c_void_p),
                ("gamma2", ctypes.c_void_p), ("beta2", ctypes.c_void_p),
                ("W_o", ctypes.c_void_p), ("b_o", ctypes.c_void_p),
                ("d", ctypes.c_int32), ("H", ctypes.c_int32), ("dh", ctypes.c_int32),
                ("G", ctypes.c_int32), ("eps", ctypes.c_float), ("alpha", ctypes.c_float)]


class LayerSaved(ctypes.Structure):
    _fields_ = [("xhat", ctypes.c_void_p), ("mean1", ctypes.c_void_p), ("rstd1", ctypes.c_void_p),
                ("zgrad", ctypes.c_void_p), ("uqkv", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("mean2", ctypes.c_void_p), ("rstd2", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class LayerGrads(ctypes.Structure):
    _fields_ = [("W_uqkv", ctypes.c_void_p), ("b_uqkv", ctypes.c_void_p),
                ("gamma1", ctypes.c_void_p), ("beta1", ctypes.c_void_p),
                ("gamma2", ctypes.c_void_p), ("beta2", ctypes.c_void_p),
                ("W_o", ctypes.c_void_p), ("b_o", ctypes.c_void_p)]


class HeadParams(ctypes.Structure):
    _fields_ = [("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("W2", ctypes.c_void_p), ("b2", ctypes.c_void_p),
                ("d", ctypes.c_int32), ("h", ctypes.c_int32), ("n_tasks", ctypes.c_int32)]


class HeadGrads(ctypes.Structure):
    _fields_ = [("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("W2", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


class LayerBwdExtras(ctypes.Structure):
    _fields_ = [("d_uqkv", ctypes.c_void_p), ("d_o", ctypes.c_void_p)]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmtgr.so (raises OSError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} not found: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "mtgr_version": ([], ctypes.c_char_p),
        "mtgr_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "mtgr_set_validate": ([ctypes.c_int], ctypes.c_int),
        "mtgr_workspace_size": ([ctypes.c_int, I32, I64, I32, I32, I32, ctypes.c_int], SZ),
        "mtgr_jagged_prep": ([P, P, I32, I64, P, P, SZ, P], ctypes.c_int),
        "mtgr_group_layernorm": ([P, P, P, P, P, I64, I32, I32, F, ctypes.c_int, P, P, P], ctypes.c_int),
        "mtgr_group_layernorm_bwd": ([P, P, P, P, P, P, I64, I32, I32, ctypes.c_int, P, P, P, P, SZ, P],
                                     ctypes.c_int),
        "mtgr_hstu_attn_fwd": ([P, P, P, I64, P, I64, P, P, P, I32, I64, I32, I32, F, F, ctypes.c_int, P, SZ, P],
                               ctypes.c_int),
        "mtgr_hstu_attn_fwd_noalloc": ([P, P, P, I64, P, I64, P, P, P, I32, I64, I32, I32, F, F, ctypes.c_int, P],
                                       ctypes.c_int),
        "mtgr_hstu_attn_bwd": ([P, P, P, I64, P, I64, P, P, P, I64, P, P, P, I32, I64, I32, I32, I32, F, F,
                                ctypes.c_int, P, SZ, P], ctypes.c_int),
        "mtgr_hstu_layer_fwd": ([ctypes.POINTER(LayerParams), P, P, ctypes.POINTER(LayerSaved), P, P, P, I32,
                                 I64, F, ctypes.c_int, P, SZ, P], ctypes.c_int),
        "mtgr_hstu_layer_bwd": ([ctypes.POINTER(LayerParams), P, ctypes.POINTER(LayerSaved), P, P,
                                 ctypes.POINTER(LayerGrads), ctypes.POINTER(LayerBwdExtras), P, P, P, I32, I64,
                                 I32, F, ctypes.c_int, P, SZ, P], ctypes.c_int),
        "mtgr_hstu_stack_fwd": ([ctypes.POINTER(LayerParams), I32, P, P, P, P, P, I32, I64, F, ctypes.c_int, P,
                                 SZ, P], ctypes.c_int),
        "mtgr_stack_graph_create": ([ctypes.POINTER(LayerParams), I32, P, P, P, P, P, I32, I64, F, ctypes.c_int,
                                     P, SZ, ctypes.POINTER(ctypes.c_void_p)], ctypes.c_int),
        "mtgr_stack_graph_launch": ([P, P], ctypes.c_int),
        "mtgr_stack_graph_destroy": ([P], ctypes.c_int),
        "mtgr_stochastic_length": ([P, P, P, P, I64, I32, I64, I32, ctypes.c_int, P, I32, I64, P, P, P, P, I64, P,
                                    P, SZ, P], ctypes.c_int),
        "mtgr_head_workspace_size": ([I32, I64, I32, I32, I32, ctypes.c_int], SZ),
        "mtgr_candidate_head_fwd": ([ctypes.POINTER(HeadParams), P, I64, P, P, I32, I64, I64, P, ctypes.c_int, P, SZ,
                                     P], ctypes.c_int),
        "mtgr_candidate_head_loss": ([ctypes.POINTER(HeadParams), P, I64, P, P, I32, I64, I64, P, P, P, P, I64,
                                      ctypes.POINTER(HeadGrads), ctypes.c_int, P, SZ, P], ctypes.c_int),
        "mtgr_serving_graph_create": ([ctypes.POINTER(LayerParams), I32, ctypes.POINTER(HeadParams), P, P, P, I64, P,
                                       P, P, I32, I64, F, ctypes.c_int, P, SZ, P, SZ,
                                       ctypes.POINTER(ctypes.c_void_p)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load_library().mtgr_status_string(status).decode()
    except OSError:
        return "library not loaded"


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MtgrError(fn, status)


def _p(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(dtype: torch.dtype) -> int:
    return _DT[dtype]


def _ld(t: torch.Tensor) -> int:
    assert t.dim() == 2 and t.stride(1) == 1, "row-major [rows, cols] view expected"
    return t.stride(0)


# ---------------------------------------------------------------------------
def mtgr_version() -> str:
    return load_library().mtgr_version().decode()


def mtgr_status_string(status: int) -> str:
    return load_library().mtgr_status_string(status).decode()


def mtgr_set_validate(on: int) -> int:
    """Validation mode on (1) / off (0), or query (-1); returns the previous state."""
    return int(load_library().mtgr_set_validate(on))


def mtgr_workspace_size(op: int, B: int, T: int, max_len: int, d: int, H: int, dtype: torch.dtype) -> int:
    return int(load_library().mtgr_workspace_size(op, B, T, max_len, d, H, dtype_code(dtype)))


def workspace(op: int, B: int, T: int, d: int, H: int, dtype: torch.dtype, device="cuda",
              max_len: int = 0) -> torch.Tensor:
    """A byte buffer of the size ``op`` needs (allocation through torch).
    ``max_len`` > 0 (a bound on every row's length) sizes the backward ops for
    stored score gradients; the same value goes to the backward call."""
    n = mtgr_workspace_size(op, B, T, max_len, d, H, dtype)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def mtgr_jagged_prep(offsets, group_ids, seg, stream=None) -> None:
    B = offsets.numel() - 1
    T = group_ids.numel()
    _check("mtgr_jagged_prep", load_library().mtgr_jagged_prep(
        _p(offsets), _p(group_ids), B, T, _p(seg), None, 0, _stream(stream)))


def mtgr_group_layernorm(x, y, gamma, beta, group_ids, eps, mean_out=None, rstd_out=None, stream=None) -> None:
    T, d = x.shape
    G = gamma.shape[0]
    _check("mtgr_group_layernorm", load_library().mtgr_group_layernorm(
        _p(x), _p(y), _p(gamma), _p(beta), _p(group_ids), T, d, G, eps, dtype_code(x.dtype),
        _p(mean_out), _p(rstd_out), _stream(stream)))


def mtgr_group_layernorm_bwd(dy, x, mean, rstd, gamma, group_ids, dx, dgamma, dbeta, ws, stream=None) -> None:
    T, d = x.shape
    G = gamma.shape[0]
    _check("mtgr_group_layernorm_bwd", load_library().mtgr_group_layernorm_bwd(
        _p(dy), _p(x), _p(mean), _p(rstd), _p(gamma), _p(group_ids), T, d, G, dtype_code(x.dtype),
        _p(dx), _p(dgamma), _p(dbeta), _p(ws), ws.numel(), _stream(stream)))


def mtgr_hstu_attn_fwd(q, k, v, o, offsets, group_ids, timestamps, H, dh, alpha, attn_scale, ws,
                       stream=None) -> None:
    B = offsets.numel() - 1
    T = q.shape[0]
    assert _ld(q) == _ld(k) == _ld(v)
    _check("mtgr_hstu_attn_fwd", load_library().mtgr_hstu_attn_fwd(
        _p(q), _p(k), _p(v), _ld(q), _p(o), _ld(o), _p(offsets), _p(group_ids), _p(timestamps), B, T, H, dh,
        alpha, attn_scale, dtype_code(q.dtype), _p(ws), ws.numel(), _stream(stream)))


def mtgr_hstu_attn_fwd_noalloc(q, k, v, o, offsets, group_ids, timestamps, H, dh, alpha, attn_scale,
                               stream=None) -> None:
    B = offsets.numel() - 1
    T = q.shape[0]
    assert _ld(q) == _ld(k) == _ld(v)
    _check("mtgr_hstu_attn_fwd_noalloc", load_library().mtgr_hstu_attn_fwd_noalloc(
        _p(q), _p(k), _p(v), _ld(q), _p(o), _ld(o), _p(offsets), _p(group_ids), _p(timestamps), B, T, H, dh,
        alpha, attn_scale, dtype_code(q.dtype), _stream(stream)))


def mtgr_hstu_attn_bwd(q, k, v, d_o, dq, dk, dv, offsets, group_ids, timestamps, H, dh, alpha, attn_scale, ws,
                       max_len: int = 0, stream=None) -> None:
    B = offsets.numel() - 1
    T = q.shape[0]
    assert _ld(q) == _ld(k) == _ld(v) and _ld(dq) == _ld(dk) == _ld(dv)
    _check("mtgr_hstu_attn_bwd", load_library().mtgr_hstu_attn_bwd(
        _p(q), _p(k), _p(v), _ld(q), _p(d_o), _ld(d_o), _p(dq), _p(dk), _p(dv), _ld(dq), _p(offsets),
        _p(group_ids), _p(timestamps), B, T, max_len, H, dh, alpha, attn_scale, dtype_code(q.dtype), _p(ws),
        ws.numel(), _stream(stream)))


def make_params(p: Dict[str, torch.Tensor], H: int, eps: float = 1e-5, alpha: float = 1.0) -> LayerParams:
    d = p["W_o"].shape[0]
    return LayerParams(_p(p["W_uqkv"]), _p(p.get("b_uqkv")), _p(p["gamma1"]), _p(p["beta1"]),
                       _p(p["gamma2"]), _p(p["beta2"]), _p(p["W_o"]), _p(p.get("b_o")),
                       d, H, d // H, p["gamma1"].shape[0], eps, alpha)


def make_saved(s: Dict[str, torch.Tensor]) -> LayerSaved:
    return LayerSaved(*(_p(s[k]) for k in ("xhat", "mean1", "rstd1", "zgrad", "uqkv", "o", "mean2", "rstd2", "y")))


def alloc_saved(T: int, d: int, dtype: torch.dtype, device="cuda") -> Dict[str, torch.Tensor]:
    f = dict(dtype=dtype, device=device)
    s = dict(dtype=torch.float32, device=device)
    return dict(xhat=torch.empty(T, d, **f), mean1=torch.empty(T, **s), rstd1=torch.empty(T, **s),
                zgrad=torch.empty(T, 4 * d, **f), uqkv=torch.empty(T, 4 * d, **f), o=torch.empty(T, d, **f),
                mean2=torch.empty(T, **s), rstd2=torch.empty(T, **s), y=torch.empty(T, d, **f))


def alloc_grads(d: int, G: int, bias: bool, device="cuda") -> Dict[str, torch.Tensor]:
    f = dict(dtype=torch.float32, device=device)
    g = dict(W_uqkv=torch.empty(4 * d, d, **f), gamma1=torch.empty(G, d, **f), beta1=torch.empty(G, d, **f),
             gamma2=torch.empty(G, d, **f), beta2=torch.empty(G, d, **f), W_o=torch.empty(d, d, **f))
    if bias:
        g["b_uqkv"] = torch.empty(4 * d, **f)
        g["b_o"] = torch.empty(d, **f)
    return g


def mtgr_hstu_layer_fwd(params: LayerParams, x_in, x_out, saved: Optional[LayerSaved], offsets, group_ids,
                        timestamps, attn_scale, ws, stream=None) -> None:
    B = offsets.numel() - 1
    T = x_in.shape[0]
    _check("mtgr_hstu_layer_fwd", load_library().mtgr_hstu_layer_fwd(
        ctypes.byref(params), _p(x_in), _p(x_out), ctypes.byref(saved) if saved is not None else None,
        _p(offsets), _p(group_ids), _p(timestamps), B, T, attn_scale, dtype_code(x_in.dtype), _p(ws),
        ws.numel(), _stream(stream)))


def mtgr_hstu_layer_bwd(params: LayerParams, x_in, saved: LayerSaved, dx_out, dx_in, grads: Dict[str, torch.Tensor],
                        offsets, group_ids, timestamps, attn_scale, ws, extras: Optional[Dict] = None,
                        max_len: int = 0, stream=None) -> None:
    B = offsets.numel() - 1
    T = x_in.shape[0]
    g = LayerGrads(_p(grads["W_uqkv"]), _p(grads.get("b_uqkv")), _p(grads["gamma1"]), _p(grads["beta1"]),
                   _p(grads["gamma2"]), _p(grads["beta2"]), _p(grads["W_o"]), _p(grads.get("b_o")))
    ex = None
    if extras is not None:
        ex = ctypes.byref(LayerBwdExtras(_p(extras.get("d_uqkv")), _p(extras.get("d_o"))))
    _check("mtgr_hstu_layer_bwd", load_library().mtgr_hstu_layer_bwd(
        ctypes.byref(params), _p(x_in), ctypes.byref(saved), _p(dx_out), _p(dx_in), ctypes.byref(g), ex,
        _p(offsets), _p(group_ids), _p(timestamps), B, T, max_len, attn_scale, dtype_code(x_in.dtype), _p(ws),
        ws.numel(), _stream(stream)))


def _layer_array(layers: Sequence[LayerParams]):
    arr = (LayerParams * len(layers))(*layers)
    return arr, len(layers)


def mtgr_hstu_stack_fwd(layers: Sequence[LayerParams], x_in, x_out, offsets, group_ids, timestamps, attn_scale, ws,
                        stream=None) -> None:
    arr, L = _layer_array(layers)
    B = offsets.numel() - 1
    T = x_in.shape[0]
    _check("mtgr_hstu_stack_fwd", load_library().mtgr_hstu_stack_fwd(
        arr, L, _p(x_in), _p(x_out), _p(offsets), _p(group_ids), _p(timestamps), B, T, attn_scale,
        dtype_code(x_in.dtype), _p(ws), ws.numel(), _stream(stream)))


class StackGraph:
    """Handle of mtgr_stack_graph_create.  Holds references to the tensors the
    graph reads and writes so they outlive it; ``close`` (or garbage
    collection) calls mtgr_stack_graph_destroy."""

    def __init__(self, handle: int, keep: tuple):
        self.handle = handle
        self._keep = keep

    def launch(self, stream=None) -> None:
        mtgr_stack_graph_launch(self, stream)

    def close(self) -> None:
        if self.handle:
            load_library().mtgr_stack_graph_destroy(self.handle)
            self.handle = None
            self._keep = ()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mtgr_stack_graph_create(layers: Sequence[LayerParams], x_in, x_out, offsets, group_ids, timestamps, attn_scale,
                            ws) -> StackGraph:
    arr, L = _layer_array(layers)
    B = offsets.numel() - 1
    T = x_in.shape[0]
    h = ctypes.c_void_p()
    _check("mtgr_stack_graph_create", load_library().mtgr_stack_graph_create(
        arr, L, _p(x_in), _p(x_out), _p(offsets), _p(group_ids), _p(timestamps), B, T, attn_scale,
        dtype_code(x_in.dtype), _p(ws), ws.numel(), ctypes.byref(h)))
    return StackGraph(h.value, (x_in, x_out, offsets, group_ids, timestamps, ws))


def mtgr_stack_graph_launch(graph: StackGraph, stream=None) -> None:
    _check("mtgr_stack_graph_launch", load_library().mtgr_stack_graph_launch(graph.handle, _stream(stream)))


def mtgr_stack_graph_destroy(graph: StackGraph) -> None:
    graph.close()


def mtgr_stochastic_length(offsets, group_ids, timestamps, x, u, s_keep: int, token_budget: int, offsets_out,
                           group_ids_out, timestamps_out, x_out, fit_out, ws, stream=None) -> None:
    B = offsets.numel() - 1
    T = x.shape[0]
    _check("mtgr_stochastic_length", load_library().mtgr_stochastic_length(
        _p(offsets), _p(group_ids), _p(timestamps), _p(x), _ld(x), B, T, x.shape[1], dtype_code(x.dtype), _p(u),
        s_keep, token_budget, _p(offsets_out), _p(group_ids_out), _p(timestamps_out), _p(x_out), _ld(x_out),
        _p(fit_out), _p(ws), ws.numel(), _stream(stream)))


def make_head_params(p: Dict[str, torch.Tensor]) -> HeadParams:
    h, d = p["W1"].shape
    return HeadParams(_p(p["W1"]), _p(p.get("b1")), _p(p["W2"]), _p(p.get("b2")), d, h, p["W2"].shape[0])


def head_workspace(B: int, n_cand: int, d: int, h: int, n_tasks: int, dtype: torch.dtype, device="cuda"):
    n = int(load_library().mtgr_head_workspace_size(B, n_cand, d, h, n_tasks, dtype_code(dtype)))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def mtgr_candidate_head_fwd(params: HeadParams, x, offsets, group_ids, n_cand: int, logits, ws, stream=None) -> None:
    _check("mtgr_candidate_head_fwd", load_library().mtgr_candidate_head_fwd(
        ctypes.byref(params), _p(x), _ld(x), _p(offsets), _p(group_ids), offsets.numel() - 1, x.shape[0], n_cand,
        _p(logits), dtype_code(x.dtype), _p(ws), ws.numel(), _stream(stream)))


def mtgr_candidate_head_loss(params: HeadParams, x, offsets, group_ids, n_cand: int, labels, loss, logits, dx,
                             grads: Dict[str, torch.Tensor], ws, stream=None) -> None:
    g = HeadGrads(_p(grads["W1"]), _p(grads.get("b1")), _p(grads["W2"]), _p(grads.get("b2")))
    _check("mtgr_candidate_head_loss", load_library().mtgr_candidate_head_loss(
        ctypes.byref(params), _p(x), _ld(x), _p(offsets), _p(group_ids), offsets.numel() - 1, x.shape[0], n_cand,
        _p(labels), _p(loss), _p(logits), _p(dx), _ld(dx), ctypes.byref(g), dtype_code(x.dtype), _p(ws), ws.numel(),
        _stream(stream)))


def mtgr_serving_graph_create(layers: Sequence[LayerParams], head: HeadParams, x_in, x_out, logits, n_cand: int,
                              offsets, group_ids, timestamps, attn_scale, ws, head_ws) -> StackGraph:
    arr, L = _layer_array(layers)
    B = offsets.numel() - 1
    T = x_in.shape[0]
    h = ctypes.c_void_p()
    _check("mtgr_serving_graph_create", load_library().mtgr_serving_graph_create(
        arr, L, ctypes.byref(head), _p(x_in), _p(x_out), _p(logits), n_cand, _p(offsets), _p(group_ids),
        _p(timestamps), B, T, attn_scale, dtype_code(x_in.dtype), _p(ws), ws.numel(), _p(head_ws), head_ws.numel(),
        ctypes.byref(h)))
    return StackGraph(h.value, (x_in, x_out, logits, offsets, group_ids, timestamps, ws, head_ws))
