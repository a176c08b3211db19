"""Python binding of libttr.so, the MI355X (gfx950) TTR hybrid-attention library.

Argument marshalling only: every function checks tensor placement, dtype and
contiguity, allocates outputs/workspace with torch, and calls the C ABI of
include/ttr.h with raw device pointers on torch's current HIP stream. All
arithmetic runs in the library's HIP kernels; nothing falls back to the CPU.

The method (web pages, by title and section): "Flux2TTRTrainer", "How the
distillation works" (linear kernel branch + exact softmax over landmark tokens,
blended by a bounded weight); "NNT Define Linear Attention", "The inputs" and
"How it works" (elu(x) + 1 feature map, eps, causal variant, K'^T V first).
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional, Tuple

import torch

__all__ = [
    "TTRError", "load_library", "library_path", "exported_symbols", "Dims", "FMAPS",
    "feature_map", "kv_reduce", "apply", "landmark_attn", "blend", "causal_scan",
    "hybrid_forward", "hybrid_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "workspace_bytes", "status_string", "version",
    "TTR_FP32", "TTR_BF16",
]

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HEADER = os.path.join(ROOT, "include", "ttr.h")
TTR_FP32, TTR_BF16 = 0, 1


def library_path() -> str:
    return os.path.join(HERE, "libttr.so")


class TTRError(RuntimeError):
    """A non-zero ttr_status returned by the library."""

    def __init__(self, status: int, where: str, msg: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        extra = f" (hipError {hip_error})" if status == 7 else ""
        super().__init__(f"{where}: status {status}: {msg}{extra}")


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("D", ctypes.c_int32), ("F", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("fmap", ctypes.c_int32)]


class LayerDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("E", ctypes.c_int32),
                ("H", ctypes.c_int32), ("dtype", ctypes.c_int32), ("fmap", ctypes.c_int32)]


class ReplayStats(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("first_id", ctypes.c_int64), ("pushed", ctypes.c_int64),
                ("evicted", ctypes.c_int64), ("bytes_used", ctypes.c_size_t), ("budget_bytes", ctypes.c_size_t),
                ("max_sample_bytes", ctypes.c_size_t), ("ring_bytes", ctypes.c_size_t)]


class GateConfig(ctypes.Structure):
    _fields_ = [("ema_rate", ctypes.c_double), ("threshold_on", ctypes.c_double),
                ("threshold_off", ctypes.c_double), ("min_updates", ctypes.c_int32)]


class GateState(ctypes.Structure):
    _fields_ = [("ema", ctypes.c_double), ("updates", ctypes.c_int32), ("ready", ctypes.c_int32)]


# feature maps (ttr_fmap): elu(x) + 1, relu, softmax over the features
FMAPS = {"elu1": 0, "relu": 1, "softmax": 2}


def _fmap(name: str) -> int:
    if name not in FMAPS:
        raise ValueError(f"feature map must be one of {sorted(FMAPS)}")
    return FMAPS[name]


_P = ctypes.c_void_p
_SIGS = {
    "ttr_feature_map": [Dims, _P, _P, _P, _P, _P],
    "ttr_kv_reduce": [Dims, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "ttr_apply": [Dims, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P],
    "ttr_landmark_attn": [Dims, _P, _P, _P, ctypes.c_int32, _P, _P],
    "ttr_blend": [Dims, _P, _P, _P, _P, _P],
    "ttr_causal_scan": [Dims, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P],
    "ttr_hybrid_forward": [Dims, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                           _P, _P, ctypes.c_size_t, _P],
    "ttr_hybrid_forward_noalloc": [Dims, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                   _P, _P],
    "ttr_hybrid_backward": [Dims, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int32, _P, _P, _P, _P, _P,
                            ctypes.c_size_t, _P],
    "ttr_distill_step": [Dims, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                         ctypes.c_int32, _P, _P, ctypes.c_size_t, _P],
    "ttr_distill_step_rows": [Dims, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                              ctypes.c_float, ctypes.c_float, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P],
    "ttr_cosine_distance": [Dims, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "ttr_nnt_layer_forward": [LayerDims, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_int32,
                              _P, _P, ctypes.c_size_t, _P],
}

_lib = None


def load_library() -> ctypes.CDLL:
    """Load libttr.so once; raise loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m linear_hybrid_attention_amd.build` "
                          "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.ttr_workspace_bytes.argtypes = [Dims, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.ttr_workspace_bytes.restype = ctypes.c_size_t
    lib.ttr_distill_workspace_bytes.argtypes = [Dims, ctypes.c_int32, ctypes.c_int32]
    lib.ttr_distill_workspace_bytes.restype = ctypes.c_size_t
    lib.ttr_distill_rows_workspace_bytes.argtypes = [Dims, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.ttr_distill_rows_workspace_bytes.restype = ctypes.c_size_t
    lib.ttr_backward_workspace_bytes.argtypes = [Dims, ctypes.c_int32]
    lib.ttr_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.ttr_nnt_layer_workspace_bytes.argtypes = [LayerDims, ctypes.c_int32]
    lib.ttr_nnt_layer_workspace_bytes.restype = ctypes.c_size_t
    lib.ttr_cosine_workspace_bytes.argtypes = [Dims]
    lib.ttr_cosine_workspace_bytes.restype = ctypes.c_size_t
    lib.ttr_gate_update.argtypes = [ctypes.POINTER(GateConfig), ctypes.POINTER(GateState), ctypes.c_double]
    lib.ttr_gate_update.restype = ctypes.c_int
    lib.ttr_landmark_count.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.c_int32, ctypes.c_int32]
    lib.ttr_landmark_count.restype = ctypes.c_int32
    lib.ttr_replay_sample_bytes.argtypes = [Dims, ctypes.c_int32, ctypes.c_int32]
    lib.ttr_replay_sample_bytes.restype = ctypes.c_size_t
    lib.ttr_replay_create.argtypes = [ctypes.c_size_t, ctypes.c_size_t, ctypes.POINTER(ctypes.c_void_p)]
    lib.ttr_replay_create.restype = ctypes.c_int
    lib.ttr_replay_destroy.argtypes = [_P]
    lib.ttr_replay_destroy.restype = None
    lib.ttr_replay_push.argtypes = [_P, Dims, ctypes.c_int32, _P, _P, _P, _P, _P, _P, ctypes.POINTER(ctypes.c_int64)]
    lib.ttr_replay_push.restype = ctypes.c_int
    lib.ttr_replay_wait_pushed.argtypes = [_P, _P]
    lib.ttr_replay_wait_pushed.restype = ctypes.c_int
    lib.ttr_replay_synchronize.argtypes = [_P]
    lib.ttr_replay_synchronize.restype = ctypes.c_int
    lib.ttr_replay_fetch.argtypes = [_P, ctypes.c_int64, _P, _P, _P, _P, _P, _P]
    lib.ttr_replay_fetch.restype = ctypes.c_int
    lib.ttr_replay_info.argtypes = [_P, ctypes.c_int64, ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_int32)]
    lib.ttr_replay_info.restype = ctypes.c_int
    lib.ttr_replay_get_stats.argtypes = [_P, ctypes.POINTER(ReplayStats)]
    lib.ttr_replay_get_stats.restype = ctypes.c_int
    lib.ttr_status_string.argtypes = [ctypes.c_int]
    lib.ttr_status_string.restype = ctypes.c_char_p
    lib.ttr_last_hip_error.argtypes = []
    lib.ttr_last_hip_error.restype = ctypes.c_int
    lib.ttr_set_stage_events.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.ttr_set_stage_events.restype = None
    lib.ttr_version.argtypes = []
    lib.ttr_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def exported_symbols() -> list:
    """Function names declared in include/ttr.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(ttr_\w+)\s*\(", text, flags=re.M)))


def status_string(st: int) -> str:
    return load_library().ttr_status_string(st).decode()


def version() -> str:
    return load_library().ttr_version().decode()


def _check(st: int, where: str) -> None:
    if st != 0:
        lib = load_library()
        raise TTRError(st, where, status_string(st), lib.ttr_last_hip_error())


_IO = {torch.float32: TTR_FP32, torch.bfloat16: TTR_BF16}


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype not in _IO:
        raise TypeError(f"IO tensors must be float32 or bfloat16, got {t.dtype}")
    return _IO[t.dtype]


def _dev(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dims(X: torch.Tensor, F: int, fmap: str = "elu1") -> Dims:
    if X.dim() != 4:
        raise ValueError("Q/K/V must be [B, H, N, D]")
    B, H, N, D = X.shape
    return Dims(B, H, N, D, F, _io_dtype(X), _fmap(fmap))


def _feat_dim(X: torch.Tensor, W: Optional[torch.Tensor]) -> int:
    return int(W.shape[2]) if W is not None else int(X.shape[3])


def workspace_bytes(B: int, H: int, N: int, D: int, F: int, dtype: int, L: int = 0, causal: bool = False,
                    chunk: int = 0, fmap: str = "elu1") -> int:
    return int(load_library().ttr_workspace_bytes(Dims(B, H, N, D, F, dtype, _fmap(fmap)), L, int(causal), chunk))


def _workspace(d: Dims, nbytes: int, like: torch.Tensor, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    return ws, ws.numel() * ws.element_size()


def feature_map(X: torch.Tensor, W: Optional[torch.Tensor] = None, b: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, fmap: str = "elu1") -> torch.Tensor:
    """phi(X) = map(X W_h + b_h) (elu + 1, relu or softmax), [B,H,N,F] in X's dtype (ttr_feature_map)."""
    lib = load_library()
    F = _feat_dim(X, W)
    d = _dims(X, F, fmap)
    if out is None:
        out = torch.empty((d.B, d.H, d.N, F), dtype=X.dtype, device=X.device)
    st = lib.ttr_feature_map(d, _dev(X, "X"), _dev(W, "W", X.dtype), _dev(b, "b", torch.float32),
                             _dev(out, "phi", X.dtype), _stream(X))
    _check(st, "ttr_feature_map")
    return out


def kv_reduce(K: torch.Tensor, V: torch.Tensor, W: Optional[torch.Tensor] = None,
              b: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
              fmap: str = "elu1") -> Tuple[torch.Tensor, torch.Tensor]:
    """KV = phi(K)^T V [B,H,F,D] and ksum [B,H,F], both fp32 (ttr_kv_reduce)."""
    lib = load_library()
    F = _feat_dim(K, W)
    d = _dims(K, F, fmap)
    KV = torch.empty((d.B, d.H, F, d.D), dtype=torch.float32, device=K.device)
    ksum = torch.empty((d.B, d.H, F), dtype=torch.float32, device=K.device)
    ws, wsb = _workspace(d, lib.ttr_workspace_bytes(d, 0, 0, 0), K, ws)  # the documented bound
    st = lib.ttr_kv_reduce(d, _dev(K, "K"), _dev(V, "V", K.dtype), _dev(W, "W", K.dtype),
                           _dev(b, "b", torch.float32), KV.data_ptr(), ksum.data_ptr(),
                           None if ws is None else ws.data_ptr(), wsb, _stream(K))
    _check(st, "ttr_kv_reduce")
    return KV, ksum


def apply(Q: torch.Tensor, W: Optional[torch.Tensor], b: Optional[torch.Tensor], KV: torch.Tensor,
          ksum: torch.Tensor, eps: float = 1e-6, fmap: str = "elu1") -> torch.Tensor:
    """out_lin = phi(Q) KV / (phi(Q) . ksum + eps), fp32 [B,H,N,D] (ttr_apply)."""
    lib = load_library()
    d = _dims(Q, _feat_dim(Q, W), fmap)
    out = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    st = lib.ttr_apply(d, _dev(Q, "Q"), _dev(W, "W", Q.dtype), _dev(b, "b", torch.float32),
                       _dev(KV, "KV", torch.float32), _dev(ksum, "ksum", torch.float32), float(eps),
                       out.data_ptr(), _stream(Q))
    _check(st, "ttr_apply")
    return out


def landmark_attn(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, L: int) -> torch.Tensor:
    """Exact softmax over L strided landmarks, fp32 [B,H,N,D] (ttr_landmark_attn)."""
    lib = load_library()
    d = _dims(Q, Q.shape[3])
    out = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    st = lib.ttr_landmark_attn(d, _dev(Q, "Q"), _dev(K, "K", Q.dtype), _dev(V, "V", Q.dtype), int(L),
                               out.data_ptr(), _stream(Q))
    _check(st, "ttr_landmark_attn")
    return out


def blend(out_lin: torch.Tensor, out_lm: torch.Tensor, g: torch.Tensor, dtype=torch.bfloat16) -> torch.Tensor:
    """out = sigmoid(g_h) out_lin + (1 - sigmoid(g_h)) out_lm in `dtype` (ttr_blend)."""
    lib = load_library()
    B, H, N, D = out_lin.shape
    d = Dims(B, H, N, D, D, _IO[dtype], 0)
    out = torch.empty(out_lin.shape, dtype=dtype, device=out_lin.device)
    st = lib.ttr_blend(d, _dev(out_lin, "out_lin", torch.float32), _dev(out_lm, "out_lm", torch.float32),
                       _dev(g, "g", torch.float32), out.data_ptr(), _stream(out_lin))
    _check(st, "ttr_blend")
    return out


def causal_scan(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, b: Optional[torch.Tensor] = None,
                eps: float = 1e-6, chunk: int = 128, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, fmap: str = "elu1") -> torch.Tensor:
    """Causal linear attention, chunked prefix scan, [B,H,N,D] in Q's dtype (ttr_causal_scan)."""
    lib = load_library()
    d = _dims(Q, Q.shape[3], fmap)
    if out is None:
        out = torch.empty_like(Q)
    need = lib.ttr_workspace_bytes(d, 0, 1, int(chunk))
    ws, wsb = _workspace(d, need, Q, ws)
    st = lib.ttr_causal_scan(d, _dev(Q, "Q"), _dev(K, "K", Q.dtype), _dev(V, "V", Q.dtype), None,
                             _dev(b, "b", torch.float32), float(eps), int(chunk), _dev(out, "out", Q.dtype),
                             None if ws is None else ws.data_ptr(), wsb, _stream(Q))
    _check(st, "ttr_causal_scan")
    return out


def hybrid_forward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, W: Optional[torch.Tensor],
                   b: Optional[torch.Tensor], g: Optional[torch.Tensor], eps: float = 1e-6, L: int = 0,
                   causal: bool = False, out: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, fmap: str = "elu1", chunk: int = 0) -> torch.Tensor:
    """The whole TTR forward, [B,H,N,D] in Q's dtype (ttr_hybrid_forward).
    With causal, chunk (64, 128 or 256) names the scan's chunk; 0 takes the default."""
    lib = load_library()
    d = _dims(Q, _feat_dim(Q, W), fmap)
    if out is None:
        out = torch.empty_like(Q)
    causal = (int(chunk) if chunk else 1) if causal else 0
    need = lib.ttr_workspace_bytes(d, int(L), causal, 0)
    ws, wsb = _workspace(d, need, Q, ws)
    st = lib.ttr_hybrid_forward(d, _dev(Q, "Q"), _dev(K, "K", Q.dtype), _dev(V, "V", Q.dtype),
                                _dev(W, "W", Q.dtype), _dev(b, "b", torch.float32), _dev(g, "g", torch.float32),
                                float(eps), int(L), int(causal), _dev(out, "out", Q.dtype),
                                None if ws is None else ws.data_ptr(), wsb, _stream(Q))
    _check(st, "ttr_hybrid_forward")
    return out


def hybrid_forward_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, W: Optional[torch.Tensor],
                           b: Optional[torch.Tensor], g: Optional[torch.Tensor], eps: float = 1e-6, L: int = 0,
                           causal: bool = False, out: Optional[torch.Tensor] = None, fmap: str = "elu1",
                           chunk: int = 0) -> torch.Tensor:
    """hybrid_forward with the library's fixed per-GPU workspace
    (ttr_hybrid_forward_noalloc): no workspace argument, no allocation by the
    call (out, when given, is written in place)."""
    lib = load_library()
    d = _dims(Q, _feat_dim(Q, W), fmap)
    if out is None:
        out = torch.empty_like(Q)
    causal = (int(chunk) if chunk else 1) if causal else 0
    st = lib.ttr_hybrid_forward_noalloc(d, _dev(Q, "Q"), _dev(K, "K", Q.dtype), _dev(V, "V", Q.dtype),
                                        _dev(W, "W", Q.dtype), _dev(b, "b", torch.float32),
                                        _dev(g, "g", torch.float32), float(eps), int(L), int(causal),
                                        _dev(out, "out", Q.dtype), _stream(Q))
    _check(st, "ttr_hybrid_forward_noalloc")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # TTR_NOALLOC_SCRATCH_BYTES


def nnt_layer_workspace_bytes(B: int, N: int, E: int, H: int, dtype: int, causal: bool = False,
                              fmap: str = "elu1") -> int:
    return int(load_library().ttr_nnt_layer_workspace_bytes(LayerDims(B, N, E, H, dtype, _fmap(fmap)), int(causal)))


def nnt_layer_forward(x: torch.Tensor, Wq: torch.Tensor, bq: Optional[torch.Tensor], Wk: torch.Tensor,
                      bk: Optional[torch.Tensor], Wv: torch.Tensor, bv: Optional[torch.Tensor], Wo: torch.Tensor,
                      bo: Optional[torch.Tensor], H: int, eps: float = 1e-6, causal: bool = False,
                      fmap: str = "elu1", out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """NNT linear-attention layer forward, x [B, N, E] -> [B, N, E] in x's dtype
    (ttr_nnt_layer_forward). W* are [E, E] (x @ W), b* are [E] float32 or None."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [B, N, E]")
    B, N, E = x.shape
    d = LayerDims(B, N, E, int(H), _io_dtype(x), _fmap(fmap))
    if out is None:
        out = torch.empty_like(x)
    need = lib.ttr_nnt_layer_workspace_bytes(d, int(causal))
    if need == 0:
        raise TTRError(2, "ttr_nnt_layer_forward", "invalid layer shape")
    ws, wsb = _workspace(d, need, x, ws)
    f32 = torch.float32
    st = lib.ttr_nnt_layer_forward(d, _dev(x, "x"), _dev(Wq, "Wq", x.dtype), _dev(bq, "bq", f32),
                                   _dev(Wk, "Wk", x.dtype), _dev(bk, "bk", f32), _dev(Wv, "Wv", x.dtype),
                                   _dev(bv, "bv", f32), _dev(Wo, "Wo", x.dtype), _dev(bo, "bo", f32), float(eps),
                                   int(causal), _dev(out, "out", x.dtype), None if ws is None else ws.data_ptr(), wsb,
                                   _stream(x))
    _check(st, "ttr_nnt_layer_forward")
    return out


def hybrid_backward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, W: torch.Tensor,
                    b: Optional[torch.Tensor], g: Optional[torch.Tensor], eps: float, L: int, dout: torch.Tensor,
                    ws: Optional[torch.Tensor] = None):
    """Gradients (dW [H,D,F], db [H,F], dg [H], float32) of the hybrid forward for
    dLoss/dout = dout (float32 [B,H,N,D]) (ttr_hybrid_backward)."""
    lib = load_library()
    d = _dims(Q, _feat_dim(Q, W))
    B, H, N, D = Q.shape
    F = d.F
    dW = torch.empty((H, D, F), dtype=torch.float32, device=Q.device)
    db = torch.empty((H, F), dtype=torch.float32, device=Q.device)
    dg = torch.empty((H,), dtype=torch.float32, device=Q.device)
    need = lib.ttr_backward_workspace_bytes(d, int(L))
    if need == 0:
        raise TTRError(2, "ttr_hybrid_backward", "invalid shape for the backward")
    ws, wsb = _workspace(d, need, Q, ws)
    st = lib.ttr_hybrid_backward(d, _dev(Q, "Q"), _dev(K, "K", Q.dtype), _dev(V, "V", Q.dtype),
                                 _dev(W, "W", Q.dtype), _dev(b, "b", torch.float32), _dev(g, "g", torch.float32),
                                 float(eps), int(L), _dev(dout, "dout", torch.float32), _dev(dW, "dW"), _dev(db, "db"),
                                 _dev(dg, "dg"), None if ws is None else ws.data_ptr(), wsb, _stream(Q))
    _check(st, "ttr_hybrid_backward")
    return dW, db, dg


class DistillState:
    """fp32 master parameters and Adam moments of one TTR layer for ttr_distill_step."""

    def __init__(self, W: torch.Tensor, b: torch.Tensor, g: torch.Tensor, s: Optional[torch.Tensor] = None):
        f32 = torch.float32
        self.W = W.detach().to(f32).contiguous().clone()
        self.b = b.detach().to(f32).contiguous().clone()
        self.g = g.detach().to(f32).contiguous().clone()
        self.s = torch.zeros(2, dtype=f32, device=W.device) if s is None else s.detach().to(f32).contiguous().clone()
        n = self.W.numel() + self.b.numel() + self.g.numel() + 2
        self.moments = torch.zeros(2 * n, dtype=f32, device=W.device)
        self.step = 0


def distill_step(state: DistillState, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, L: int, lr: float,
                 eps: float = 1e-6, teacher: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """One distillation step; updates ``state`` in place and returns the device
    tensor [loss, huber, 1 - cos] before the update. Q may hold fewer query
    rows than K and V (a replay sample): then ttr_distill_step_rows, with
    ``teacher`` (if given) the teacher's rows for those queries; otherwise
    ttr_distill_step."""
    lib = load_library()
    if Q.dim() != 4 or K.dim() != 4 or Q.shape[:2] != K.shape[:2] or Q.shape[3] != K.shape[3]:
        raise ValueError("Q must be [B, H, Nq, D] with K, V [B, H, N, D]")
    d = _dims(K, int(state.W.shape[2]))
    nq = int(Q.shape[2])
    rows = nq != d.N
    need = (lib.ttr_distill_rows_workspace_bytes(d, nq, int(L), int(teacher is None)) if rows else
            lib.ttr_distill_workspace_bytes(d, int(L), int(teacher is None)))
    where = "ttr_distill_step_rows" if rows else "ttr_distill_step"
    if need == 0:
        raise TTRError(2, where, "invalid shape for the distillation step")
    ws, wsb = _workspace(d, need, Q, ws)
    loss = torch.empty(3, dtype=torch.float32, device=Q.device)
    state.step += 1
    args = (_dev(Q, "Q", K.dtype), _dev(K, "K"), _dev(V, "V", K.dtype), _dev(teacher, "teacher", torch.float32),
            _dev(state.W, "W"), _dev(state.b, "b"), _dev(state.g, "g"), _dev(state.s, "s"),
            _dev(state.moments, "moments"), state.step, float(lr), float(eps), int(L), _dev(loss, "loss"),
            None if ws is None else ws.data_ptr(), wsb, _stream(Q))
    st = lib.ttr_distill_step_rows(d, nq, *args) if rows else lib.ttr_distill_step(d, *args)
    if st != 0:
        state.step -= 1
    _check(st, where)
    return loss


def cosine_distance(student: torch.Tensor, teacher: torch.Tensor, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mean over rows of 1 - cos(student_row, teacher_row), [B,H,N,D] in the IO dtype
    (ttr_cosine_distance); returns a one-element float32 device tensor."""
    lib = load_library()
    d = _dims(student, int(student.shape[3]))
    out = torch.empty(1, dtype=torch.float32, device=student.device)
    ws, wsb = _workspace(d, lib.ttr_cosine_workspace_bytes(d), student, ws)
    st = lib.ttr_cosine_distance(d, _dev(student, "student"), _dev(teacher, "teacher", student.dtype),
                                 _dev(out, "out"), None if ws is None else ws.data_ptr(), wsb, _stream(student))
    _check(st, "ttr_cosine_distance")
    return out


class ReadinessGate:
    """Per-layer fail-closed readiness gate (ttr_gate_update): serve the student only while ``ready``."""

    def __init__(self, ema_rate: float = 0.9, threshold_on: float = 0.1, threshold_off: float = 0.15,
                 min_updates: int = 50):
        self.cfg = GateConfig(ema_rate, threshold_on, threshold_off, min_updates)
        self.state = GateState(0.0, 0, 0)

    def update(self, distance: float) -> bool:
        st = load_library().ttr_gate_update(ctypes.byref(self.cfg), ctypes.byref(self.state), float(distance))
        if st not in (0, 2):
            _check(st, "ttr_gate_update")
        if st == 2 and math.isfinite(distance):
            _check(st, "ttr_gate_update")
        return bool(self.state.ready)

    @property
    def ready(self) -> bool:
        return bool(self.state.ready)

    @property
    def ema(self) -> float:
        return float(self.state.ema)

    @property
    def updates(self) -> int:
        return int(self.state.updates)


def landmark_count(N: int, fraction: float, lmin: int, lmax: int) -> int:
    """Landmarks from the fraction/min/max knobs (ttr_landmark_count)."""
    L = load_library().ttr_landmark_count(int(N), float(fraction), int(lmin), int(lmax))
    if L < 0:
        raise ValueError("landmark_count: need N >= 0, fraction >= 0 and 0 <= lmin <= lmax")
    return int(L)


def replay_sample_bytes(B: int, H: int, N: int, D: int, dtype: torch.dtype, Nq: int, teacher: bool) -> int:
    """Budget footprint of one replay sample (ttr_replay_sample_bytes); 0 for an invalid shape."""
    d = Dims(B, H, N, D, D, _IO[dtype], 0)
    return int(load_library().ttr_replay_sample_bytes(d, int(Nq), 1 if teacher else 0))


class ReplayBuffer:
    """FIFO replay buffer in pinned host memory (ttr_replay_*): full K/V, the query
    rows at a strictly increasing index subset and, optionally, the teacher's fp32
    rows there. Pushes copy on the library's side stream; the pushed tensors are
    kept referenced here until wait_pushed() or synchronize() orders the current
    stream after the copies."""

    DEFAULT_BUDGET = 768 << 20

    def __init__(self, budget_bytes: int = DEFAULT_BUDGET, max_sample_bytes: Optional[int] = None):
        lib = load_library()
        if max_sample_bytes is None:
            max_sample_bytes = min(int(budget_bytes), 256 << 20)
        h = ctypes.c_void_p()
        _check(lib.ttr_replay_create(int(budget_bytes), int(max_sample_bytes), ctypes.byref(h)), "ttr_replay_create")
        self._h = h
        self._pending = []

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value is not None:
            load_library().ttr_replay_destroy(self._h)
            self._h = None
            self._pending = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def push(self, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, q_index,
             teacher: Optional[torch.Tensor] = None) -> int:
        """Push one sample (Q, K, V [B,H,N,D] IO dtype, teacher fp32 [B,H,N,D] or None,
        q_index host int32 indices); returns its id."""
        import numpy as np
        lib = load_library()
        d = _dims(K, int(K.shape[3]))
        idx = np.ascontiguousarray(np.asarray(q_index, dtype=np.int32).reshape(-1))
        if idx.size < 1:
            raise ValueError("q_index must hold at least one index")
        sid = ctypes.c_int64(-1)
        st = lib.ttr_replay_push(self._h, d, int(idx.size), _dev(Q, "Q", K.dtype), _dev(K, "K"), _dev(V, "V", K.dtype),
                                 _dev(teacher, "teacher", torch.float32), idx.ctypes.data, _stream(K),
                                 ctypes.byref(sid))
        _check(st, "ttr_replay_push")
        self._pending.extend(t for t in (Q, K, V, teacher) if t is not None)
        return int(sid.value)

    def wait_pushed(self) -> None:
        """Order the current stream's later work after every push's copies."""
        dev = torch.cuda.current_device()
        _check(load_library().ttr_replay_wait_pushed(self._h, torch.cuda.current_stream(dev).cuda_stream),
               "ttr_replay_wait_pushed")
        self._pending = []

    def synchronize(self) -> None:
        _check(load_library().ttr_replay_synchronize(self._h), "ttr_replay_synchronize")
        self._pending = []

    def info(self, sid: int):
        d, nq, ht = Dims(), ctypes.c_int32(), ctypes.c_int32()
        _check(load_library().ttr_replay_info(self._h, int(sid), ctypes.byref(d), ctypes.byref(nq), ctypes.byref(ht)),
               "ttr_replay_info")
        return d, int(nq.value), bool(ht.value)

    def fetch(self, sid: int, teacher: bool = True):
        """Copy sample ``sid`` back to the GPU on the current stream: returns
        (Q rows [B,H,Nq,D], K, V [B,H,N,D], teacher rows fp32 or None, q_index numpy int32)."""
        import numpy as np
        d, nq, has_t = self.info(sid)
        dt = torch.bfloat16 if d.dtype == TTR_BF16 else torch.float32
        dev = torch.device("cuda", torch.cuda.current_device())
        Qs = torch.empty(d.B, d.H, nq, d.D, dtype=dt, device=dev)
        K = torch.empty(d.B, d.H, d.N, d.D, dtype=dt, device=dev)
        V = torch.empty_like(K)
        T = torch.empty(d.B, d.H, nq, d.D, dtype=torch.float32, device=dev) if (teacher and has_t) else None
        idx = np.empty(nq, dtype=np.int32)
        st = load_library().ttr_replay_fetch(self._h, int(sid), Qs.data_ptr(), K.data_ptr(), V.data_ptr(),
                                             None if T is None else T.data_ptr(), idx.ctypes.data,
                                             torch.cuda.current_stream(dev).cuda_stream)
        _check(st, "ttr_replay_fetch")
        return Qs, K, V, T, idx

    def stats(self) -> ReplayStats:
        out = ReplayStats()
        _check(load_library().ttr_replay_get_stats(self._h, ctypes.byref(out)), "ttr_replay_get_stats")
        return out

    def ids(self):
        st = self.stats()
        return list(range(st.first_id, st.first_id + st.count)) if st.count else []
