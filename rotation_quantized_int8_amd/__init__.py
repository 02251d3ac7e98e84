"""INT8ConvRot linear layer on AMD MI355X (gfx950): Python binding.

A thin ctypes layer over ``libconvrot.so`` (C ABI in ``include/convrot.h``).
It only marshals arguments: PyTorch tensors supply device memory and the
current stream; every step of the layer runs in the library's HIP kernels.
There is no CPU fallback: if the library is missing or the device is not
gfx950, the calls raise.

Functions mirror the C entry points:
  quantize_weights, linear_w8a8, linear_w8a8_noalloc, linear_w8a8_ex, linear_w8a16, linear_w8a16_rs,
  linear_dequant, dequantize_weights, act_quant, act_rotate_f16, act_rotate_scaled,
  gemm_i8_i32, gemm_i8_f16, gemm_f16, workspace_bytes.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence, Tuple

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libconvrot.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG_DIR), "include", "convrot.h")

PATH_W8A8 = 0
PATH_W8A16 = 1
PATH_DEQUANT = 2
PATH_W8A16_RS = 3
DTYPE_F16 = 0
DTYPE_BF16 = 1
GROUP = 256
K_MAX = 131072
LORA_RANK_MAX = 64

_vp, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


class _Lora(ctypes.Structure):
    _fields_ = [("down", _vp), ("up", _vp), ("rank", _i64), ("scale", _f32)]


_SIGNATURES = {
    "convrot_abi_version": (ctypes.c_int, []),
    "convrot_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "convrot_workspace_bytes": (_sz, [ctypes.c_int, _i64, _i64, _i64, _i64]),
    "convrot_quantize_weights": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "convrot_linear_w8a8": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "convrot_linear_w8a8_noalloc": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp]),
    "convrot_linear_w8a8_ex": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i64, _vp, ctypes.POINTER(_Lora),
                                              _vp, _vp, _vp, _sz, _vp]),
    "convrot_linear_w8a16": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i64, _vp,
                                            ctypes.POINTER(_Lora), _vp, _vp, _sz, _vp]),
    "convrot_linear_dequant": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "convrot_dequantize_weights": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "convrot_linear_w8a16_rs": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp,
                                               ctypes.c_int, _vp, _sz, _vp]),
    "convrot_act_rotate_scaled": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _vp]),
    "convrot_act_quant": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "convrot_act_rotate_f16": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "convrot_gemm_i8_i32": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "convrot_gemm_i8_f16": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "convrot_gemm_f16": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp]),
}

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m rotation_quantized_int8_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> Sequence[str]:
    """Names of the functions declared in include/convrot.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(convrot_[a-z0-9_]+)\s*\(", text)))


class ConvRotError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().convrot_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != 0:
        raise ConvRotError(status, where)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _prep(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    t = t.contiguous()
    if t.data_ptr() % 16:
        t = t.clone()  # fresh allocation: 16-byte aligned
    return t


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def workspace_bytes(path: int, M: int, N: int, K: int, lora_rank: int = 0) -> int:
    v = lib().convrot_workspace_bytes(path, M, N, K, lora_rank)
    if v == ctypes.c_size_t(-1).value:
        raise ValueError(f"invalid sizes for workspace: M={M} N={N} K={K} rank={lora_rank}")
    return v


def _workspace(path: int, M: int, N: int, K: int, rank: int, device,
               workspace: Optional[torch.Tensor]) -> Tuple[torch.Tensor, int]:
    need = workspace_bytes(path, M, N, K, rank)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor")
    return workspace, workspace.numel()


def quantize_weights(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Offline: W fp32 [N, K] -> (Q_W int8 [N, K], s_W fp32 [N])."""
    w = _prep(w, torch.float32, "W")
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.int8, device=w.device)
    s = torch.empty((N,), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        _check(lib().convrot_quantize_weights(_ptr(w), N, K, _ptr(q), _ptr(s), _stream(w)),
               "convrot_quantize_weights")
    return q, s


def _flatten(x: torch.Tensor):
    if x.dim() == 0:
        raise ValueError("input must have at least one dimension")
    lead = x.shape[:-1]
    rows = 1
    for d in lead:
        rows *= d
    return x.reshape(rows, x.shape[-1]), lead   # explicit rows: K may be 0


def linear_w8a8(x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor,
                bias: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W8A8 ConvRot linear: x fp16 [..., K] -> fp16 [..., N]."""
    x2, lead = _flatten(_prep(x, torch.float16, "x"))
    q_w = _prep(q_w, torch.int8, "Q_W")
    s_w = _prep(s_w, torch.float32, "s_W")
    bias = None if bias is None else _prep(bias, torch.float32, "bias")
    M, K = x2.shape
    N = q_w.shape[0]
    if q_w.shape[1] != K:
        raise ValueError(f"Q_W has K={q_w.shape[1]}, x has K={K}")
    y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    ws, nbytes = _workspace(PATH_W8A8, M, N, K, 0, x.device, workspace)
    with torch.cuda.device(x.device):
        _check(lib().convrot_linear_w8a8(_ptr(x2), M, K, _ptr(q_w), _ptr(s_w), N, _ptr(bias),
                                         _ptr(y), _ptr(ws), nbytes, _stream(x2)),
               "convrot_linear_w8a8")
    return y.reshape(*lead, N)


def linear_w8a8_noalloc(x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor,
                        bias: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W8A8 ConvRot linear through the allocation-free entry point (the
    library's fixed per-GPU scratch instead of a workspace).  With ``out``
    (fp16 [M, N], contiguous, 16-byte aligned) the call allocates nothing."""
    x2, lead = _flatten(_prep(x, torch.float16, "x"))
    q_w = _prep(q_w, torch.int8, "Q_W")
    s_w = _prep(s_w, torch.float32, "s_W")
    bias = None if bias is None else _prep(bias, torch.float32, "bias")
    M, K = x2.shape
    N = q_w.shape[0]
    if q_w.shape[1] != K:
        raise ValueError(f"Q_W has K={q_w.shape[1]}, x has K={K}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    elif out.dtype != torch.float16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp16 tensor [M, N]")
    with torch.cuda.device(x.device):
        _check(lib().convrot_linear_w8a8_noalloc(_ptr(x2), M, K, _ptr(q_w), _ptr(s_w), N, _ptr(bias),
                                                 _ptr(out), _stream(x2)),
               "convrot_linear_w8a8_noalloc")
    return out.reshape(*lead, N)


def _lora_args(lora, N: int, K: int):
    """(ctypes struct or None, rank, tensors to keep alive) for (down, up, scale)."""
    if lora is None:
        return None, 0, None
    down, up, scale = lora
    down = _prep(down, torch.float32, "lora_down")
    up = _prep(up, torch.float32, "lora_up")
    rank = down.shape[0]
    if down.shape != (rank, K) or up.shape != (N, rank):
        raise ValueError("lora_down must be [R, K] and lora_up [N, R]")
    return _Lora(down.data_ptr(), up.data_ptr(), rank, float(scale)), rank, (down, up)


def linear_w8a8_ex(x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor,
                   bias: Optional[torch.Tensor] = None,
                   lora: Optional[Tuple[torch.Tensor, torch.Tensor, float]] = None,
                   residual: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W8A8 ConvRot linear with optional bias, unmerged LoRA (down, up, scale)
    and fp16 residual [..., N] added to the output; ``out`` (contiguous fp16
    [..., N]) receives the result and may be ``residual`` itself."""
    x2, lead = _flatten(_prep(x, torch.float16, "x"))
    q_w = _prep(q_w, torch.int8, "Q_W")
    s_w = _prep(s_w, torch.float32, "s_W")
    bias = None if bias is None else _prep(bias, torch.float32, "bias")
    M, K = x2.shape
    N = q_w.shape[0]
    if q_w.shape[1] != K:
        raise ValueError(f"Q_W has K={q_w.shape[1]}, x has K={K}")
    lora_struct, rank, keep = _lora_args(lora, N, K)
    if out is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        if out.dtype != torch.float16 or not out.is_contiguous() or out.numel() != M * N:
            raise ValueError("out must be a contiguous fp16 tensor with M * N elements")
        y = out.view(M, N)
    res = None
    if residual is not None:
        if residual.numel() != M * N:
            raise ValueError("residual must have M * N elements")
        if out is not None and residual.data_ptr() == out.data_ptr() and residual.is_contiguous():
            res = y   # in-place residual update
        else:
            res = _prep(residual, torch.float16, "residual").view(M, N)
    ws, nbytes = _workspace(PATH_W8A8, M, N, K, rank, x.device, workspace)
    with torch.cuda.device(x.device):
        _check(lib().convrot_linear_w8a8_ex(
            _ptr(x2), M, K, _ptr(q_w), _ptr(s_w), N, _ptr(bias),
            ctypes.byref(lora_struct) if lora_struct is not None else None,
            _ptr(res), _ptr(y), _ptr(ws), nbytes, _stream(x2)), "convrot_linear_w8a8_ex")
    del keep
    return y.reshape(*lead, N)


def linear_w8a16(x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor,
                 bias: Optional[torch.Tensor] = None,
                 lora: Optional[Tuple[torch.Tensor, torch.Tensor, float]] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Weight-only ConvRot linear with optional unmerged LoRA (down, up, scale)."""
    x2, lead = _flatten(_prep(x, torch.float16, "x"))
    q_w = _prep(q_w, torch.int8, "Q_W")
    s_w = _prep(s_w, torch.float32, "s_W")
    bias = None if bias is None else _prep(bias, torch.float32, "bias")
    M, K = x2.shape
    N = q_w.shape[0]
    if q_w.shape[1] != K:
        raise ValueError(f"Q_W has K={q_w.shape[1]}, x has K={K}")
    lora_struct, rank, keep = _lora_args(lora, N, K)
    y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    ws, nbytes = _workspace(PATH_W8A16, M, N, K, rank, x.device, workspace)
    with torch.cuda.device(x.device):
        _check(lib().convrot_linear_w8a16(
            _ptr(x2), M, K, _ptr(q_w), _ptr(s_w), N, _ptr(bias),
            ctypes.byref(lora_struct) if lora_struct is not None else None,
            _ptr(y), _ptr(ws), nbytes, _stream(x2)), "convrot_linear_w8a16")
    del keep
    return y.reshape(*lead, N)


def dequantize_weights(q_w: torch.Tensor, s_w: torch.Tensor) -> torch.Tensor:
    """Q_W int8 [N, K], s_W fp32 [N] -> fp16((Q_W * s_W) H) [N, K] (un-rotated)."""
    q_w = _prep(q_w, torch.int8, "Q_W")
    s_w = _prep(s_w, torch.float32, "s_W")
    N, K = q_w.shape
    out = torch.empty((N, K), dtype=torch.float16, device=q_w.device)
    with torch.cuda.device(q_w.device):
        _check(lib().convrot_dequantize_weights(_ptr(q_w), _ptr(s_w), N, K, _ptr(out), _stream(q_w)),
               "convrot_dequantize_weights")
    return out


def linear_dequant(x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor,
                   bias: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dequantise-every-call baseline: fp16(x W_deq^T [+ bias]), W_deq rebuilt each call."""
    x2, lead = _flatten(_prep(x, torch.float16, "x"))
    q_w = _prep(q_w, torch.int8, "Q_W")
    s_w = _prep(s_w, torch.float32, "s_W")
    bias = None if bias is None else _prep(bias, torch.float32, "bias")
    M, K = x2.shape
    N = q_w.shape[0]
    if q_w.shape[1] != K:
        raise ValueError(f"Q_W has K={q_w.shape[1]}, x has K={K}")
    y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    ws, nbytes = _workspace(PATH_DEQUANT, M, N, K, 0, x.device, workspace)
    with torch.cuda.device(x.device):
        _check(lib().convrot_linear_dequant(_ptr(x2), M, K, _ptr(q_w), _ptr(s_w), N, _ptr(bias),
                                            _ptr(y), _ptr(ws), nbytes, _stream(x2)),
               "convrot_linear_dequant")
    return y.reshape(*lead, N)


_DTYPES = {torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16}


def _prep16(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be a float16 or bfloat16 tensor")
    return _prep(t, t.dtype, name)


def linear_w8a16_rs(x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor,
                    bias: Optional[torch.Tensor] = None, residual: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Range-safe weight-only linear: x fp16/bf16 [..., K] -> out_dtype [..., N]
    (default x.dtype), optional bias and residual (out_dtype, may be ``out``)."""
    x2, lead = _flatten(_prep16(x, "x"))
    out_dtype = out_dtype or x.dtype
    if out_dtype not in _DTYPES:
        raise TypeError("out_dtype must be float16 or bfloat16")
    q_w = _prep(q_w, torch.int8, "Q_W")
    s_w = _prep(s_w, torch.float32, "s_W")
    bias = None if bias is None else _prep(bias, torch.float32, "bias")
    M, K = x2.shape
    N = q_w.shape[0]
    if q_w.shape[1] != K:
        raise ValueError(f"Q_W has K={q_w.shape[1]}, x has K={K}")
    if out is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        if out.dtype != out_dtype or not out.is_contiguous() or out.numel() != M * N:
            raise ValueError("out must be a contiguous tensor of out_dtype with M * N elements")
        y = out.view(M, N)
    res = None
    if residual is not None:
        if residual.dtype != out_dtype or residual.numel() != M * N:
            raise ValueError("residual must have out_dtype and M * N elements")
        if out is not None and residual.data_ptr() == out.data_ptr() and residual.is_contiguous():
            res = y
        else:
            res = _prep(residual, out_dtype, "residual").view(M, N)
    ws, nbytes = _workspace(PATH_W8A16_RS, M, N, K, 0, x.device, workspace)
    with torch.cuda.device(x.device):
        _check(lib().convrot_linear_w8a16_rs(_ptr(x2), _DTYPES[x2.dtype], M, K, _ptr(q_w), _ptr(s_w), N,
                                             _ptr(bias), _ptr(res), _ptr(y), _DTYPES[out_dtype], _ptr(ws),
                                             nbytes, _stream(x2)), "convrot_linear_w8a16_rs")
    return y.reshape(*lead, N)


def act_rotate_scaled(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Range-safe prologue alone: x fp16/bf16 [M, K] -> (fp16(x H 2^-e) [M, K], e int32 [M])."""
    x = _prep16(x, "x")
    M, K = x.shape
    out = torch.empty((M, K), dtype=torch.float16, device=x.device)
    e = torch.empty((M,), dtype=torch.int32, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().convrot_act_rotate_scaled(_ptr(x), _DTYPES[x.dtype], M, K, _ptr(out), _ptr(e), _stream(x)),
               "convrot_act_rotate_scaled")
    return out, e


def act_quant(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Prologue alone: x fp16 [M, K] -> (Q_X int8 [M, K], s_X fp32 [M])."""
    x = _prep(x, torch.float16, "x")
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    s = torch.empty((M,), dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().convrot_act_quant(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(x)),
               "convrot_act_quant")
    return q, s


def act_rotate_f16(x: torch.Tensor) -> torch.Tensor:
    """Weight-only prologue alone: x fp16 [M, K] -> fp16(x H) [M, K]."""
    x = _prep(x, torch.float16, "x")
    M, K = x.shape
    out = torch.empty_like(x)
    with torch.cuda.device(x.device):
        _check(lib().convrot_act_rotate_f16(_ptr(x), M, K, _ptr(out), _stream(x)),
               "convrot_act_rotate_f16")
    return out


def gemm_i8_i32(q_x: torch.Tensor, q_w: torch.Tensor) -> torch.Tensor:
    """A int32 [M, N] = Q_X Q_W^T."""
    q_x = _prep(q_x, torch.int8, "Q_X")
    q_w = _prep(q_w, torch.int8, "Q_W")
    M, K = q_x.shape
    N = q_w.shape[0]
    if q_w.shape[1] != K:
        raise ValueError("K mismatch")
    a = torch.empty((M, N), dtype=torch.int32, device=q_x.device)
    with torch.cuda.device(q_x.device):
        _check(lib().convrot_gemm_i8_i32(_ptr(q_x), _ptr(q_w), M, N, K, _ptr(a), _stream(q_x)),
               "convrot_gemm_i8_i32")
    return a


def gemm_i8_f16(q_x: torch.Tensor, s_x: torch.Tensor, q_w: torch.Tensor, s_w: torch.Tensor,
                bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y fp16 [M, N] = fp16(fp32(Q_X Q_W^T) * fp32(s_X s_W) [+ bias])."""
    q_x = _prep(q_x, torch.int8, "Q_X")
    s_x = _prep(s_x, torch.float32, "s_X")
    q_w = _prep(q_w, torch.int8, "Q_W")
    s_w = _prep(s_w, torch.float32, "s_W")
    bias = None if bias is None else _prep(bias, torch.float32, "bias")
    M, K = q_x.shape
    N = q_w.shape[0]
    if q_w.shape[1] != K:
        raise ValueError("K mismatch")
    y = torch.empty((M, N), dtype=torch.float16, device=q_x.device)
    with torch.cuda.device(q_x.device):
        _check(lib().convrot_gemm_i8_f16(_ptr(q_x), _ptr(s_x), _ptr(q_w), _ptr(s_w), _ptr(bias),
                                         M, N, K, _ptr(y), _stream(q_x)), "convrot_gemm_i8_f16")
    return y


def gemm_f16(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """fp16 baseline: Y fp16 [M, N] = X [M, K] . W [N, K]^T (fp32 accumulation)."""
    x = _prep(x, torch.float16, "x")
    w = _prep(w, torch.float16, "W")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("K mismatch")
    y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().convrot_gemm_f16(_ptr(x), _ptr(w), M, N, K, _ptr(y), _stream(x)),
               "convrot_gemm_f16")
    return y
