"""ctypes binding of libattn_fwd.so (include/attn_fwd.h).

Argument marshalling only: every step of the attention computation runs in
the library's gfx950 kernels.  PyTorch supplies device memory and the current
stream.  If the library cannot be loaded the calls raise; there is no other
code path.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import numpy as np

import torch

from . import build as _build

_lock = threading.Lock()
_lib = None

ATTN_OK = 0
ATTN_DTYPE_BF16, ATTN_DTYPE_FP16 = 0, 1
VARLEN_RECORD_INTS = 8  # ints per tile record of attn_varlen_plan


class Strides(ctypes.Structure):
    """attn_strides: element strides (batch, head, row) of a [B, H, L, d] tensor."""
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong),
                ("row", ctypes.c_longlong)]


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_build.LIBRARY):
            _build.build()
        try:
            lib = ctypes.CDLL(_build.LIBRARY)
        except OSError as exc:  # pragma: no cover - exercised only when broken
            raise RuntimeError(f"cannot load the HIP attention library {_build.LIBRARY}: {exc}")
        vp, i = ctypes.c_void_p, ctypes.c_int
        lib.attn_fwd.restype = i
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, ctypes.c_float, vp]
        lib.attn_fwd_dbg.restype = i
        lib.attn_fwd_dbg.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                     ctypes.c_float, vp, ctypes.c_float, i, vp]
        lib.attn_fwd_ex.restype = i
        lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                    Strides, Strides, Strides, Strides, i, i, ctypes.c_float, vp]
        lib.attn_bwd.restype = i
        lib.attn_bwd.argtypes = [vp] * 10 + [i] * 8 + [ctypes.c_float, vp]
        lib.attn_bwd_ex.restype = i
        lib.attn_bwd_ex.argtypes = [vp] * 10 + [i] * 9 + [ctypes.c_float, vp]
        lib.attn_bwd_noalloc.restype = i
        lib.attn_bwd_noalloc.argtypes = [vp] * 9 + [i] * 8 + [ctypes.c_float, vp]
        lib.attn_split_keys.restype = i
        lib.attn_split_keys.argtypes = [i, i]
        lib.attn_fwd_split.restype = i
        lib.attn_fwd_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                       ctypes.c_float, i, vp]
        lib.attn_fwd_decode.restype = i
        lib.attn_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                        ctypes.c_float, i, vp]
        lib.attn_merge.restype = i
        lib.attn_merge.argtypes = [vp, vp, vp, vp, i, ctypes.c_longlong, i, vp]
        lib.attn_varlen_plan.restype = i
        lib.attn_varlen_plan.argtypes = [ctypes.POINTER(i), ctypes.POINTER(i), i, i, i, i,
                                         ctypes.POINTER(i), i, ctypes.POINTER(i)]
        lib.attn_fwd_varlen.restype = i
        lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                        ctypes.c_float, vp]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_status_string.argtypes = [i]
        lib.attn_abi_version.restype = i
        lib.attn_abi_version.argtypes = []
        _lib = lib
        return lib


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _load()


def status_string(rc: int) -> str:
    return _load().attn_status_string(int(rc)).decode()


def _check_inputs(q, k, v, dtypes=(torch.bfloat16,)):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in dtypes or t.dtype != q.dtype:
            raise TypeError(f"{name} must be one of {dtypes} (as q), got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, L, d] tensor")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    B, Hq, Lq, dqk = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if Bk != B or dk != dqk or tuple(v.shape[:3]) != (B, Hkv, Lk):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    return B, Hq, Hkv, Lq, Lk, dqk, v.shape[3]


def _require_device(t, device, name):
    """Caller-supplied buffers must live on the device of the inputs: the
    kernels write through their addresses."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _outputs(q, dv, out, lse):
    B, Hq, Lq, _ = q.shape
    if out is None:
        out = torch.empty((B, Hq, Lq, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    _require_device(out, q.device, "out")
    _require_device(lse, q.device, "lse")
    if out.shape != (B, Hq, Lq, dv) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [B, Hq, Lq, d_v] tensor")
    if lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, Hq, Lq] tensor")
    return out, lse


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
             stream=None):
    """O, lse = attention forward on the GPU (see include/attn_fwd.h).

    q [B,Hq,Lq,d_qk], k [B,Hkv,Lk,d_qk], v [B,Hkv,Lk,d_v]: contiguous bf16 on
    one GPU.  scale defaults to 1/sqrt(d_qk).  Enqueued on `stream` (default:
    torch's current stream on q's device)."""
    lib = _load()
    B, Hq, Hkv, Lq, Lk, dqk, dv = _check_inputs(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    out, lse = _outputs(q, dv, out, lse)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        rc = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), B, Hq, Hkv, Lq, Lk, dqk, dv, int(bool(causal)),
                          float(scale), s.cuda_stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_fwd failed: {status_string(rc)} (code {rc})")
    return out, lse


def attn_fwd_dbg(q, k, v, causal: bool = False, scale: float | None = None,
                 rescale_threshold: float = 8.0, rescale_count=None, out=None, lse=None,
                 stream=None, exp_mode: int = 0):
    """attn_fwd with the rescale threshold exposed; rescale_count, if given, is a
    zeroed int64 GPU tensor of one element that receives the event count.
    exp_mode 0 (v_exp_f32) is the only mode the library builds."""
    lib = _load()
    B, Hq, Hkv, Lq, Lk, dqk, dv = _check_inputs(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    out, lse = _outputs(q, dv, out, lse)
    cnt = 0
    if rescale_count is not None:
        if (rescale_count.dtype != torch.int64 or rescale_count.numel() != 1
                or rescale_count.device != q.device):
            raise ValueError("rescale_count must be a one-element int64 tensor on q's device")
        cnt = rescale_count.data_ptr()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        rc = lib.attn_fwd_dbg(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, Hq, Hkv, Lq, Lk, dqk, dv, int(bool(causal)),
                              float(scale), s.cuda_stream, float(rescale_threshold),
                              int(exp_mode), cnt)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_fwd_dbg failed: {status_string(rc)} (code {rc})")
    return out, lse


def _strides(t) -> Strides:
    sb, sh, sr, sc = t.stride()
    if sc != 1:
        raise ValueError("the head dim must be contiguous (stride 1)")
    return Strides(sb, sh, sr)


def attn_fwd_ex(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
                stream=None):
    """O, lse for [B, H, L, d]-shaped views of any strides with a contiguous head
    dim (e.g. [B, S, H, d] tensors passed as .transpose(1, 2)), bf16 or fp16.

    out defaults to the layout of q (row-major [B, Lq, Hq, d_v] viewed as
    [B, Hq, Lq, d_v] when q's rows are further apart than its heads, else
    contiguous [B, Hq, Lq, d_v]); lse is always contiguous fp32 [B, Hq, Lq]."""
    lib = _load()
    ts = (q, k, v)
    for name, t in zip("qkv", ts):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in (torch.bfloat16, torch.float16):
            raise TypeError(f"{name} must be bfloat16 or float16, got {t.dtype}")
        if t.device.type != "cuda" or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D tensor on a GPU device")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must have one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    B, Hq, Lq, dqk = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if Bk != B or dk != dqk or tuple(v.shape[:3]) != (B, Hkv, Lk):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    dv = v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if out is None:
        if q.stride(2) > q.stride(1):
            out = torch.empty((B, Lq, Hq, dv), dtype=q.dtype, device=q.device).transpose(1, 2)
        else:
            out = torch.empty((B, Hq, Lq, dv), dtype=q.dtype, device=q.device)
    _require_device(out, q.device, "out")
    if tuple(out.shape) != (B, Hq, Lq, dv) or out.dtype != q.dtype:
        raise ValueError("out must be a [B, Hq, Lq, d_v] view of q's dtype on q's device")
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    _require_device(lse, q.device, "lse")
    if lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, Hq, Lq] tensor")
    dtype = ATTN_DTYPE_FP16 if q.dtype == torch.float16 else ATTN_DTYPE_BF16
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        rc = lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, Hq, Hkv, Lq, Lk, dqk, dv, _strides(q),
                             _strides(k), _strides(v), _strides(out), dtype, int(bool(causal)),
                             float(scale), s.cuda_stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_fwd_ex failed: {status_string(rc)} (code {rc})")
    return out, lse


def attn_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, delta=None, stream=None):
    """dq, dk, dv (and delta = rowsum(dout * o)) of the attention forward pass
    that produced o and lse from q, k, v: contiguous [B, H, L, d] tensors, all
    bf16 (attn_bwd) or all fp16 (attn_bwd_ex), (d_qk, d_v) one of (64, 64),
    (128, 128), (192, 128)."""
    lib = _load()
    B, Hq, Hkv, Lq, Lk, dqk, dvd = _check_inputs(q, k, v, (torch.bfloat16, torch.float16))
    for name, t, shape in (("o", o, (B, Hq, Lq, dvd)), ("dout", dout, (B, Hq, Lq, dvd))):
        if (not isinstance(t, torch.Tensor) or t.dtype != q.dtype or t.device != q.device
                or tuple(t.shape) != shape or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {q.dtype} {shape} tensor on q's "
                             "device")
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Lq) or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError("lse must be the forward's contiguous fp32 [B, Hq, Lq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty_like(lse) if delta is None else delta
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v), ("delta", delta, lse)):
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like {tuple(ref.shape)}")
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
            B, Hq, Hkv, Lq, Lk, dqk, dvd)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        if q.dtype == torch.bfloat16:
            name = "attn_bwd"
            rc = lib.attn_bwd(*ptrs, int(bool(causal)), float(scale), s.cuda_stream)
        else:
            name = "attn_bwd_ex"
            rc = lib.attn_bwd_ex(*ptrs, ATTN_DTYPE_FP16, int(bool(causal)), float(scale),
                                 s.cuda_stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"{name} failed: {status_string(rc)} (code {rc})")
    return dq, dk, dv, delta


BWD_NOALLOC_MAX_ROWS = 4 << 20  # ATTN_BWD_NOALLOC_MAX_ROWS of include/attn_fwd.h


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal: bool = False,
                     scale: float | None = None, stream=None):
    """attn_bwd for callers that cannot allocate: dq, dk and dv (caller-owned,
    contiguous, on q's device) are written by the same kernels, with D kept in
    the library's static device scratch (B * Hq * Lq <= BWD_NOALLOC_MAX_ROWS).
    Calls that overlap on one device race on that scratch."""
    lib = _load()
    B, Hq, Hkv, Lq, Lk, dqk, dvd = _check_inputs(q, k, v)
    for name, t, shape in (("o", o, (B, Hq, Lq, dvd)), ("dout", dout, (B, Hq, Lq, dvd))):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.device != q.device
                or tuple(t.shape) != shape or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bf16 {shape} tensor on q's device")
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32
            or tuple(lse.shape) != (B, Hq, Lq) or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError("lse must be the forward's contiguous fp32 [B, Hq, Lq] tensor")
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if (not isinstance(t, torch.Tensor) or t.shape != ref.shape or t.dtype != ref.dtype
                or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous tensor like {tuple(ref.shape)} on "
                             "q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        rc = lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), B, Hq, Hkv, Lq, Lk, dqk, dvd,
                                  int(bool(causal)), float(scale), s.cuda_stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_bwd_noalloc failed: {status_string(rc)} (code {rc})")
    return dq, dk, dv


def split_keys(Lk: int, n_split: int) -> int:
    """Keys per split: split s covers keys [s*W, min(Lk, (s+1)*W))."""
    w = _load().attn_split_keys(int(Lk), int(n_split))
    if w < 0:
        raise ValueError(f"attn_split_keys: {status_string(-w)}")
    return w


def _split_call(name, q, k, v, n_split, causal, scale, o_part, lse_part, stream):
    lib = _load()
    B, Hq, Hkv, Lq, Lk, dqk, dv = _check_inputs(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    n = int(n_split)
    if o_part is None:
        o_part = torch.empty((n, B, Hq, Lq, dv), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((n, B, Hq, Lq), dtype=torch.float32, device=q.device)
    _require_device(o_part, q.device, "o_part")
    _require_device(lse_part, q.device, "lse_part")
    if (o_part.shape != (n, B, Hq, Lq, dv) or o_part.dtype != torch.float32
            or not o_part.is_contiguous()):
        raise ValueError("o_part must be a contiguous fp32 [n_split, B, Hq, Lq, d_v] tensor")
    if (lse_part.shape != (n, B, Hq, Lq) or lse_part.dtype != torch.float32
            or not lse_part.is_contiguous()):
        raise ValueError("lse_part must be a contiguous fp32 [n_split, B, Hq, Lq] tensor")
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        rc = getattr(lib, name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(),
                                lse_part.data_ptr(), B, Hq, Hkv, Lq, Lk, dqk, dv,
                                int(bool(causal)), float(scale), n, s.cuda_stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"{name} failed: {status_string(rc)} (code {rc})")
    return o_part, lse_part


def attn_fwd_split(q, k, v, n_split: int, causal: bool = False, scale: float | None = None,
                   o_part=None, lse_part=None, stream=None):
    """Per-split states (o_part fp32 [n_split,B,Hq,Lq,d_v], lse_part fp32
    [n_split,B,Hq,Lq]): the forward pass over each key split alone."""
    return _split_call("attn_fwd_split", q, k, v, n_split, causal, scale, o_part, lse_part,
                       stream)


def attn_fwd_decode(q, k, v, n_split: int, causal: bool = False, scale: float | None = None,
                    o_part=None, lse_part=None, stream=None):
    """attn_fwd_split's per-split states from the key-streaming decode kernel
    (Lq * Hq / Hkv <= 16, d_qk == d_v in {64, 128}); attn_fwd_split selects it
    by itself for such shapes."""
    return _split_call("attn_fwd_decode", q, k, v, n_split, causal, scale, o_part, lse_part,
                       stream)


def attn_merge(o_part, lse_part, out=None, lse=None, stream=None):
    """Merge per-split states [n_split, ..., d_v] / [n_split, ...] into the bf16
    output [..., d_v] and lse [...] (leading dims as in the per-split tensors)."""
    lib = _load()
    for name, t in (("o_part", o_part), ("lse_part", lse_part)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
    if o_part.device.type != "cuda":
        raise ValueError(f"o_part must be on a GPU device, got {o_part.device}")
    _require_device(lse_part, o_part.device, "lse_part")
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise TypeError("o_part and lse_part must be float32")
    if not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("o_part and lse_part must be contiguous")
    if o_part.dim() < 2 or tuple(o_part.shape[:-1]) != tuple(lse_part.shape):
        raise ValueError(f"o_part {tuple(o_part.shape)} and lse_part {tuple(lse_part.shape)} "
                         "do not match")
    n, dv = o_part.shape[0], o_part.shape[-1]
    lead = tuple(o_part.shape[1:-1])
    rows = 1
    for x in lead:
        rows *= x
    if out is None:
        out = torch.empty(lead + (dv,), dtype=torch.bfloat16, device=o_part.device)
    if lse is None:
        lse = torch.empty(lead, dtype=torch.float32, device=o_part.device)
    _require_device(out, o_part.device, "out")
    _require_device(lse, o_part.device, "lse")
    if tuple(out.shape) != lead + (dv,) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor of the merged shape")
    if tuple(lse.shape) != lead or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 tensor of the merged shape")
    with torch.cuda.device(o_part.device):
        s = stream if stream is not None else torch.cuda.current_stream(o_part.device)
        rc = lib.attn_merge(o_part.data_ptr(), lse_part.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), int(n), int(rows), int(dv), s.cuda_stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_merge failed: {status_string(rc)} (code {rc})")
    return out, lse


def attn_fwd_splitkv(q, k, v, n_split: int, causal: bool = False, scale: float | None = None,
                     stream=None):
    """O, lse by the split-key path: attn_fwd_split, then attn_merge."""
    o_part, lse_part = attn_fwd_split(q, k, v, n_split, causal=causal, scale=scale,
                                      stream=stream)
    return attn_merge(o_part, lse_part, stream=stream)


def _host_offsets(cu, name):
    """cu_seqlens (list, numpy array or tensor on any device) -> contiguous int32 numpy."""
    if isinstance(cu, torch.Tensor):
        cu = cu.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(cu, dtype=np.int64).ravel())
    if a.size < 2 or a.min() < 0 or a.max() > np.iinfo(np.int32).max:
        raise ValueError(f"{name} must hold n_seq + 1 offsets in int32 range")
    return np.ascontiguousarray(a.astype(np.int32))


def varlen_plan(cu_seqlens_q, cu_seqlens_k, Hq: int, Hkv: int, causal: bool):
    """Schedule of a packed variable-length batch, computed on the host by
    attn_varlen_plan: int32 [n_records, 8] tile records (n_records a multiple of 8)."""
    lib = _load()
    cq = _host_offsets(cu_seqlens_q, "cu_seqlens_q")
    ck = _host_offsets(cu_seqlens_k, "cu_seqlens_k")
    if cq.size != ck.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    n_seq = cq.size - 1
    n = ctypes.c_int(0)
    i32p = ctypes.POINTER(ctypes.c_int)
    rc = lib.attn_varlen_plan(cq.ctypes.data_as(i32p), ck.ctypes.data_as(i32p), n_seq, int(Hq),
                              int(Hkv), int(bool(causal)), None, 0, ctypes.byref(n))
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_varlen_plan failed: {status_string(rc)} (code {rc})")
    plan = np.zeros((n.value, VARLEN_RECORD_INTS), dtype=np.int32)
    if n.value:
        rc = lib.attn_varlen_plan(cq.ctypes.data_as(i32p), ck.ctypes.data_as(i32p), n_seq,
                                  int(Hq), int(Hkv), int(bool(causal)),
                                  plan.ctypes.data_as(i32p), n.value, ctypes.byref(n))
        if rc != ATTN_OK:
            raise RuntimeError(f"attn_varlen_plan failed: {status_string(rc)} (code {rc})")
    return plan


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool = False,
                    scale: float | None = None, plan=None, out=None, lse=None, stream=None):
    """O [Tq, Hq, d_v] bf16 and lse [Hq, Tq] fp32 of a packed variable-length
    batch: q [Tq, Hq, d_qk], k [Tk, Hkv, d_qk], v [Tk, Hkv, d_v] contiguous bf16
    on one GPU; sequence s owns query tokens [cu_seqlens_q[s], cu_seqlens_q[s+1])
    and key tokens [cu_seqlens_k[s], cu_seqlens_k[s+1]).  plan, if given, is the
    device int32 [n, 8] result of varlen_plan for the same batch; otherwise it is
    computed on the host and copied to q's device."""
    lib = _load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be a bfloat16 torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous token-major [T, H, d] tensor")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    Tq, Hq, dqk = q.shape
    Tk, Hkv, dk = k.shape
    if dk != dqk or tuple(v.shape[:2]) != (Tk, Hkv):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    dv = v.shape[2]
    cq = _host_offsets(cu_seqlens_q, "cu_seqlens_q")
    ck = _host_offsets(cu_seqlens_k, "cu_seqlens_k")
    if int(cq[-1]) != Tq or int(ck[-1]) != Tk:
        raise ValueError("the last offsets must equal the token counts of q and k")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if plan is None:
        plan = torch.from_numpy(varlen_plan(cq, ck, Hq, Hkv, causal)).to(q.device)
    if (not isinstance(plan, torch.Tensor) or plan.dtype != torch.int32 or plan.dim() != 2
            or plan.shape[1] != VARLEN_RECORD_INTS or plan.device != q.device
            or not plan.is_contiguous()):
        raise ValueError("plan must be a contiguous int32 [n, 8] tensor on q's device")
    if out is None:
        out = torch.empty((Tq, Hq, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    _require_device(out, q.device, "out")
    _require_device(lse, q.device, "lse")
    if tuple(out.shape) != (Tq, Hq, dv) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [Tq, Hq, d_v] tensor")
    if tuple(lse.shape) != (Hq, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [Hq, Tq] tensor")
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        rc = lib.attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), plan.data_ptr(), int(plan.shape[0]), Tq, Tk,
                                 Hq, Hkv, dqk, dv, int(bool(causal)), float(scale),
                                 s.cuda_stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_fwd_varlen failed: {status_string(rc)} (code {rc})")
    return out, lse
