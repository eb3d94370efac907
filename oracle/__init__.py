"""CPU fp64 oracle for exact attention forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library and never imports
it; the two meet only through the seeded inputs both are fed.

The arithmetic lives in ``attn_oracle.c`` (plain C, double precision, OpenMP
over query rows).  This module compiles it with gcc when no built library is
present and marshals arguments through ctypes.

Functions
---------
attn_rows      the definition, materialised one score row at a time; with
               k_range=(k0, k1) the partial state of one key segment
merge          the two-block merge rule folded over the partial states of
               several key segments
attn_varlen    the definition inside each sequence of a packed
               variable-length batch (token-major [T, H, d] tensors)
online_rows    the tiled method (always-rescale Algorithm 1, or conditional
               base-2 rescaling per row or per row group), for checking the
               algorithm against the definition
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *extra_flags, "-o", output + ".tmp", source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


ELEM_BF16, ELEM_FP16 = 0, 1


def _as_bits(t) -> np.ndarray:
    """bf16 tensor (torch, any device) or uint16 array -> contiguous uint16."""
    bits, elem = _as_bits_elem(t)
    if elem != ELEM_BF16:
        raise TypeError("expected bfloat16 input")
    return bits


def _as_bits_elem(t):
    """16-bit tensor (torch bf16 or fp16, any device and strides) or uint16 array of
    bf16 patterns -> (contiguous uint16 bit patterns, element type)."""
    if isinstance(t, np.ndarray):
        if t.dtype != np.uint16:
            raise TypeError("numpy inputs must hold bf16 bit patterns as uint16")
        return np.ascontiguousarray(t), ELEM_BF16
    import torch

    if t.dtype == torch.bfloat16:
        elem = ELEM_BF16
    elif t.dtype == torch.float16:
        elem = ELEM_FP16
    else:
        raise TypeError(f"expected a bfloat16 or float16 tensor, got {t.dtype}")
    bits = t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return bits, elem


class Oracle:
    """ctypes handle on one built copy of attn_oracle.c."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_attn_rows.argtypes = [
            _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
            ctypes.c_int, ctypes.c_double, _ptr, _i64, _ptr, _ptr, ctypes.c_int]
        lib.oracle_attn_rows_range.restype = ctypes.c_int
        lib.oracle_attn_rows_range.argtypes = [
            _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
            ctypes.c_int, ctypes.c_double, _i64, _i64, _ptr, _i64, _ptr, _ptr, ctypes.c_int]
        lib.oracle_attn_rows_elem.restype = ctypes.c_int
        lib.oracle_attn_rows_elem.argtypes = [
            _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
            ctypes.c_int, ctypes.c_double, _i64, _i64, _ptr, _i64, _ptr, _ptr, ctypes.c_int,
            ctypes.c_int]
        lib.oracle_attn_varlen.restype = ctypes.c_int
        lib.oracle_attn_varlen.argtypes = [
            _ptr, _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
            ctypes.c_double, _ptr, _i64, _ptr, _ptr, ctypes.c_int, ctypes.c_int]
        lib.oracle_widen.restype = ctypes.c_double
        lib.oracle_widen.argtypes = [ctypes.c_uint16, ctypes.c_int]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [
            _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
            ctypes.c_int, ctypes.c_double, ctypes.c_int, _ptr, _ptr, _ptr, _ptr, ctypes.c_int]
        lib.oracle_merge_states.restype = ctypes.c_int
        lib.oracle_merge_states.argtypes = [_ptr, _ptr, _i64, _i64, _i64, _ptr, _ptr]
        lib.oracle_online_rows.restype = ctypes.c_int
        lib.oracle_online_rows.argtypes = [
            _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
            ctypes.c_int, ctypes.c_double, _i64, ctypes.c_int, ctypes.c_double,
            _i64, _ptr, _i64, _ptr, _ptr, _ptr, _ptr, ctypes.c_int]
        self._lib = lib

    @staticmethod
    def _shapes(q, k, v):
        if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
            raise ValueError("q, k, v must be [B, H, L, d]")
        B, Hq, Lq, dqk = q.shape
        Bk, Hkv, Lk, dk = k.shape
        Bv, Hv, Lv, dv = v.shape
        if (Bk, dk) != (B, dqk) or (Bv, Hv, Lv) != (B, Hkv, Lk):
            raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} "
                             f"v{tuple(v.shape)}")
        return B, Hq, Hkv, Lq, Lk, dqk, dv

    @staticmethod
    def _rows(rows, total):
        if rows is None:
            return None, total
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).ravel())
        return r, r.size

    def attn_rows(self, q, k, v, causal: bool, scale: float | None = None,
                  rows=None, threads: int = 0, k_range=None):
        """Exact O [n, dv] and lse [n] (float64) for the requested query rows of
        bf16 or fp16 inputs (any strides; q, k, v of one element type).

        A row index is (b*Hq + h)*Lq + i; rows=None means every row in order.
        k_range=(k0, k1) restricts the softmax to the visible keys in [k0, k1):
        the partial state of that key segment (O = 0, lse = -inf where the
        segment holds no visible key).
        """
        (qb, eq), (kb, ek), (vb, ev) = _as_bits_elem(q), _as_bits_elem(k), _as_bits_elem(v)
        if not eq == ek == ev:
            raise TypeError("q, k and v must have one element type")
        B, Hq, Hkv, Lq, Lk, dqk, dv = self._shapes(qb, kb, vb)
        if scale is None:
            scale = 1.0 / math.sqrt(dqk)
        k0, k1 = (0, Lk) if k_range is None else (int(k_range[0]), int(k_range[1]))
        r, n = self._rows(rows, B * Hq * Lq)
        o = np.empty((n, dv), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self._lib.oracle_attn_rows_elem(
            qb.ctypes.data, kb.ctypes.data, vb.ctypes.data,
            B, Hq, Hkv, Lq, Lk, dqk, dv, int(bool(causal)), float(scale), k0, k1,
            None if r is None else r.ctypes.data, n,
            o.ctypes.data, lse.ctypes.data, int(threads), eq)
        if rc != 0:
            raise ValueError(f"oracle_attn_rows rejected its arguments (code {rc})")
        return o, lse

    def attn_varlen(self, q, k, v, cu_q, cu_k, causal: bool, scale: float | None = None,
                    rows=None, threads: int = 0):
        """Exact O [n, dv] and lse [n] (float64) of a packed variable-length
        batch: q [Tq, Hq, dqk], k [Tk, Hkv, dqk], v [Tk, Hkv, dv] (bf16 or fp16),
        sequence s owning tokens [cu_q[s], cu_q[s+1]) and keys [cu_k[s], cu_k[s+1]).
        A row index is h*Tq + t; rows=None means every row in order."""
        (qb, eq), (kb, ek), (vb, ev) = _as_bits_elem(q), _as_bits_elem(k), _as_bits_elem(v)
        if not eq == ek == ev:
            raise TypeError("q, k and v must have one element type")
        if qb.ndim != 3 or kb.ndim != 3 or vb.ndim != 3:
            raise ValueError("varlen q, k, v must be [T, H, d]")
        Tq, Hq, dqk = qb.shape
        Tk, Hkv, dk = kb.shape
        if dk != dqk or vb.shape[:2] != (Tk, Hkv):
            raise ValueError(f"shape mismatch q{qb.shape} k{kb.shape} v{vb.shape}")
        dv = vb.shape[2]
        cq = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int64).ravel())
        ck = np.ascontiguousarray(np.asarray(cu_k, dtype=np.int64).ravel())
        if cq.size != ck.size or cq.size < 2 or cq[-1] != Tq or ck[-1] != Tk:
            raise ValueError("cu_q / cu_k must have n_seq + 1 entries ending at Tq / Tk")
        if scale is None:
            scale = 1.0 / math.sqrt(dqk)
        r, n = self._rows(rows, Hq * Tq)
        o = np.empty((n, dv), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self._lib.oracle_attn_varlen(
            qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, cq.ctypes.data, ck.ctypes.data,
            cq.size - 1, Hq, Hkv, dqk, dv, int(bool(causal)), float(scale),
            None if r is None else r.ctypes.data, n, o.ctypes.data, lse.ctypes.data,
            int(threads), eq)
        if rc != 0:
            raise ValueError(f"oracle_attn_varlen rejected its arguments (code {rc})")
        return o, lse

    def attn_bwd(self, q, k, v, dout, causal: bool, scale: float | None = None,
                 threads: int = 0):
        """Exact gradients (float64) of <dO, O> for the definition:
        dq [B,Hq,Lq,dqk], dk [B,Hkv,Lk,dqk], dv [B,Hkv,Lk,dv], delta [B,Hq,Lq]
        (delta_i = sum_j P_ij dP_ij = dO_i . O_i).  Inputs bf16 or fp16 [B,H,L,d]."""
        ins = [_as_bits_elem(t) for t in (q, k, v, dout)]
        elems = {e for _, e in ins}
        if len(elems) != 1:
            raise TypeError("q, k, v and dout must have one element type")
        (qb, _), (kb, _), (vb, _), (gb, _) = ins
        B, Hq, Hkv, Lq, Lk, dqk, dv = self._shapes(qb, kb, vb)
        if gb.shape != (B, Hq, Lq, dv):
            raise ValueError(f"dout must be [B, Hq, Lq, d_v], got {gb.shape}")
        if scale is None:
            scale = 1.0 / math.sqrt(dqk)
        dq = np.empty((B, Hq, Lq, dqk), dtype=np.float64)
        dk = np.empty((B, Hkv, Lk, dqk), dtype=np.float64)
        dvo = np.empty((B, Hkv, Lk, dv), dtype=np.float64)
        delta = np.empty((B, Hq, Lq), dtype=np.float64)
        rc = self._lib.oracle_attn_bwd(
            qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, gb.ctypes.data,
            B, Hq, Hkv, Lq, Lk, dqk, dv, int(bool(causal)), float(scale), elems.pop(),
            dq.ctypes.data, dk.ctypes.data, dvo.ctypes.data, delta.ctypes.data, int(threads))
        if rc != 0:
            raise ValueError(f"oracle_attn_bwd rejected its arguments (code {rc})")
        return dq, dk, dvo, delta

    def widen(self, bits: int, elem: int) -> float:
        """The oracle's exact widening of one 16-bit pattern (ELEM_BF16 / ELEM_FP16)."""
        return self._lib.oracle_widen(int(bits), int(elem))

    def merge(self, o_parts, lse_parts):
        """Merge segment states: o_parts [n, rows, dv], lse_parts [n, rows]
        (float64) -> (O [rows, dv], lse [rows])."""
        op = np.ascontiguousarray(np.asarray(o_parts, dtype=np.float64))
        lp = np.ascontiguousarray(np.asarray(lse_parts, dtype=np.float64))
        if op.ndim != 3 or lp.shape != op.shape[:2]:
            raise ValueError(f"o_parts {op.shape} and lse_parts {lp.shape} do not match")
        n, rows, dv = op.shape
        o = np.empty((rows, dv), dtype=np.float64)
        lse = np.empty((rows,), dtype=np.float64)
        rc = self._lib.oracle_merge_states(op.ctypes.data, lp.ctypes.data, n, rows, dv,
                                           o.ctypes.data, lse.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_merge_states rejected its arguments (code {rc})")
        return o, lse

    def online_rows(self, q, k, v, causal: bool, scale: float | None = None,
                    bn: int = 64, mode: int = 1, tau: float = 8.0, group: int = 1,
                    rows=None, threads: int = 0):
        """Tiled method; returns (O, lse, state[n, 2], n_rescale_events).

        mode 0: always rescale, natural exponent; mode 1: conditional base-2
        rescale decided per row; mode 2: decision shared by `group` rows.
        state[:, 0] is the final reference, state[:, 1] the final denominator.
        """
        qb, kb, vb = _as_bits(q), _as_bits(k), _as_bits(v)
        B, Hq, Hkv, Lq, Lk, dqk, dv = self._shapes(qb, kb, vb)
        if scale is None:
            scale = 1.0 / math.sqrt(dqk)
        r, n = self._rows(rows, B * Hq * Lq)
        o = np.empty((n, dv), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        state = np.empty((n, 2), dtype=np.float64)
        events = ctypes.c_int64(0)
        rc = self._lib.oracle_online_rows(
            qb.ctypes.data, kb.ctypes.data, vb.ctypes.data,
            B, Hq, Hkv, Lq, Lk, dqk, dv, int(bool(causal)), float(scale),
            int(bn), int(mode), float(tau), int(group),
            None if r is None else r.ctypes.data, n,
            o.ctypes.data, lse.ctypes.data, state.ctypes.data,
            ctypes.addressof(events), int(threads))
        if rc != 0:
            raise ValueError(f"oracle_online_rows rejected its arguments (code {rc})")
        return o, lse, state, int(events.value)


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle built from this directory (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def attn_rows(*args, **kwargs):
    return load().attn_rows(*args, **kwargs)


def attn_varlen(*args, **kwargs):
    return load().attn_varlen(*args, **kwargs)


def online_rows(*args, **kwargs):
    return load().online_rows(*args, **kwargs)


def merge(*args, **kwargs):
    return load().merge(*args, **kwargs)
