"""Tolerances and comparison used by the GPU parity tests.

Bar (fixed for this kernel): bf16 output within max |dO| <= 1e-2 and
mean |dO| <= 1e-3 of the fp64 oracle, lse within 1e-3 (fp32 output).  Rows
with no visible key must come back exactly as O = 0, lse = -inf.  The floor
printed beside the error, mean |bf16(O_oracle) - O_oracle|, is what rounding
the exact result to bf16 alone costs.

Stress inputs (Q scaled by 6 at more rows than the tiny workload) make rows
nearly one-hot with |O| up to ~4, where one bf16 ulp is 1.6e-2: rounding P to
bf16 before the PV product (the method's design) can then move an output by
one ulp.  For those cases the max bound is the one the FA4 chapter validates
its kernel with (assert_close with rtol = atol = 1e-2, section on compile and
validation constraints): |dO| <= 1e-2 + 1e-2 |O_ref| per element; the mean
and lse bars are unchanged.
"""
from __future__ import annotations

import math

import numpy as np
import torch

TOL_O_MAX = 1e-2
TOL_O_MEAN = 1e-3
TOL_LSE_MAX = 1e-3


def parity_stats(o_gpu, lse_gpu, o_ref, lse_ref):
    og = o_gpu.detach().cpu().double().numpy().reshape(o_ref.shape)
    lg = lse_gpu.detach().cpu().double().numpy().reshape(lse_ref.shape)
    empty = np.isneginf(lse_ref)
    full = ~empty
    err = np.abs(og[full] - o_ref[full])
    floor = np.abs(torch.from_numpy(o_ref[full]).to(torch.bfloat16).double().numpy()
                   - o_ref[full])
    dl = np.abs(lg[full] - lse_ref[full])
    rel_excess = err - TOL_O_MAX * np.abs(o_ref[full])
    return {
        "o_max_minus_rtol": float(rel_excess.max()) if rel_excess.size else 0.0,
        "rows": int(o_ref.shape[0]),
        "empty_rows": int(empty.sum()),
        "o_max": float(err.max()) if err.size else 0.0,
        "o_mean": float(err.mean()) if err.size else 0.0,
        "o_floor_mean": float(floor.mean()) if floor.size else 0.0,
        "lse_max": float(dl.max()) if dl.size else 0.0,
        "empty_ok": bool(np.all(og[empty] == 0.0) and np.all(np.isneginf(lg[empty]))),
        "finite": bool(np.all(np.isfinite(og)) and np.all(np.isfinite(lg[full]))),
    }


def assert_parity(tag, o_gpu, lse_gpu, o_ref, lse_ref, stress=False):
    st = parity_stats(o_gpu, lse_gpu, o_ref, lse_ref)
    print(f"[parity] {tag}: " + ", ".join(
        f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in st.items()),
        flush=True)
    assert st["finite"], f"{tag}: non-finite output"
    assert st["empty_ok"], f"{tag}: rows without keys must give O = 0 and lse = -inf"
    if stress:
        assert st["o_max_minus_rtol"] <= TOL_O_MAX, (
            f"{tag}: max |dO| - 1e-2 |O| = {st['o_max_minus_rtol']:.3e} > {TOL_O_MAX}")
    else:
        assert st["o_max"] <= TOL_O_MAX, f"{tag}: max |dO| {st['o_max']:.3e} > {TOL_O_MAX}"
    assert st["o_mean"] <= TOL_O_MEAN, f"{tag}: mean |dO| {st['o_mean']:.3e} > {TOL_O_MEAN}"
    assert st["lse_max"] <= TOL_LSE_MAX, f"{tag}: max |dlse| {st['lse_max']:.3e} > {TOL_LSE_MAX}"
    return st


def gather_rows(o, lse, rows):
    """o [B,H,L,dv] and lse [B,H,L] (any device) at flat row indices."""
    idx = torch.as_tensor(rows, dtype=torch.int64)
    dv = o.shape[-1]
    o2 = o.reshape(-1, dv).index_select(0, idx.to(o.device)).cpu()
    l2 = lse.reshape(-1).index_select(0, idx.to(lse.device)).cpu()
    return o2, l2


def default_scale(dqk):
    return 1.0 / math.sqrt(dqk)
