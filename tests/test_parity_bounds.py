"""The tolerances of the GPU parity tests, checked on the CPU.

1. The bf16-weight bound (tests/parity.py) on the inputs that use it: a plain
   float32 emulation of the method's arithmetic (scores in fp32, weights
   rounded to bf16, normalised by their own sum, bf16 output) stays within
   max(1e-2, bound) on every element, and passes the absolute 1e-2 bar
   somewhere, so the absolute bar is unreachable for any kernel that rounds
   the weights and the output to bf16 on these inputs.
2. The bars of the true-fp16 test: the same emulation with fp16 weights and
   output meets them, while rounding the inputs, the weights or the output to
   bf16 instead fails them, so the GPU test notices bf16 truncation anywhere
   on the fp16 path.
The emulation is test arithmetic for sizing tolerances, not a reference: the
expected values come from the oracle.
"""
import numpy as np
import pytest
import torch

import parity
from exact_attention_forward_02_amd.inputs import make_qkv, make_qkv_fp16


def _emulate(q, k, v, causal, scale, wdt, odt):
    """Method arithmetic in float32 with weights rounded to wdt and the output to odt."""
    G = q.shape[1] // k.shape[1]
    kf = k.float().repeat_interleave(G, 1)
    vf = v.float().repeat_interleave(G, 1)
    s = torch.matmul(q.float(), kf.transpose(-1, -2).contiguous())
    Lq, Lk = s.shape[-2:]
    if causal:
        i = torch.arange(Lq)[:, None]
        j = torch.arange(Lk)[None, :]
        s = s.masked_fill(j > i + (Lk - Lq), -float("inf"))
    c2 = scale * 1.4426950408889634
    m = s.amax(-1, keepdim=True)
    p = torch.exp2(s * c2 - m * c2).to(wdt).float()
    o = torch.matmul(p, vf) / p.sum(-1, keepdim=True)
    return o.to(odt).double().numpy().reshape(-1, v.shape[-1])


def test_half_ulp_bf16():
    x = np.array([1.0, 1.5, 2.0, 3.99, 4.0, 0.25, -2.5])
    want = np.array([2 ** -8, 2 ** -8, 2 ** -7, 2 ** -7, 2 ** -6, 2 ** -10, 2 ** -7])
    assert np.array_equal(parity.half_ulp_bf16(x), want)


def test_weight_bound_two_key_tie():
    """Two keys of equal weight with V = +4 and -4: O = 0 exactly, and the bound's
    first term is u/(1-u) * 4."""
    w = np.array([[0.5, 0.5]])
    v = np.array([[4.0], [-4.0]])
    o = np.zeros((1, 1))
    b = parity.bf16_weight_bound(w, v, o)
    u = 2.0 ** -8
    first = u / (1 - u) * 4.0
    assert b[0, 0] == pytest.approx(first + parity.half_ulp_bf16(first), rel=1e-12)


@pytest.mark.parametrize("shape", [(2, 4, 4, 513, 513, 128, 128, True, 6.0)])
def test_bf16_weight_bound_covers_the_method(orc, shape):
    B, Hq, Hkv, Lq, Lk, dqk, dv, causal, qm = shape
    q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, dqk, dv, seed=hash(shape) % 10007, q_mult=qm)
    scale = parity.default_scale(dqk)
    o_ref, _ = orc.attn_rows(q, k, v, causal=causal)
    bound = parity.dense_bound(q, k, v, causal, scale, o_ref)
    err = np.abs(_emulate(q, k, v, causal, scale, torch.bfloat16, torch.bfloat16) - o_ref)
    assert np.all(err <= np.maximum(parity.TOL_O_MAX, bound))
    assert err.max() > parity.TOL_O_MAX, "this input does not need the bound"
    # the bound lifts the bar on a small share of the elements only
    assert (bound > parity.TOL_O_MAX).mean() < 0.01


FP16_SHAPES = [(1, 2, 2, 300, 300, 128, 128, False), (1, 4, 4, 513, 513, 128, 128, True),
               (1, 3, 1, 517, 517, 64, 64, False)]


@pytest.mark.parametrize("shape", FP16_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp16_bars_detect_bf16_truncation(orc, shape):
    causal = shape[7]
    q, k, v = make_qkv_fp16(*shape[:7], seed=sum(shape[:7]))
    assert not torch.equal(q.to(torch.bfloat16).to(torch.float16), q)
    scale = parity.default_scale(shape[5])
    o_ref, _ = orc.attn_rows(q, k, v, causal=causal)

    def stats(qq, kk, vv, wdt, odt):
        e = np.abs(_emulate(qq, kk, vv, causal, scale, wdt, odt) - o_ref)
        return e.max(), e.mean()

    mx, mean = stats(q, k, v, torch.float16, torch.float16)
    assert mx <= parity.TOL_FP16_O_MAX and mean <= parity.TOL_FP16_O_MEAN
    bq, bk, bv = (t.to(torch.bfloat16) for t in (q, k, v))
    for what, args in (("inputs", (bq, bk, bv, torch.float16, torch.float16)),
                       ("weights", (q, k, v, torch.bfloat16, torch.float16)),
                       ("output", (q, k, v, torch.float16, torch.bfloat16))):
        _, mean_b = stats(*args)
        assert mean_b > parity.TOL_FP16_O_MEAN, f"bf16 {what} would pass the fp16 bar"
