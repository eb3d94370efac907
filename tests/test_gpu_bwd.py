"""GPU parity of the backward pass (attn_bwd through the C ABI) against the
fp64 oracle's gradients of the definition.  Needs an MI355X."""
import numpy as np
import pytest
import torch

from exact_attention_forward_02_amd import attn_bwd, attn_fwd, attn_fwd_ex
from exact_attention_forward_02_amd.inputs import make_qkv, make_qkv_fp16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# Bar for bf16 gradients, per tensor X against the exact X_ref:
#   max |X - X_ref| <= 1.5e-2 * max|X_ref|  and  mean |X - X_ref| <= 5e-3 * mean|X_ref|.
# Four bf16 roundings stand between the inputs and each gradient element: the
# forward's output o (through D = rowsum(dO * o)), P and dS as MFMA operands,
# and the stored gradient.  Each moves a value by at most half an ulp, 2^-8
# of it, and the max bound allows all four at once (4 * 2^-8 = 1.56e-2); a
# single rounding moves it by about 2^-10 on average, and the mean bound
# allows five of those.
TOL_MAX = 1.5e-2
TOL_MEAN = 5e-3
# fp16 (u = 2^-11): the same four roundings bound the max error by 4 * 2^-11 and
# five average ones the mean error by 5 * 2^-13
TOL_MAX_FP16 = 2e-3
TOL_MEAN_FP16 = 6.5e-4

# B, Hq, Hkv, Lq, Lk, d_qk, d_v, causal
SHAPES = [
    (1, 2, 2, 200, 300, 128, 128, False),
    (2, 4, 2, 256, 256, 128, 128, True),    # GQA 2
    (1, 4, 1, 130, 700, 64, 64, False),     # MQA, d = 64
    (1, 2, 2, 300, 129, 64, 64, True),      # Lq > Lk: rows without keys
    (1, 2, 2, 64, 64, 128, 128, True),      # one block
    (2, 8, 8, 1024, 1024, 128, 128, True),  # several blocks per workgroup and wave
    (1, 2, 2, 200, 300, 192, 128, False),   # (192, 128): dV and dK in two passes
    (2, 4, 2, 333, 333, 192, 128, True),    # (192, 128), GQA 2, ragged
    (1, 2, 2, 300, 129, 192, 128, True),    # (192, 128), rows without keys
    (1, 4, 4, 1024, 1024, 192, 128, True),  # (192, 128), several blocks
]
# fp16 at full precision (inputs drawn straight into fp16)
SHAPES_FP16 = [
    (1, 2, 2, 200, 300, 128, 128, False),
    (2, 4, 2, 256, 256, 128, 128, True),
    (1, 4, 1, 130, 700, 64, 64, False),
    (2, 4, 2, 333, 333, 192, 128, True),
]


def _ids(s):
    return "x".join(map(str, s))


def _stats(name, got, ref, tol_max=TOL_MAX, tol_mean=TOL_MEAN):
    g = got.detach().cpu().double().numpy()
    err = np.abs(g - ref)
    scale_max = float(np.abs(ref).max())
    scale_mean = float(np.abs(ref).mean())
    st = {"max": float(err.max()), "mean": float(err.mean()), "ref_max": scale_max,
          "ref_mean": scale_mean}
    print(f"[bwd parity] {name}: " + ", ".join(f"{k}={v:.3e}" for k, v in st.items()), flush=True)
    assert np.all(np.isfinite(g)), f"{name}: non-finite gradient"
    assert st["max"] <= tol_max * scale_max, f"{name}: max error {st['max']:.3e}"
    assert st["mean"] <= tol_mean * scale_mean, f"{name}: mean error {st['mean']:.3e}"


def _check_backward(orc, shape, dtype):
    B, Hq, Hkv, Lq, Lk, dqk, dvd, causal = shape
    print(f"[case] bwd {dtype} {shape}", flush=True)
    if dtype == torch.float16:
        q, k, v = make_qkv_fp16(B, Hq, Hkv, Lq, Lk, dqk, dvd, seed=hash(shape) % 10007)
        tol = (TOL_MAX_FP16, TOL_MEAN_FP16)
    else:
        q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, dqk, dvd, seed=hash(shape) % 10007)
        tol = (TOL_MAX, TOL_MEAN)
    g = torch.Generator().manual_seed(hash(shape) % 997)
    dout = torch.randn((B, Hq, Lq, dvd), generator=g).to(dtype)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    if dtype == torch.float16:
        o, lse = attn_fwd_ex(qd, kd, vd, causal=causal)
    else:
        o, lse = attn_fwd(qd, kd, vd, causal=causal)
    dq, dk, dv, delta = attn_bwd(qd, kd, vd, o, lse, gd, causal=causal)
    torch.cuda.synchronize()
    assert dq.dtype == dk.dtype == dv.dtype == dtype
    want_dq, want_dk, want_dv, want_delta = orc.attn_bwd(q, k, v, dout, causal=causal)
    tag = f"{'fp16' if dtype == torch.float16 else 'bf16'} {shape}"
    _stats(f"dq {tag}", dq, want_dq, *tol)
    _stats(f"dk {tag}", dk, want_dk, *tol)
    _stats(f"dv {tag}", dv, want_dv, *tol)
    _stats(f"delta {tag}", delta, want_delta, *tol)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_backward_matches_the_oracle(orc, shape):
    _check_backward(orc, shape, torch.bfloat16)


@pytest.mark.parametrize("shape", SHAPES_FP16, ids=_ids)
def test_backward_fp16_matches_the_oracle(orc, shape):
    """fp16 tensors (attn_bwd_ex) with values bf16 cannot hold, to the fp16 bar."""
    _check_backward(orc, shape, torch.float16)


def test_backward_gqa_equals_repeated_heads_summed():
    """dK, dV of a GQA problem equal the per-group sums of the MHA problem
    with repeated K/V heads (up to bf16 rounding of the summands)."""
    B, Hq, Hkv, L, d = 1, 8, 2, 256, 128
    q, k, v = (t.to(DEV) for t in make_qkv(B, Hq, Hkv, L, L, d, d, seed=5))
    dout = torch.randn((B, Hq, L, d), generator=torch.Generator().manual_seed(6)).to(
        torch.bfloat16).to(DEV)
    for causal in (False, True):
        o, lse = attn_fwd(q, k, v, causal=causal)
        dq, dk, dv, _ = attn_bwd(q, k, v, o, lse, dout, causal=causal)
        kr = k.repeat_interleave(4, 1).contiguous()
        vr = v.repeat_interleave(4, 1).contiguous()
        o2, lse2 = attn_fwd(q, kr, vr, causal=causal)
        dq2, dk2, dv2, _ = attn_bwd(q, kr, vr, o2, lse2, dout, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq2)
        for a, b2 in ((dk, dk2), (dv, dv2)):
            summed = b2.float().reshape(B, Hkv, 4, L, d).sum(2)
            err = (a.float() - summed).abs().max().item()
            assert err <= 2e-2 * summed.abs().max().item(), err


@pytest.mark.parametrize("name,n_heads", [("mha_l2k", 2), ("causal_l8k", 1), ("dsv3_l32k", 1)])
def test_backward_full_size_sampled_heads(orc, name, n_heads):
    """The backward at a full workload size, as bench.py --backward runs it:
    gradients of one head depend only on that head's q, k, v and dout, so
    the oracle's backward of the sliced one-head problem is the exact
    reference for sampled heads."""
    from exact_attention_forward_02_amd.inputs import WORKLOADS, workload_qkv

    w = WORKLOADS[name]
    print(f"[case] bwd {w.name} {w.as_dict()}", flush=True)
    q, k, v = workload_qkv(w)
    g = torch.Generator().manual_seed(w.seed + 1)
    dout = torch.randn((w.B, w.Hq, w.Lq, w.dv), generator=g).to(torch.bfloat16)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    o, lse = attn_fwd(qd, kd, vd, causal=w.causal)
    dq, dk, dv, delta = attn_bwd(qd, kd, vd, o, lse, gd, causal=w.causal)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, delta):
        assert torch.isfinite(t.float()).all().item()
    rng = np.random.default_rng(w.seed)
    for _ in range(n_heads):
        b, h = int(rng.integers(w.B)), int(rng.integers(w.Hq))
        sl = lambda t: t[b:b + 1, h:h + 1].contiguous()  # noqa: E731  (MHA: kv head h)
        ref = orc.attn_bwd(sl(q), sl(k), sl(v), sl(dout), causal=w.causal)
        for nm, got, want in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), ref):
            _stats(f"{nm} {w.name} b{b} h{h}", got[b:b + 1, h:h + 1], want)
