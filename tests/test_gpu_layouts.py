"""GPU parity of the strided, fp16-capable entry point attn_fwd_ex against the
fp64 oracle, through the C ABI: fp16 inputs, the [B, S, H, d] layout of the
pages' usage example, views into packed QKV tensors, output written into a
caller's view.  Needs an MI355X."""
import pytest
import torch

from exact_attention_forward_02_amd import attn_fwd, attn_fwd_ex
from exact_attention_forward_02_amd.inputs import WORKLOADS, make_qkv, make_qkv_fp16, sample_rows
from parity import (TOL_FP16_LSE_MAX, TOL_FP16_O_MAX, TOL_FP16_O_MEAN, assert_parity,
                    gather_rows, parity_stats)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# B, Hq, Hkv, Lq, Lk, dqk, dv, causal, q_mult
SHAPES = [
    (1, 2, 2, 300, 300, 128, 128, False, 1.0),
    (2, 8, 2, 200, 333, 128, 128, True, 1.0),    # GQA 4, Lq < Lk
    (1, 6, 3, 257, 129, 64, 64, True, 1.0),      # Lq > Lk: rows without keys
    (1, 3, 1, 100, 517, 192, 128, False, 1.0),   # (192, 128)
    (2, 4, 4, 513, 513, 128, 128, True, 6.0),    # Q x 6
    (1, 4, 1, 130, 700, 64, 64, False, 1.0),     # MQA
]


def _ids(s):
    return "x".join(map(str, s))


def _inputs(shape, dtype):
    B, Hq, Hkv, Lq, Lk, dqk, dv, causal, qm = shape
    q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, dqk, dv, seed=hash(shape) % 10007, q_mult=qm)
    return [t.float().to(dtype) for t in (q, k, v)]


def _bshd_view(t):
    """The same values stored [B, L, H, d], viewed as [B, H, L, d]."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _check(tag, o, lse, q, k, v, causal, orc):
    dv = o.shape[-1]
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal)
    return assert_parity(tag, o.reshape(-1, dv).cpu(), lse.reshape(-1).cpu(), o_ref, l_ref)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_fp16_contiguous(orc, shape):
    print(f"[case] fp16 bhsd {shape}", flush=True)
    q, k, v = _inputs(shape, torch.float16)
    o, lse = attn_fwd_ex(q.to(DEV), k.to(DEV), v.to(DEV), causal=shape[7])
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    _check(f"fp16 {shape}", o, lse, q, k, v, shape[7], orc)


# Shapes of the true-fp16 test: B, Hq, Hkv, Lq, Lk, dqk, dv, causal
FP16_SHAPES = [(1, 2, 2, 300, 300, 128, 128, False), (1, 4, 4, 513, 513, 128, 128, True),
               (1, 3, 1, 517, 517, 64, 64, False), (2, 8, 2, 200, 333, 128, 128, True),
               (1, 2, 2, 100, 517, 192, 128, False),
               # chained sweeps over 2-3 tiles per workgroup
               (2, 160, 160, 300, 1100, 128, 128, False), (4, 64, 16, 500, 640, 64, 64, False)]


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
@pytest.mark.parametrize("shape", FP16_SHAPES, ids=_ids)
def test_fp16_full_precision(orc, shape, layout):
    """Inputs drawn straight into fp16, so most values carry mantissa bits bf16
    cannot hold, against the oracle's exact fp16 widening.  The bars (max
    |dO| <= 2e-3, mean |dO| <= 5e-5, max |dlse| <= 1e-4) sit below what
    rounding the inputs, the weights P or the output to bf16 would cost on
    these inputs (sized on the CPU by emulation in test_parity_bounds.py)."""
    causal = shape[7]
    print(f"[case] fp16 full precision {layout} {shape}", flush=True)
    q, k, v = make_qkv_fp16(*shape[:7], seed=sum(shape[:7]))
    assert not torch.equal(q.to(torch.bfloat16).to(torch.float16), q)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    if layout == "bshd":
        qd, kd, vd = (_bshd_view(t) for t in (qd, kd, vd))
    o, lse = attn_fwd_ex(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal)
    st = parity_stats(o.reshape(-1, shape[6]), lse.reshape(-1), o_ref, l_ref)
    print(f"[parity] fp16 full precision {layout} {shape}: " + ", ".join(
        f"{k_}={v_:.3e}" if isinstance(v_, float) else f"{k_}={v_}" for k_, v_ in st.items()),
        flush=True)
    assert st["finite"] and st["empty_ok"]
    assert st["o_max"] <= TOL_FP16_O_MAX, st
    assert st["o_mean"] <= TOL_FP16_O_MEAN, st
    assert st["lse_max"] <= TOL_FP16_LSE_MAX, st


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("shape", SHAPES[:4], ids=_ids)
def test_bshd_layout(orc, shape, dtype):
    """[B, S, H, d] storage (the pages' usage example): result and output layout."""
    print(f"[case] bshd {dtype} {shape}", flush=True)
    q, k, v = _inputs(shape, dtype)
    qd, kd, vd = (_bshd_view(t.to(DEV)) for t in (q, k, v))
    o, lse = attn_fwd_ex(qd, kd, vd, causal=shape[7])
    torch.cuda.synchronize()
    assert o.transpose(1, 2).is_contiguous(), "output should follow q's [B, S, H, d] layout"
    _check(f"bshd {dtype} {shape}", o, lse, q, k, v, shape[7], orc)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_packed_qkv_views(orc, dtype):
    """q, k, v as views into one [B, S, 3, H, d] tensor; output into a view of a
    wider [B, S, H, d + 64] buffer."""
    B, H, L, d = 2, 4, 300, 128
    print(f"[case] packed qkv {dtype} B{B} H{H} L{L} d{d}", flush=True)
    g = torch.Generator().manual_seed(17)
    qkv = torch.randn((B, L, 3, H, d), generator=g).to(dtype)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    qkv_d = qkv.to(DEV)
    qd, kd, vd = (qkv_d[:, :, i].transpose(1, 2) for i in range(3))
    wide = torch.full((B, L, H, d + 64), 7.0, dtype=dtype, device=DEV)
    out = wide[..., :d].transpose(1, 2)
    for causal in (False, True):
        o, lse = attn_fwd_ex(qd, kd, vd, causal=causal, out=out)
        torch.cuda.synchronize()
        assert o.data_ptr() == out.data_ptr()
        assert torch.all(wide[..., d:] == 7.0), "wrote outside the output view"
        _check(f"packed {dtype} causal={causal}", o, lse, q, k, v, causal, orc)


def test_contiguous_bf16_equals_attn_fwd():
    """attn_fwd_ex on contiguous bf16 tensors is attn_fwd, bit for bit."""
    q, k, v = (t.to(DEV) for t in make_qkv(2, 8, 2, 333, 555, 128, 128, seed=31))
    for causal in (False, True):
        o1, l1 = attn_fwd(q, k, v, causal=causal)
        o2, l2 = attn_fwd_ex(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_layout_does_not_change_the_result(dtype):
    """The same values in [B, H, L, d] and [B, S, H, d] storage give the same
    bits (only addresses differ), on a launch of more than 256 tiles."""
    q, k, v = (t.float().to(dtype).to(DEV)
               for t in make_qkv(2, 16, 16, 2100, 700, 128, 128, seed=123))
    for causal in (False, True):
        o1, l1 = attn_fwd_ex(q, k, v, causal=causal)
        o2, l2 = attn_fwd_ex(*(_bshd_view(t) for t in (q, k, v)), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp16_bshd_full_size_sampled(orc):
    """mha_l2k's shape in fp16 with [B, S, H, d] storage, sampled rows."""
    w = WORKLOADS["mha_l2k"]
    print(f"[case] fp16 bshd {w.as_dict()}", flush=True)
    q, k, v = (t.float().to(torch.float16)
               for t in make_qkv(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.dqk, w.dv, w.seed))
    qd, kd, vd = (_bshd_view(t.to(DEV)) for t in (q, k, v))
    o, lse = attn_fwd_ex(qd, kd, vd, causal=w.causal)
    torch.cuda.synchronize()
    rows = sample_rows(w.B, w.Hq, w.Lq, 256, seed=w.seed)
    og, lg = gather_rows(o, lse, rows)
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=w.causal, rows=rows.numpy())
    assert_parity("fp16 bshd mha_l2k", og, lg, o_ref, l_ref)
    assert torch.isfinite(o).all().item()
