"""The allocation-free backward entry point, attn_bwd_noalloc, through the C
ABI: its dq, dk and dv equal attn_bwd's bit for bit, on two calls in a row,
the second on a smaller problem (the static scratch keeps the first call's D
rows; each call must write every row it reads).  Needs an MI355X."""
import pytest
import torch

from exact_attention_forward_02_amd import attn_bwd, attn_bwd_noalloc, attn_fwd
from exact_attention_forward_02_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# B, Hq, Hkv, Lq, Lk, d, causal: the second is smaller in every dimension
CALLS = [(2, 8, 2, 700, 900, 128, True), (1, 4, 4, 300, 257, 64, False)]


def _problem(shape, seed):
    B, Hq, Hkv, Lq, Lk, d, causal = shape
    q, k, v = (t.to(DEV) for t in make_qkv(B, Hq, Hkv, Lq, Lk, d, d, seed=seed))
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn((B, Hq, Lq, d), generator=g).to(torch.bfloat16).to(DEV)
    o, lse = attn_fwd(q, k, v, causal=causal)
    return q, k, v, o, lse, dout


def test_noalloc_backward_equals_attn_bwd_twice():
    for i, shape in enumerate(CALLS):
        causal = shape[6]
        print(f"[case] attn_bwd_noalloc call {i + 1}: {shape}", flush=True)
        q, k, v, o, lse, dout = _problem(shape, seed=40 + i)
        dq, dk, dv, _ = attn_bwd(q, k, v, o, lse, dout, causal=causal)
        torch.cuda.synchronize()
        # outputs pre-filled with NaN: every element must be written
        nq, nk, nv = (torch.full_like(t, float("nan")) for t in (q, k, v))
        attn_bwd_noalloc(q, k, v, o, lse, dout, nq, nk, nv, causal=causal)
        torch.cuda.synchronize()
        for name, want, got in (("dq", dq, nq), ("dk", dk, nk), ("dv", dv, nv)):
            assert torch.equal(want, got), f"call {i + 1} {name} differs from attn_bwd"
        print(f"[parity] attn_bwd_noalloc call {i + 1}: dq, dk, dv bitwise equal to attn_bwd",
              flush=True)


def test_noalloc_backward_refuses_more_rows_than_its_scratch():
    from exact_attention_forward_02_amd import _binding

    q, k, v = (t.to(DEV) for t in make_qkv(1, 1, 1, 64, 64, 64, 64, seed=1))
    lib = _binding.library()
    rows_too_many = _binding.BWD_NOALLOC_MAX_ROWS + 1
    rc = lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), q.data_ptr(),
                              q.data_ptr(), q.data_ptr(), q.data_ptr(), k.data_ptr(),
                              v.data_ptr(), 1, rows_too_many, 1, 1, 64, 64, 64, 0, 0.125, None)
    assert _binding.status_string(rc).startswith("B * Hq * Lq exceeds")
