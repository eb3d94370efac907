"""A seeded sweep of small random shapes through every forward entry point,
against the fp64 oracle: the fused kernel (attn_fwd), the split-key path
(attn_fwd_splitkv, which takes the decode kernel for <= 16 rows per K/V
head) and packed variable-length batches (attn_fwd_varlen).  The shapes mix
what the hand-picked cases test one at a time: single rows and keys, ragged
tails, Lq > Lk under the causal mask, grouped-query ratios up to 16 and all
three head shapes.  Needs an MI355X."""
import random

import pytest
import torch

from exact_attention_forward_02_amd import attn_fwd, attn_fwd_splitkv, attn_fwd_varlen
from exact_attention_forward_02_amd.inputs import make_qkv, make_varlen_qkv
from parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DIMS = [(64, 64), (128, 128), (192, 128)]


def _shapes(seed, n):
    rnd = random.Random(seed)
    out = []
    for _ in range(n):
        Hkv = rnd.choice([1, 1, 2, 3, 4])
        G = rnd.choice([1, 2, 3, 4, 8, 16])
        Lq = rnd.choice([1, 2, 5, 31, 64, 65, 200, 257, 511])
        Lk = rnd.choice([1, 3, 63, 64, 65, 130, 300, 700])
        dqk, dv = rnd.choice(DIMS)
        out.append((rnd.choice([1, 2]), Hkv * G, Hkv, Lq, Lk, dqk, dv, rnd.random() < 0.5))
    return out


DENSE = _shapes(2024, 24)


@pytest.mark.parametrize("shape", DENSE, ids=lambda s: "x".join(map(str, s)))
def test_random_shape_fused(orc, shape):
    B, Hq, Hkv, Lq, Lk, dqk, dv, causal = shape
    print(f"[case] fused {shape}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, dqk, dv, seed=hash(shape) % 100003)
    o, lse = attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal)
    assert_parity(f"fused {shape}", o.reshape(-1, dv).cpu(), lse.reshape(-1).cpu(), o_ref, l_ref)


SPLIT = [s for s in _shapes(77, 40) if s[5] == s[6] and s[5] in (64, 128)][:16]
# the (192, 128) head shape through the same path: the decode kernel where a
# K/V head serves at most 16 rows, the fused kernel's split path elsewhere
SPLIT_WIDE = [s for s in _shapes(91, 80) if s[5] == 192][:10]


def _check_split(orc, shape):
    B, Hq, Hkv, Lq, Lk, dqk, dv, causal = shape
    n = 1 + hash(shape) % 7
    print(f"[case] split {shape} n={n} rows/head={Lq * Hq // Hkv}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, dqk, dv, seed=hash(shape) % 100019)
    o, lse = attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), n, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal)
    assert_parity(f"split {shape} n={n}", o.reshape(-1, dv).cpu(), lse.reshape(-1).cpu(), o_ref,
                  l_ref)


@pytest.mark.parametrize("shape", SPLIT, ids=lambda s: "x".join(map(str, s)))
def test_random_shape_split(orc, shape):
    _check_split(orc, shape)


@pytest.mark.parametrize("shape", SPLIT_WIDE, ids=lambda s: "x".join(map(str, s)))
def test_random_shape_split_wide(orc, shape):
    _check_split(orc, shape)


def _varlen_cases(seed, n):
    rnd = random.Random(seed)
    out = []
    for _ in range(n):
        Hkv = rnd.choice([1, 2, 4])
        G = rnd.choice([1, 2, 4, 8])
        dqk, dv = rnd.choice(DIMS)
        ns = rnd.randint(1, 6)
        lq = [rnd.choice([0, 1, 7, 64, 100, 300]) for _ in range(ns)]
        same = rnd.random() < 0.5
        lk = lq[:] if same else [rnd.choice([0, 1, 9, 64, 130, 400]) for _ in range(ns)]
        if sum(lq) == 0:
            lq[0] = 5
        out.append((tuple(lq), tuple(lk), Hkv * G, Hkv, dqk, dv, rnd.random() < 0.5))
    return out


VARLEN = _varlen_cases(4242, 12)


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"{len(c[0])}seq-{c[2]}-{c[3]}-{c[4]}-"
                                                       f"{c[6]}-{sum(c[0])}")
def test_random_varlen(orc, case):
    lq, lk, Hq, Hkv, dqk, dv, causal = case
    print(f"[case] varlen {case}", flush=True)
    q, k, v, cu_q, cu_k = make_varlen_qkv(list(lq), list(lk), Hq, Hkv, dqk, dv,
                                          seed=sum(lq) * 31 + sum(lk))
    if k.shape[0] == 0:  # no key in any sequence: one zero key row keeps the tensors non-empty
        k = torch.zeros((1, Hkv, dqk), dtype=torch.bfloat16)
        v = torch.zeros((1, Hkv, dv), dtype=torch.bfloat16)
        cu_k = cu_k.clone()
        cu_k[-1] = 1
    o, lse = attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q, cu_k, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_varlen(q, k, v, cu_q, cu_k, causal=causal)
    assert_parity(f"varlen {case}", o.permute(1, 0, 2).reshape(-1, dv).cpu(),
                  lse.reshape(-1).cpu(), o_ref, l_ref)
