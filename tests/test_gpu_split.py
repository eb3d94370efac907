"""GPU parity of the split-key path (per-split states and their merge) against
the fp64 oracle, through the C ABI.  Needs an MI355X."""
import numpy as np
import pytest
import torch

from exact_attention_forward_02_amd import (attn_fwd, attn_fwd_split, attn_fwd_splitkv,
                                            attn_merge, split_keys)
from exact_attention_forward_02_amd.inputs import make_qkv, sample_rows
from parity import assert_parity, gather_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# B, Hq, Hkv, Lq, Lk, dqk, dv, causal, q_mult, n_split
SHAPES = [
    (1, 2, 2, 200, 700, 128, 128, False, 1.0, 4),
    (1, 2, 2, 300, 300, 128, 128, True, 1.0, 3),     # splits past the diagonal are empty
    (2, 8, 2, 130, 517, 128, 128, True, 1.0, 5),     # GQA 4, ragged Lk
    (1, 6, 3, 257, 129, 64, 64, True, 1.0, 2),       # Lq > Lk: rows with no key anywhere
    (1, 3, 1, 100, 1000, 192, 128, False, 1.0, 7),   # (192,128), one head per workgroup
    (1, 4, 4, 64, 640, 64, 64, False, 6.0, 10),      # Q x 6: rescales inside each split
    (1, 2, 2, 50, 100, 128, 128, False, 1.0, 8),     # more splits than key blocks
]


def _ids(s):
    return "x".join(map(str, s))


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_split_states_match_the_oracle_per_segment(orc, shape):
    """Split s's fp32 state equals the definition restricted to its keys."""
    B, Hq, Hkv, Lq, Lk, dqk, dv, causal, qm, n = shape
    print(f"[case] split states {shape}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, dqk, dv, seed=hash(shape) % 10007, q_mult=qm)
    o_part, lse_part = attn_fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), n, causal=causal)
    torch.cuda.synchronize()
    w = split_keys(Lk, n)
    for s in range(n):
        o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal, k_range=(s * w, (s + 1) * w))
        og = o_part[s].reshape(-1, dv).cpu()
        lg = lse_part[s].reshape(-1).cpu()
        assert_parity(f"split {s} of {shape}", og, lg, o_ref, l_ref)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_split_then_merge_matches_the_definition(orc, shape):
    B, Hq, Hkv, Lq, Lk, dqk, dv, causal, qm, n = shape
    print(f"[case] split + merge {shape}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, dqk, dv, seed=hash(shape) % 10007, q_mult=qm)
    o, lse = attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), n, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal)
    assert_parity(f"merged {shape}", o.reshape(-1, dv).cpu(), lse.reshape(-1).cpu(), o_ref, l_ref)


def test_merge_kernel_on_oracle_states(orc):
    """The merge kernel alone: exact segment states from the oracle (rounded
    to fp32) in, the oracle's own merge of the same states as the reference."""
    B, Hq, Hkv, Lq, Lk, dqk, dv, causal = 1, 4, 2, 96, 900, 64, 64, True
    q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, dqk, dv, seed=21, q_mult=6.0)
    cuts = (0, 5, 300, 301, 899, 900, 1200)   # includes one-key and empty segments
    parts = [orc.attn_rows(q, k, v, causal=causal, k_range=(a, b))
             for a, b in zip(cuts[:-1], cuts[1:])]
    op = np.stack([p[0] for p in parts])
    lp = np.stack([p[1] for p in parts])
    o_ref, l_ref = orc.merge(op, lp)
    o, lse = attn_merge(torch.from_numpy(op.astype(np.float32)).to(DEV),
                        torch.from_numpy(lp.astype(np.float32)).to(DEV))
    torch.cuda.synchronize()
    st = assert_parity("merge kernel", o.cpu(), lse.cpu(), o_ref, l_ref)
    assert st["empty_rows"] == 0


def test_one_split_equals_the_fused_forward():
    """n_split = 1 is the whole key range: the merged result is attn_fwd's,
    bit for bit (the merge of one state multiplies by exp(0) = 1)."""
    q, k, v = make_qkv(2, 8, 2, 333, 555, 128, 128, seed=31)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        o1, l1 = attn_fwd(qd, kd, vd, causal=causal)
        o2, l2 = attn_fwd_splitkv(qd, kd, vd, 1, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_shape_sampled(orc, causal):
    """A decode-like shape (few query rows, long keys, many splits) at full
    size, checked on sampled rows and on every row being finite."""
    B, Hq, Hkv, Lq, Lk, d = 4, 32, 8, 4, 32768, 128
    n = 32
    print(f"[case] decode B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} d{d} splits {n} causal={causal}",
          flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, d, d, seed=41)
    o, lse = attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), n, causal=causal)
    torch.cuda.synchronize()
    rows = sample_rows(B, Hq, Lq, 64, seed=41)
    og, lg = gather_rows(o, lse, rows)
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal, rows=rows.numpy())
    assert_parity(f"decode causal={causal}", og, lg, o_ref, l_ref)
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()


def test_split_many_tiles_sampled(orc):
    """768 tiles of 16 splits: workgroups loop over tiles of different splits."""
    B, Hq, Hkv, Lq, Lk, d, n = 2, 8, 8, 600, 3000, 128, 16
    print(f"[case] split B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} d{d} splits {n}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Lq, Lk, d, d, seed=51)
    for causal in (False, True):
        o, lse = attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), n, causal=causal)
        torch.cuda.synchronize()
        rows = sample_rows(B, Hq, Lq, 128, seed=52)
        og, lg = gather_rows(o, lse, rows)
        o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal, rows=rows.numpy())
        assert_parity(f"split many tiles causal={causal}", og, lg, o_ref, l_ref)


@pytest.mark.parametrize("name", ["decode_l32k", "decode_dsv3_l32k"])
def test_decode_workload_in_bench_configuration(orc, name):
    """The decode workloads with the 4 key splits bench.py times: sampled rows
    against the oracle."""
    from exact_attention_forward_02_amd.inputs import WORKLOADS, workload_qkv

    w = WORKLOADS[name]
    print(f"[case] {w.name} {w.as_dict()} splits 4", flush=True)
    q, k, v = workload_qkv(w)
    o, lse = attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), 4, causal=w.causal)
    torch.cuda.synchronize()
    rows = sample_rows(w.B, w.Hq, w.Lq, 96, seed=w.seed)
    og, lg = gather_rows(o, lse, rows)
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=w.causal, rows=rows.numpy())
    assert_parity(w.name, og, lg, o_ref, l_ref)
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
