"""GPU parity of the key-streaming decode kernel (attn_fwd_decode: at most 16
query rows per K/V head) against the fp64 oracle, through the C ABI: each
split's state against the oracle's state of the same key segment, and split
+ merge against the whole definition.  Needs an MI355X."""
import pytest
import torch

from exact_attention_forward_02_amd import (attn_fwd_decode, attn_fwd_split, attn_merge,
                                            split_keys)
from exact_attention_forward_02_amd.inputs import make_qkv
from parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# B, Hq, Hkv, Lq, Lk, (d_qk, d_v), causal, q_mult, n_split
SHAPES = [
    (1, 1, 1, 1, 1000, (128, 128), False, 1.0, 3),    # one row per K/V head, ragged last split
    (2, 8, 2, 1, 777, (128, 128), False, 1.0, 4),     # GQA 4: 4 rows
    (1, 16, 2, 2, 300, (64, 64), True, 1.0, 2),       # 16 rows, two positions under the mask
    (1, 12, 4, 5, 129, (128, 128), True, 1.0, 1),     # 15 rows, one split
    (1, 4, 1, 4, 3, (64, 64), True, 1.0, 2),          # Lq > Lk: rows without keys; an empty split
    (2, 16, 1, 1, 5000, (128, 128), False, 6.0, 7),   # MQA 16 rows, Q x 6: references move
    (1, 8, 8, 2, 65, (64, 64), False, 1.0, 9),        # more splits than key blocks
    (3, 6, 3, 3, 2049, (128, 128), True, 1.0, 5),     # 6 rows, tails in every wave's run
    (2, 4, 4, 1, 3001, (192, 128), False, 1.0, 4),    # the (192, 128) head shape, one row
    (1, 16, 2, 2, 700, (192, 128), True, 6.0, 3),     # (192, 128), 16 rows, Q x 6
]


def _ids(s):
    return "x".join(map(str, s))


def _inputs(shape):
    B, Hq, Hkv, Lq, Lk, (dqk, dv), causal, qm, n = shape
    return make_qkv(B, Hq, Hkv, Lq, Lk, dqk, dv, seed=(B * 131 + Hq * 17 + Lq * 7 + Lk) % 10007,
                    q_mult=qm)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_decode_split_states_match_the_oracle(orc, shape):
    B, Hq, Hkv, Lq, Lk, (dqk, d), causal, qm, n = shape
    print(f"[case] decode states {shape}", flush=True)
    q, k, v = _inputs(shape)
    o_part, lse_part = attn_fwd_decode(q.to(DEV), k.to(DEV), v.to(DEV), n, causal=causal)
    torch.cuda.synchronize()
    w = split_keys(Lk, n)
    for s in range(n):
        o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal, k_range=(s * w, (s + 1) * w))
        assert_parity(f"decode split {s} of {shape}", o_part[s].reshape(-1, d).cpu(),
                      lse_part[s].reshape(-1).cpu(), o_ref, l_ref)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_decode_then_merge_matches_the_definition(orc, shape):
    B, Hq, Hkv, Lq, Lk, (dqk, d), causal, qm, n = shape
    print(f"[case] decode + merge {shape}", flush=True)
    q, k, v = _inputs(shape)
    o_part, lse_part = attn_fwd_decode(q.to(DEV), k.to(DEV), v.to(DEV), n, causal=causal)
    o, lse = attn_merge(o_part, lse_part)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal)
    assert_parity(f"decode merged {shape}", o.reshape(-1, d).cpu(), lse.reshape(-1).cpu(),
                  o_ref, l_ref)


def test_split_entry_point_selects_the_decode_kernel():
    """attn_fwd_split on a shape with <= 16 rows per K/V head returns the decode
    kernel's states bit for bit."""
    q, k, v = make_qkv(2, 8, 2, 1, 3000, 128, 128, seed=77)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = attn_fwd_split(qd, kd, vd, 6, causal=False)
    o2, l2 = attn_fwd_decode(qd, kd, vd, 6, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
