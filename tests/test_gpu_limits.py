"""GPU parity at the largest size the forward accepts: one K (and V) head of
Lk = 8388607 keys at d = 128, the longest whose rows span less than 2^31
bytes (the kernel addresses a head with 32-bit buffer offsets; one key more
is rejected with ATTN_ERR_TOO_LARGE before any launch).  Needs an MI355X and
about 4.3 GB of device memory."""
import numpy as np
import pytest
import torch

from exact_attention_forward_02_amd import attn_fwd
from exact_attention_forward_02_amd.inputs import make_qkv
from parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LK_MAX = (2 ** 31 - 1) // 256  # keys of 256 bytes (d = 128 bf16) below 2^31 bytes


def test_largest_kv_head(orc):
    d, Lq, Lk = 128, 64, LK_MAX
    w = 4096  # seeded random key windows at the start, the middle and the very end
    print(f"[case] largest head: Lq={Lq} Lk={Lk} d={d}", flush=True)
    q, kr, vr = make_qkv(1, 1, 1, Lq, 3 * w, d, d, seed=31, q_mult=6.0)
    k = torch.zeros((1, 1, Lk, d), dtype=torch.bfloat16)
    v = torch.zeros((1, 1, Lk, d), dtype=torch.bfloat16)
    mid = Lk // 2
    for i, start in enumerate((0, mid, Lk - w)):
        k[0, 0, start:start + w] = kr[0, 0, i * w:(i + 1) * w]
        v[0, 0, start:start + w] = vr[0, 0, i * w:(i + 1) * w]
    # the last window decides the output of some rows (Q x 6 makes the random
    # keys dominate the zero ones)
    tail = k[0, 0, Lk - w:].double() @ q[0, 0].double().T
    rest = torch.cat([k[0, 0, :w], k[0, 0, mid:mid + w]]).double() @ q[0, 0].double().T
    wins = int((tail.max(0).values > rest.max(0).values).sum())
    print(f"[case] rows whose best key is in the last window: {wins}", flush=True)
    assert wins > 0
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        o, lse = attn_fwd(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal)
        assert_parity(f"largest head causal={causal}", o.reshape(-1, d).cpu(),
                      lse.reshape(-1).cpu(), o_ref, l_ref, stress=True)
        assert np.isfinite(lse.cpu().numpy()).all()
