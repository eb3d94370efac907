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
from parity import U_BF16, assert_parity, half_ulp_bf16

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
    starts = (0, mid, Lk - w)
    for causal in (False, True):
        o, lse = attn_fwd(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = orc.attn_rows(q, k, v, causal=causal)
        bound = _bound(q, k, v, starts, w, Lk, causal, o_ref, l_ref)
        assert_parity(f"largest head causal={causal}", o.reshape(-1, d).cpu(),
                      lse.reshape(-1).cpu(), o_ref, l_ref, bound=bound)
        assert np.isfinite(lse.cpu().numpy()).all()


def _bound(q, k, v, starts, w, Lk, causal, o_ref, l_ref):
    """Per-element bound for this input: the bf16-weight bound of the window
    keys plus the zero keys (score 0, V = 0), and the fp32 accumulation of the
    numerator and of the denominator over Lk / 16 MFMA steps each (recursive
    summation: at most gamma_n * sum_j w_j |v_j| relative to O's scale, with
    gamma_n = n u32 / (1 - n u32), u32 = 2^-24).  Rows whose best key sits on a
    near tie with large, opposite V values pass 1e-2 (measured 1.569e-2, one
    bf16 ulp at |O| in [2, 4)); each element is held to max(1e-2, bound)."""
    d = q.shape[-1]
    Lq = q.shape[2]
    scale = 1.0 / np.sqrt(d)
    keys = np.concatenate([np.arange(s, s + w) for s in starts])
    kw = k[0, 0, keys].double().numpy()
    vw = v[0, 0, keys].double().numpy()
    qq = q[0, 0].double().numpy()
    s = scale * qq @ kw.T                           # [Lq, 3w] window scores
    i = np.arange(Lq)[:, None]
    last = (i + Lk - Lq) if causal else np.full((Lq, 1), Lk - 1)
    vis = keys[None, :] <= last
    lse = np.asarray(l_ref)[:, None]
    ww = np.where(vis, np.exp(s - lse), 0.0)        # weights of the window keys
    n_zero = (last[:, 0] + 1) - vis.sum(axis=1)     # visible keys outside the windows
    w0 = n_zero * np.exp(-lse[:, 0])                # their total weight (score 0)
    o = np.asarray(o_ref)
    n_steps = Lk / 16.0
    gamma = n_steps * 2.0 ** -24 / (1.0 - n_steps * 2.0 ** -24)
    spread = np.einsum("rk,rkc->rc", ww, np.abs(vw[None] - o[:, None])) + w0[:, None] * np.abs(o)
    mass = ww @ np.abs(vw)
    pre = U_BF16 / (1.0 - U_BF16) * spread + 2.0 * gamma * mass
    return pre + half_ulp_bf16(np.abs(o) + pre)
