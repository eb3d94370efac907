"""Seeded synthetic inputs and the named workloads.

This module holds no attention arithmetic.  It is the only code that both the
GPU path and the CPU oracle are fed from: tests, the benchmark and the smoke
check draw Q, K, V here and hand the same tensors to both sides.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws Q,
then K, then V as float32 N(0, 1) (Q optionally multiplied by a constant in
float32), each rounded to bfloat16 with round-to-nearest-even.  Layout is
[B, H, L, d], contiguous.

Variable-length batches pack their sequences along the token axis ([T, H, d],
token-major).  Their lengths come from the same kind of seeded generator:
lengths drawn uniformly from [lo, hi] until the tokens reach the total, the
last one cut so the total is exact.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    dqk: int
    dv: int
    causal: bool
    seed: int
    q_mult: float = 1.0

    def flops(self) -> float:
        """Algorithmic FLOPs: 2*B*Hq*Lq*Lk*(dqk+dv), halved under the causal mask."""
        f = 2.0 * self.B * self.Hq * self.Lq * self.Lk * (self.dqk + self.dv)
        return f / 2.0 if self.causal else f

    def valid_pairs(self) -> int:
        """Exact count of visible (query, key) pairs per (b, h)."""
        if not self.causal:
            return self.Lq * self.Lk
        off = self.Lk - self.Lq
        total = 0
        for i in range(self.Lq):
            total += max(0, min(self.Lk, i + off + 1))
        return total

    def min_hbm_bytes(self) -> int:
        """Q, K, V read once and O, lse written once."""
        q = self.B * self.Hq * self.Lq * self.dqk * 2
        k = self.B * self.Hkv * self.Lk * self.dqk * 2
        v = self.B * self.Hkv * self.Lk * self.dv * 2
        o = self.B * self.Hq * self.Lq * self.dv * 2
        lse = self.B * self.Hq * self.Lq * 4
        return q + k + v + o + lse

    def as_dict(self) -> dict:
        return asdict(self)


# The five workloads of the study (sizes as the attention-forward benchmark
# grid describes them: 32k total tokens at hidden 2048, long causal sequences,
# a grouped-query case and the (192, 128) head shape).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 256, 256, 64, 64, False, seed=1),
    "tiny_q6": Workload("tiny_q6", 1, 1, 1, 256, 256, 64, 64, False, seed=1, q_mult=6.0),
    "mha_l2k": Workload("mha_l2k", 16, 16, 16, 2048, 2048, 128, 128, False, seed=2),
    "causal_l8k": Workload("causal_l8k", 4, 16, 16, 8192, 8192, 128, 128, True, seed=3),
    "gqa_l16k": Workload("gqa_l16k", 2, 32, 8, 16384, 16384, 128, 128, True, seed=4),
    "dsv3_l32k": Workload("dsv3_l32k", 1, 16, 16, 32768, 32768, 192, 128, True, seed=5),
    # one decode step over a long key cache (split-key path): B8 Hq32 Hkv8,
    # one new query per sequence, 32k cached keys
    "decode_l32k": Workload("decode_l32k", 8, 32, 8, 1, 32768, 128, 128, False, seed=6),
    # one decode step with the (192, 128) head shape: B8 H16, one new query per
    # sequence, 32k cached keys per head
    "decode_dsv3_l32k": Workload("decode_dsv3_l32k", 8, 16, 16, 1, 32768, 192, 128, False,
                                 seed=9),
    # one GPU's share of dsv3_l32k when its 16 heads are sharded over 8 GPUs
    "dsv3_l32k_h2": Workload("dsv3_l32k_h2", 1, 2, 2, 32768, 32768, 192, 128, True, seed=8),
}


def make_qkv(B: int, Hq: int, Hkv: int, Lq: int, Lk: int, dqk: int, dv: int,
             seed: int, q_mult: float = 1.0):
    """Seeded bf16 CPU tensors q [B,Hq,Lq,dqk], k [B,Hkv,Lk,dqk], v [B,Hkv,Lk,dv]."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((B, Hq, Lq, dqk), generator=g, dtype=torch.float32)
    if q_mult != 1.0:
        q.mul_(float(q_mult))
    q = q.to(torch.bfloat16)
    k = torch.randn((B, Hkv, Lk, dqk), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Lk, dv), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v


def make_qkv_fp16(B: int, Hq: int, Hkv: int, Lq: int, Lk: int, dqk: int, dv: int, seed: int):
    """Seeded fp16 CPU tensors with the full fp16 precision: float32 N(0, 1)
    draws (Q, then K, then V) rounded to float16 with RNE, so most values carry
    mantissa bits that bf16 cannot hold."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((B, Hq, Lq, dqk), generator=g, dtype=torch.float32).to(torch.float16)
    k = torch.randn((B, Hkv, Lk, dqk), generator=g, dtype=torch.float32).to(torch.float16)
    v = torch.randn((B, Hkv, Lk, dv), generator=g, dtype=torch.float32).to(torch.float16)
    return q, k, v


@dataclass(frozen=True)
class VarlenWorkload:
    """A packed batch of sequences of different lengths (self-attention: each
    sequence's queries attend its own keys, Lq_s = Lk_s)."""
    name: str
    total: int      # tokens over all sequences
    lo: int         # sequence lengths are drawn uniformly from [lo, hi]
    hi: int
    Hq: int
    Hkv: int
    dqk: int
    dv: int
    causal: bool
    seed: int

    def lengths(self):
        return seq_lengths(self.total, self.lo, self.hi, self.seed)

    def flops(self) -> float:
        """Algorithmic FLOPs: sum over sequences of 2*Hq*L_s^2*(dqk+dv), halved
        under the causal mask."""
        f = sum(2.0 * self.Hq * L * L * (self.dqk + self.dv) for L in self.lengths())
        return f / 2.0 if self.causal else f

    def min_hbm_bytes(self) -> int:
        T = self.total
        return (T * self.Hq * self.dqk * 2 + T * self.Hkv * (self.dqk + self.dv) * 2
                + T * self.Hq * self.dv * 2 + T * self.Hq * 4)

    def as_dict(self) -> dict:
        return asdict(self)


# 32k tokens at hidden 2048 (16 heads of 128) as one packed batch of causal
# sequences of 256 to 8192 tokens
VARLEN_WORKLOADS = {
    "varlen_32k": VarlenWorkload("varlen_32k", 32768, 256, 8192, 16, 16, 128, 128, True, seed=7),
}


def seq_lengths(total: int, lo: int, hi: int, seed: int):
    """Seeded sequence lengths: uniform integers in [lo, hi] drawn until they
    reach `total` tokens, the last one cut so that they sum to `total`."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    lens, acc = [], 0
    while acc < total:
        n = int(torch.randint(lo, hi + 1, (1,), generator=g).item())
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def make_varlen_qkv(lens_q, lens_k, Hq: int, Hkv: int, dqk: int, dv: int, seed: int,
                    q_mult: float = 1.0):
    """Seeded bf16 CPU tensors of a packed batch: q [Tq, Hq, dqk], k [Tk, Hkv, dqk],
    v [Tk, Hkv, dv], and the int64 offsets cu_q, cu_k (n_seq + 1 entries each;
    sequence s owns tokens [cu[s], cu[s+1]))."""
    if len(lens_q) != len(lens_k) or not lens_q:
        raise ValueError("lens_q and lens_k must list the same, nonzero number of sequences")
    cu_q = torch.tensor([0] + list(lens_q), dtype=torch.int64).cumsum(0)
    cu_k = torch.tensor([0] + list(lens_k), dtype=torch.int64).cumsum(0)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((Tq, Hq, dqk), generator=g, dtype=torch.float32)
    if q_mult != 1.0:
        q.mul_(float(q_mult))
    q = q.to(torch.bfloat16)
    k = torch.randn((Tk, Hkv, dqk), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((Tk, Hkv, dv), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, cu_q, cu_k


def varlen_workload_qkv(w: VarlenWorkload):
    lens = w.lengths()
    return make_varlen_qkv(lens, lens, w.Hq, w.Hkv, w.dqk, w.dv, w.seed)


def workload_qkv(w: Workload):
    return make_qkv(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.dqk, w.dv, w.seed, w.q_mult)


def sample_rows(B: int, Hq: int, Lq: int, n: int, seed: int = 0):
    """n distinct flat row indices (b*Hq + h)*Lq + i, always including the first
    and last position of the first and last head, drawn with a fixed seed."""
    total = B * Hq * Lq
    if n >= total:
        return torch.arange(total, dtype=torch.int64)
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    picked = torch.randperm(total, generator=g)[:n]
    fixed = torch.tensor([0, Lq - 1, total - Lq, total - 1], dtype=torch.int64)
    rows = torch.unique(torch.cat([fixed, picked]))
    return rows
