"""Planted mistakes in copies of the oracle must each trip at least one pin.

Each mutation rewrites one line of oracle/attn_oracle.c (the committed source
is never touched), builds the copy into a temporary library and runs every pin
against it.  A mutation that no pin notices would mean the pins leave that
part of the oracle unchecked.  CPU only.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins

MUTATIONS = {
    "gqa_head_mapping": ("int64_t hk = h / group;", "int64_t hk = h % group;"),
    "causal_top_left": ("int64_t last = i + d->Lk - d->Lq;", "int64_t last = i;"),
    "dropped_scale": ("s[j] = d->scale * dot;", "s[j] = dot;"),
    "exp_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "lse_dropped_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "transposed_k": ("            dot += qd[c] * widen(d, kj[c]);\n        s[j]",
                     "            dot += qd[c] * widen(d, rr.kh[c * d->Lk + j]);\n        s[j]"),
    "value_index": ("o_row[c] += p * widen(d, vj[c]);",
                    "o_row[c] += p * widen(d, vj[d->dv - 1 - c]);"),
    "bf16_widening": ("uint32_t word = ((uint32_t)bits) << 16;",
                      "uint32_t word = ((uint32_t)bits) << 15;"),
    "threshold_not_strict": ("if (delta < -tau)", "if (delta <= -tau)"),
    "rescale_dropped": ("acc_scale = exp2((s->ref - cand) * scale_log2);", "acc_scale = 1.0;"),
    "online_lse_units": ("lse[t] = (mode == 0) ? s->ref + log(s->l)\n                                         : scale * s->ref + log(s->l);",
                         "lse[t] = s->ref + log(s->l);"),
    "group_decision_ignored": ("int do_switch = (mode == 1) ? wants[a] : any_switch;",
                               "int do_switch = wants[a];"),
    "first_block_not_adopted": ("s->ref = bmax[a];\n                acc_scale = 1.0;",
                                "s->ref = 0.0;\n                acc_scale = 1.0;"),
    "segment_start_ignored": ("    if (j0 < 0)\n        j0 = 0;", "    j0 = 0;"),
    "merge_unweighted": ("double beta = exp(mb - mm);", "double beta = 1.0;"),
    "merge_old_state_not_rescaled": ("u[c] = alpha * u[c] + beta * ob[c];",
                                     "u[c] = u[c] + beta * ob[c];"),
    "merge_lse_without_max": ("lse[r] = m + log(l);", "lse[r] = log(l);"),
    "fp16_exponent_bias": ("v = ldexp((double)(1024 + f), e - 25);",
                           "v = ldexp((double)(1024 + f), e - 24);"),
    "fp16_subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "fp16_sign_dropped": ("return (bits & 0x8000) ? -v : v;", "return v;"),
    "bwd_delta_dropped": ("const double ds = p[j] * (dp[j] - di);",
                          "const double ds = p[j] * dp[j];"),
    "bwd_dv_transposed": ("dvh[j * dv + c] += p[j] * gd[c];",
                          "dvh[j * dv + c] += p[j] * gd[dv - 1 - c];"),
    "bwd_dk_unscaled": ("dkh[j * dqk + c] += scale * ds * qd[c];",
                        "dkh[j * dqk + c] += ds * qd[c];"),
    "bwd_dk_one_thread_partial": ("for (int th = 0; th < nthr; ++th)\n                acc += part_k",
                                  "for (int th = 0; th < 1; ++th)\n                acc += part_k"),
    "bwd_gqa_first_head_only": ("for (int64_t hi = 0; hi < group * Lq; ++hi) {",
                                "for (int64_t hi = 0; hi < Lq; ++hi) {"),
    "fp16_read_as_bf16": ("return d->elem == ELEM_FP16 ? fp16_bits_to_double(bits) : "
                          "bf16_bits_to_double(bits);", "return bf16_bits_to_double(bits);"),
    "varlen_keys_at_query_offset": (
        "const uint16_t* kj = k + ((cu_k[sq] + j) * Hkv + kvh) * dqk;",
        "const uint16_t* kj = k + ((cu_q[sq] + j) * Hkv + kvh) * dqk;"),
    "varlen_causal_top_left": ("const int64_t last = i + Lk - Lq;",
                               "const int64_t last = i;"),
    "varlen_sequence_boundary": ("while (cu_q[sq + 1] <= tok)", "while (cu_q[sq + 1] < tok)"),
    "varlen_value_head": ("const uint16_t* vj = v + ((cu_k[sq] + j) * Hkv + kvh) * dv;",
                          "const uint16_t* vj = v + ((cu_k[sq] + j) * Hkv + 0) * dv;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    with open(oracle.SOURCE, encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path_c = os.path.join(tmp, "mutant.c")
        with open(path_c, "w", encoding="utf-8") as f:
            f.write(src.replace(old, new))
        lib = oracle.build(path_c, os.path.join(tmp, "libmutant.so"))
        mutant = oracle.Oracle(lib)
        tripped = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError):
                tripped.append(pin.__name__)
        assert tripped, f"no pin notices the planted mistake {name!r}"
