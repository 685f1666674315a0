"""CPU-only: the oracle against its pins, and planted mistakes against the pins.

The planted-mistake test copies the oracle's C source, changes one thing (a
dropped term, a wrong sign or index, a transposed operand, a wrong format
constant), builds it with gcc into a temporary directory and runs the same
battery: every such build must fail at least one check.  This shows that the
pins would catch each of those mistakes in the real oracle.
"""
from __future__ import annotations

import os
import shutil
import tempfile

import pytest

import oracle_pins
from oracle import oracle as oracle_mod


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle, check):
    check(oracle)


# (label, original text, replacement) -- each applied alone to a copy.
MUTATIONS = [
    ("drop_softmax_scale", "double s = P->scale * P->qs * P->ks * dot;",
     "double s = P->qs * P->ks * dot;"),
    ("drop_q_descale", "double s = P->scale * P->qs * P->ks * dot;",
     "double s = P->scale * P->ks * dot;"),
    ("drop_v_descale", "o_row[e] += p * P->vs * elem(", "o_row[e] += p * elem("),
    ("causal_off_by_one", "if (wr >= 0 && j > d0 + wr) return 0;",
     "if (wr >= 0 && j >= d0 + wr) return 0;"),
    ("top_left_causal", "int d0 = i + sk - sq;", "int d0 = i;"),
    ("window_left_off_by_one", "if (wl >= 0 && j < d0 - wl) return 0;",
     "if (wl >= 0 && j <= d0 - wl) return 0;"),
    ("gqa_modulo_mapping", "int hk = h / (P->hq / P->hkv);", "int hk = h % P->hkv;"),
    ("lse_without_max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("lse_log2", "*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    ("k_row_ignores_sequence_start",
     "int64_t krow = ((int64_t)(ks0 + j) * P->hkv + hk) * P->dqk;",
     "int64_t krow = ((int64_t)(j) * P->hkv + hk) * P->dqk;"),
    ("v_row_uses_q_head",
     "int64_t vrow = ((int64_t)(ks0 + j) * P->hkv + hk) * P->dv;",
     "int64_t vrow = ((int64_t)(ks0 + j) * P->hkv + (h % P->hkv)) * P->dv;"),
    ("transposed_k_index",
     "dot += elem(P->q, P->dtype, qrow + d) * elem(P->k, P->dtype, krow + d);",
     "dot += elem(P->q, P->dtype, qrow + d) * elem(P->k, P->dtype, krow + (d * 7) % P->dqk);"),
    ("unnormalised_probabilities", "double p = exp(scores[j - klo] - m) / l;",
     "double p = exp(scores[j - klo] - m);"),
    ("no_key_rows_written", "if (sk == 0) continue; /* rows of a query sequence with no keys: untouched */",
     "/* mutated */"),
    ("split_range_short", "khi = klo + chunk;", "khi = klo + chunk - 1;"),
    ("combine_weights_vs_max",
     "double w = exp(lse_part[((int64_t)s * hq + h) * tq + t] - total);",
     "double w = exp(lse_part[((int64_t)s * hq + h) * tq + t] - L);"),
    ("combine_drops_last_split", "int nsb = (sk + chunk - 1) / chunk;",
     "int nsb = sk / chunk;"),
    ("rows_driver_wrong_sequence",
     "while (b < batch && seq_start(cu_q, seqlen_q, b) + seq_len(cu_q, seqlen_q, b) <= t) ++b;",
     "while (b < batch && seq_start(cu_q, seqlen_q, b) + seq_len(cu_q, seqlen_q, b) < t) ++b;"),
    ("e4m3_bias", "v = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("f16_subnormal_scale", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    ("bf16_shift", "uint32_t u = ((uint32_t)b) << 16;", "uint32_t u = ((uint32_t)b) << 15;"),
]


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("label,orig,repl", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(mutant_dir, label, orig, repl):
    src = open(oracle_mod.SRC).read()
    assert src.count(orig) == 1, f"mutation anchor not unique/present: {label}"
    path = os.path.join(mutant_dir, f"{label}.c")
    with open(path, "w") as f:
        f.write(src.replace(orig, repl))
    lib = oracle_mod.build(path, os.path.join(mutant_dir, f"lib{label}.so"))
    mutant = oracle_mod.load(lib)
    failures = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mutant)
        except AssertionError as e:  # the pin caught it
            failures.append(f"{check.__name__}: {str(e)[:80]}")
        except ValueError as e:
            failures.append(f"{check.__name__}: rejected ({e})")
    assert failures, f"planted mistake '{label}' passed every pin"
