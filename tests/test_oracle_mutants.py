"""The pins catch plausible mistakes: each mutant is a copy of the oracle's C
source with one planted error, compiled with gcc and checked in a child
process against the CPU pins; a failing pin (or a crash) counts as caught."""

import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = [
    ("ties_to_higher_id", "return !isnan(a) && (isnan(b) || a > b);", "return !isnan(a) && (isnan(b) || a >= b);"),
    ("nan_ranks_first", "return !isnan(a) && (isnan(b) || a > b);", "return isnan(a) ? !isnan(b) : (!isnan(b) && a > b);"),
    ("nan_compares_as_is", "return !isnan(a) && (isnan(b) || a > b);", "return a > b;"),
    ("no_renormalisation", "w[t * k + j] = (float)(p[ids[t * k + j]] / sel);", "w[t * k + j] = (float)(p[ids[t * k + j]]);"),
    ("send_offsets_not_rank_based", "int32_t acc = (int32_t)(src * Tp * k);", "int32_t acc = 0;"),
    ("unstable_bucket_order", "int32_t c = cur[src * E + e]++;", "int32_t c = o->n[src * E + e] - 1 - cur[src * E + e]++;"),
    ("source_major_receive_order", "for (int64_t src = 0; src < P; ++src) { o->recv_off[e * P + src] = acc; acc += o->n[src * E + e]; }",
     "for (int64_t src = P - 1; src >= 0; --src) { o->recv_off[e * P + src] = acc; acc += o->n[src * E + e]; }"),
    ("tokens_round_robin_over_ranks", "o->n[(t / Tp) * E + ids[t * k + j]] += 1;", "o->n[(t % P) * E + ids[t * k + j]] += 1;"),
    ("combine_slot_swapped", "memcpy(comb + (t * s->k + m->slot) * s->H", "memcpy(comb + (t * s->k + (s->k - 1 - m->slot)) * s->H"),
    ("reduce_in_reverse_slot_order", "for (int64_t j = 0; j < k; ++j) {\n            float v = oracle_bf16_to_f32(comb[(t * k + j) * H + h]);",
     "for (int64_t j = k - 1; j >= 0; --j) {\n            float v = oracle_bf16_to_f32(comb[(t * k + j) * H + h]);"),
    ("e4m3_truncates", "    double q = ldexp(1.0, e - 4);          /* 4 significant bits */\n    double r = rint(a / q) * q;",
     "    double q = ldexp(1.0, e - 4);          /* 4 significant bits */\n    double r = floor(a / q) * q;"),
    ("bf16_truncates", "    double r = rint(a / q) * q;            /* rint: nearest, ties to even (default mode) */",
     "    double r = floor(a / q) * q;            /* rint: nearest, ties to even (default mode) */"),
    ("fnuz_scale_240", "float scale = amax / 448.0f;", "float scale = amax / 240.0f;"),
    ("stub_multiplier_without_one", "return (float)(E + e) / (float)E;", "return (float)(e + 1) / (float)E;"),
    ("exchange_rows_crossed", "memcpy(o->recv_rows + q * rb, o->send_rows + p * rb, (size_t)rb);",
     "memcpy(o->recv_rows + p * rb, o->send_rows + q * rb, (size_t)rb);"),
    ("weight_from_wrong_slot", "m.weight = w[t * k + j];", "m.weight = w[t * k + (k - 1 - j)];"),
    ("count_matrix_transposed", "o->C[src * P + dst] = c;", "o->C[dst * P + src] = c;"),
    ("stub_dequantises_with_block0_scale", "d = qv * scales[h / FP8_BLOCK];", "d = qv * scales[0];"),
    ("amax_always_from_block0",
     "for (int64_t h = b * FP8_BLOCK; h < (b + 1) * FP8_BLOCK; ++h) {\n            float a = fabsf",
     "for (int64_t h = 0; h < FP8_BLOCK; ++h) {\n            float a = fabsf"),
    ("stub_uses_local_expert", "oracle_stub_row(s, e, recv_rows", "oracle_stub_row(s, e % (s->E / s->P), recv_rows"),
]

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
from oracle import oracle as orc
orc.use_library({lib!r})
import test_oracle_path as tp, test_oracle_formats as tf
pins = [
    ("worked_example", lambda: tp.test_worked_top2_example_receive_layout(orc)),
    ("prefix_sum", lambda: tp.test_prefix_sum_example(orc)),
    ("transpose", lambda: tp.test_all_to_all_transpose_example(orc)),
    ("brute_positions", lambda: tp.test_positions_brute_force_random(orc, 3, 5, 6, 3)),
    ("route_ties", lambda: tp.test_route_selection_brute_force_with_ties(orc)),
    ("route_weights", lambda: tp.test_route_weights_special_cases(orc)),
    ("route_nan", lambda: tp.test_route_nan_logits_rank_last(orc)),
    ("identity", lambda: tp.test_combine_of_dispatch_is_identity_for_top1_expert0(orc)),
    ("slot_order", lambda: tp.test_reduce_slot_order_closed_form(orc)),
    ("stub_bf16", lambda: tp.test_stub_closed_form_bf16(orc)),
    ("combine_c1", lambda: tp.test_combine_closed_form(orc, "c1")),
    ("bf16_torch", lambda: tf.test_bf16_matches_torch_on_float32(orc)),
    ("e4m3_torch", lambda: tf.test_e4m3_encode_matches_torch_in_range(orc)),
    ("quantize", lambda: tf.test_quantize_row_properties(orc)),
    ("invariants_c1", lambda: tp.test_invariants_on_workloads(orc, "c1")),
    ("byte_model_c3", lambda: tp.test_byte_model_closed_form(orc)),
    ("combine_c3", lambda: tp.test_combine_closed_form(orc, "c3")),
]
for name, fn in pins:
    try:
        fn()
    except AssertionError:
        print("CAUGHT", name, flush=True)
        sys.exit(3)
print("SURVIVED", flush=True)
sys.exit(0)
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mutated = tmp_path / "moe_oracle.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-ffp-contract=off", "-shared", "-o", str(lib), str(mutated),
                    "-lm"], check=True)
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=str(lib))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "SURVIVED" not in out, f"mutant {name} survived every pin"
    assert "CAUGHT" in out or r.returncode < 0, f"mutant {name}: unexpected failure\n{out[-2000:]}"
