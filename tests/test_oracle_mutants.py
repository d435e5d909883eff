"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a textual change to a copy of oracle/oracle.c (a flipped tie
rule, a transposed compare, a dropped bound, a wrong index), compiled with gcc
into a temporary library.  The pins then run against it in a child process, so
a mutant that reads out of bounds and crashes also counts as caught.  The real
oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

MUTANTS = {
    "ties_b_first": ("A[i] <= B[j]", "A[i] < B[j]"),
    "compare_transposed": ("A[i] <= B[j]", "B[j] <= A[i]"),
    "b_exhaustion_dropped": ("    if (j >= n)\n        return 1;\n", ""),
    "a_exhaustion_dropped": ("if (i < m && A[i] <= B[j])", "if (A[i] <= B[j])"),
    "key_index_off_by_one": ("C[k] = A[i];", "C[k] = A[i > 0 ? i - 1 : 0];"),
    "payload_index_off_by_one": ("Cv[k] = Av[i];", "Cv[k] = Av[i > 0 ? i - 1 : 0];"),
    "payload_from_key": ("Cv[k] = Av[i];", "Cv[k] = (uint32_t)Ak[i];"),
    "co_rank_shifted": ("I[k + 1] = i;", "I[k] = i;"),
    "co_rank_counts_b": ("            ++i;\n        else\n            ++j;\n        I[k + 1] = i;",
                         "            ++j;\n        else\n            ++i;\n        I[k + 1] = i;"),
    "co_rank_start_one": ("I[0] = 0;", "I[0] = 1;"),
    "zeros_equal": ("return x_neg >= y_neg;", "return 1;"),
    "zeros_reversed": ("return x_neg >= y_neg;", "return x_neg <= y_neg;"),
    "nan_sign_ignored": ("        return x_neg;             /* -NaN before anything",
                         "        return 0;             /* -NaN before anything"),
    "nan_pair_sign_ignored": ("            return x_neg;         /* -NaN before +NaN */",
                              "            return y_neg;         /* -NaN before +NaN */"),
    "neg_nan_payload_ascending": ("x_neg ? x_frac >= y_frac", "x_neg ? x_frac <= y_frac"),
    "nan_payload_ignored": ("return x_neg ? x_frac >= y_frac : x_frac <= y_frac;",
                            "return x_frac + y_frac + 1u > 0u;"),
    "float_as_signed_int": ("        return total_order_f32((uint32_t)x, (uint32_t)y);",
                            "        return total_order_f32((uint32_t)x, (uint32_t)x) && "
                            "(int32_t)(uint32_t)x <= (int32_t)(uint32_t)y;"),
    "u32_as_signed": ("        return x <= y;", "        return (int32_t)x <= (int32_t)y;"),
    "descending_ties_b_first": ("return le_ascending(kind, y, x);",
                                "return !le_ascending(kind, x, y);"),
    "descending_not_reversed": ("return le_ascending(kind, y, x);",
                                "return le_ascending(kind, x, y);"),
    "i64_as_unsigned": ("        return (int64_t)x <= (int64_t)y;", "        return x <= y;"),
    "u64_low_word_only": ("    case KIND_U64:\n        return x <= y;",
                          "    case KIND_U64:\n        return (uint32_t)x <= (uint32_t)y;"),
    "f64_zeros_equal": ("        if (x == 0.0)\n            return x_neg >= y_neg;",
                        "        if (x == 0.0)\n            return x_neg >= 0;"),
    "f64_nan_payload_reversed": ("        return x_neg ? x_frac >= y_frac : x_frac <= y_frac;\n    }\n    if (x_nan)\n        return x_neg;\n    return !y_neg;\n}\n\n/* Ascending",
                                 "        return x_neg ? x_frac <= y_frac : x_frac <= y_frac;\n    }\n    if (x_nan)\n        return x_neg;\n    return !y_neg;\n}\n\n/* Ascending"),
    "f64_as_f32": ("        return total_order_f64(x, y);",
                   "        return total_order_f64(x, x) && total_order_f32((uint32_t)(x >> 32), (uint32_t)(y >> 32));"),
    "key_size_64_for_f64_only": ("return kind >= KIND_I64 ? 8 : 4;", "return kind >= KIND_F64 ? 8 : 4;"),
    "payload_half_copied": ("memcpy(cv + vs * k, av + vs * i, vs);", "memcpy(cv + vs * k, av + vs * i, 4);"),
    "sort_right_run_first": ("            merge_range(order, vs, src_k + ks * i, vs ? src_v + vs * i : 0,\n                        la, src_k + ks * (i + la),\n                        vs ? src_v + vs * (i + la) : 0, lb, dst_k + ks * i,",
                             "            merge_range(order, vs, src_k + ks * (i + la),\n                        vs ? src_v + vs * (i + la) : 0, lb, src_k + ks * i,\n                        vs ? src_v + vs * i : 0, la, dst_k + ks * i,"),
    "sort_last_pass_dropped": ("for (width = 1; width < n; width *= 2)",
                               "for (width = 1; 2 * width < n; width *= 2)"),
    "batched_output_at_a_offset": ("int64_t c0 = a0 + b0;", "int64_t c0 = a0 + (b0 > 0 ? b0 - 1 : 0);"),
    "typed_b_exhaustion_dropped": ("    if (j >= n)\n        return 1;\n    if (i < m && oracle_key_le",
                                   "    if (i < m && oracle_key_le"),
    "typed_payload_from_b": ("memcpy(cv + vs * k, av + vs * i, vs);",
                             "memcpy(cv + vs * k, (n ? bv : av) + vs * (j < n ? j : 0), vs);"),
    "runs_ties_to_later_run": ("if (best < 0 || !oracle_key_le(order, key_at(k8, ks, pos[best]),\n                                               key_at(k8, ks, pos[r])))",
                               "if (best < 0 || oracle_key_le(order, key_at(k8, ks, pos[r]),\n                                              key_at(k8, ks, pos[best])))"),
    "runs_last_way_dropped": ("        for (r = 0; r < ways; ++r) {\n                if (pos[r] >= end[r])",
                              "        for (r = 0; r + 1 < ways; ++r) {\n                if (pos[r] >= end[r])"),
    "runs_group_stride_one_run": ("for (g0 = 0; g0 < n; g0 += run * ways)",
                                  "for (g0 = 0; g0 < n; g0 += run * (ways > 1 ? ways - 1 : 1))"),
    "runs_payload_from_next": ("memcpy(ov + vs * out, v8 + vs * pos[best], vs);",
                               "memcpy(ov + vs * out, v8 + vs * (pos[best] + 1 < n ? pos[best] + 1 : pos[best]), vs);"),
    "runs_order_ignored": ("!oracle_key_le(order, key_at(k8, ks, pos[best]),",
                           "!oracle_key_le(order & 7, key_at(k8, ks, pos[best]),"),
}

RUNNER = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
failed = oracle_pins.run_all(oracle.Oracle({lib!r}))
print("FAILED_PINS", failed)
sys.exit(1 if failed else 0)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, "mutation site missing: %r" % old
    mutated = src.replace(old, new)
    assert mutated != src
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    lib = str(tmp_path / "libmutant.so")
    oracle.compile_c(str(c), lib)
    code = RUNNER.format(root=os.path.dirname(HERE), tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode != 0, "mutant %s passed every pin:\n%s" % (name, r.stdout)


def test_unmutated_copy_passes(tmp_path):
    """Control: the same harness on an unchanged copy passes every pin."""
    lib = str(tmp_path / "libcopy.so")
    oracle.compile_c(oracle.SRC, lib)
    code = RUNNER.format(root=os.path.dirname(HERE), tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
