"""The oracle's pins must catch plausible mistakes.

Each case copies oracle.c, plants one mistake (a wrong gather index, a
dropped term, a transposed mask bit, ...), builds the copy with gcc on the
CPU and runs the pin battery of the other oracle tests against it.  At
least one pin must fail for every mutant, and none for the unmodified
source.  Nothing here touches a GPU.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_csr as tcsr
import test_oracle_forward as tfwd
import workloads as W

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "key_gathered_at_destination": (
        "const double* kj = k + ((int64_t)col_idx[p] * h + hh) * d;",
        "const double* kj = k + ((int64_t)i * h + hh) * d;"),
    "value_gathered_at_destination": (
        "const double* vj = v + ((int64_t)col_idx[p] * h + hh) * d;",
        "const double* vj = v + ((int64_t)i * h + hh) * d;"),
    "query_head_offset_dropped": (
        "const double* qi = q + ((int64_t)i * h + hh) * d;",
        "const double* qi = q + ((int64_t)i * h) * d;"),
    "epsilon_dropped": ("if (clipped) z += eps;", "if (clipped) z += 0.0;"),
    "elementwise_clamp_dropped": (
        "double x = clampd(scale * qi[c] * kj[c], lo, hi);",
        "double x = scale * qi[c] * kj[c];"),
    "summed_logit_clamp_dropped": ("logit[t] = clampd(s, lo, hi);", "logit[t] = s;"),
    "scale_dropped": ("logit[t] = scale * s;", "logit[t] = s;"),
    "weights_not_normalised": ("double a = logit[t] / z;", "double a = logit[t];"),
    "weight_of_wrong_edge": ("double a = logit[t] / z;", "double a = logit[deg - 1 - t] / z;"),
    "edge_projection_ignored": (
        "s += qi[c] * kj[c] * (ep ? ep[c] : 1.0);", "s += qi[c] * kj[c];"),
    "edge_projection_reversed_in_row": (
        "const int64_t row = edge_ids ? (int64_t)edge_ids[p] : p;",
        "const int64_t row = edge_ids ? (int64_t)edge_ids[p] : (int64_t)(row_ptr[i + 1] - 1 - t);"),
    "edge_update_before_clamp": (
        "        if (e_out) e_out[(row * h + hh) * d + c] = x;   /* the edge update before the sum */\n",
        "        if (e_out) e_out[(row * h + hh) * d + c] = scale * qi[c] * kj[c] * (ep ? ep[c] : 1.0);\n"),
    "aggregate_weight_of_position": (
        "        const double wp = w[wrow * h + hh];", "        const double wp = w[(int64_t)p * h + hh];"),
    "aggregate_normalised_without_eps": ("o[c] /= (z + eps);", "o[c] /= z;"),
    "csr_rows_descending": (
        "return (x > y) - (x < y);\n}\nstatic int cmp_i32",
        "return (x < y) - (x > y);\n}\nstatic int cmp_i32"),
    "csr_edge_id_tiebreak_reversed": (
        "| (uint64_t)(uint32_t)e;", "| (uint64_t)(uint32_t)(0x7fffffff - e);"),
    "magnitude_without_weight": (
        "if (mg) mg[c] += a * fabs(vj[c]);", "if (mg) mg[c] += fabs(vj[c]);"),
    "magnitude_signed": ("if (mg) mg[c] += a * fabs(vj[c]);", "if (mg) mg[c] += a * vj[c];"),
    "window_padding_zero": ("t < u ? buf[t] : -1;", "t < u ? buf[t] : 0;"),
    "window_mask_transposed": (
        "tile_mask[tile * 16 + (r - r0)] |= (uint16_t)(1u << (t % 16));",
        "tile_mask[tile * 16 + (t % 16)] |= (uint16_t)(1u << (r - r0));"),
}


def battery(orc):
    """The non-randomised pins of the oracle test modules, run in order."""
    for seed in (0, 3, 5):
        for multi in (False, True):
            tcsr.test_csr_matches_lexsort(orc, seed, multi)
    for seed in (0, 2, 4):
        tcsr.test_rowwindows_roundtrip(orc, seed)
    tfwd.test_clip_order_worked_example(orc)
    tfwd.test_isolated_and_single_edge_exact(orc)
    tfwd.test_sdpa_complete_digraphs(orc)
    tfwd.test_equal_logits_give_scipy_mean(orc, 1)
    tfwd.test_clipped_closed_forms(orc)
    tfwd.test_e_out_is_the_elementwise_update(orc)
    for mode in ("standard", "clipped"):
        tfwd.test_edge_ids_indirection(orc, mode)
    for normalize in (False, True):
        tfwd.test_aggregate_matches_scipy(orc, normalize, True)
    tfwd.test_aggregate_closed_form(orc)
    for mode in ("standard", "clipped"):
        tfwd.test_magnitude_is_weighted_abs_sum(orc, mode, 0)
        tfwd.test_weights_sum(orc, mode)
        tfwd.test_invariants(orc, mode)
    for seed in range(4):
        for mode in ("standard", "clipped"):
            n = [7, 23, 40, 16][seed]
            src, dst = W.random_graph(950, seed, n, 10)
            q, k, v, e = tfwd.feats(seed, n, src.shape[0], 2, 16, True)
            q *= 3.0
            got = tfwd.run_oracle(orc, n, src, dst, q, k, v, e, mode, 0.25)
            ref = tfwd.dense_bruteforce(n, src, dst, q, k, v, e, mode, 0.25, -5.0, 5.0, 1e-6)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def build_variant(tmp_path, name, old, new):
    text = open(SRC).read()
    if old is not None:
        assert text.count(old) == 1, f"mutation site for {name} must be unique"
        text = text.replace(old, new)
    c = tmp_path / f"{name}.c"
    c.write_text(text)
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                           "-I", os.path.dirname(SRC), "-o", str(so), str(c), "-lm"])
    return str(so)


def test_unmodified_source_passes(tmp_path):
    with oracle.use_library(build_variant(tmp_path, "original", None, None)):
        battery(oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with oracle.use_library(build_variant(tmp_path, name, old, new)):
        with pytest.raises((AssertionError, oracle.OracleError)):
            battery(oracle)
