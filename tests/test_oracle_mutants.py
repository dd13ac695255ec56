"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of ``oracle/moe_oracle.c`` (on
the CPU, in a temporary directory), builds it, and runs the pin tests against
that copy; the pins must fail.  The unmodified source must pass the same run.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "offset_drops_running_sum": (
        "expert_first_token_offset[e + 1] = expert_first_token_offset[e] + counts[e];",
        "expert_first_token_offset[e + 1] = counts[e];"),
    "order_not_stable": (
        "for (int64_t r = 0; r < num_rows; ++r) {\n        int32_t id = topk_ids[r];",
        "for (int64_t r = num_rows - 1; r >= 0; --r) {\n        int32_t id = topk_ids[r];"),
    "perm_and_inv_swapped": (
        "permuted_idx[j] = (int32_t)r;\n        inv_permuted_idx[r] = (int32_t)j;",
        "permuted_idx[r] = (int32_t)j;\n        inv_permuted_idx[j] = (int32_t)r;"),
    "gather_wrong_source_token": (
        "int64_t t = permuted_idx[j] / topk;",
        "int64_t t = j / topk;"),
    "scale_not_permuted": (
        "permuted_scale[j] = token_scale[t];",
        "permuted_scale[j] = token_scale[j / topk];"),
    "weight_index_transposed": (
        "acc += (double)topk_weights[r] * (double)expanded_output[j * hidden_size + h];",
        "acc += (double)topk_weights[k * num_tokens + t] * (double)expanded_output[j * hidden_size + h];"),
    "unpermute_ignores_inverse": (
        "int64_t j = inv_permuted_idx[r];\n                if (j < 0)\n                    continue;\n"
        "                acc += (double)topk_weights[r] *\n",
        "int64_t j = r;\n                if (j < 0)\n                    continue;\n"
        "                acc += (double)topk_weights[r] *\n"),
    "unpermute_drops_last_slot": (
        "for (int32_t k = 0; k < topk; ++k) {\n                int64_t r = t * topk + k;\n"
        "                int64_t j = inv_permuted_idx[r];\n                if (j < 0)\n                    continue;\n"
        "                acc += (double)topk_weights[r] * (double)",
        "for (int32_t k = 0; k < topk - 1; ++k) {\n                int64_t r = t * topk + k;\n"
        "                int64_t j = inv_permuted_idx[r];\n                if (j < 0)\n                    continue;\n"
        "                acc += (double)topk_weights[r] * (double)"),
    # fp8 E4M3FN and the quantiser
    "e4m3_ties_away": (
        "double v = nearbyint(a / quantum) * quantum;",
        "double v = round(a / quantum) * quantum;"),
    "e4m3_no_saturation": (
        "if (a > 448.0)\n        a = 448.0;",
        "if (a > 1e30)\n        a = 448.0;"),
    "e4m3_wrong_bias": (
        "mag = ldexp(8.0 + (double)frac, expo - 7 - 3);",
        "mag = ldexp(8.0 + (double)frac, expo - 8 - 3);"),
    "quant_wrong_fp8_max": (
        "amax > 0.0f ? amax / 448.0f : 1.0f;",
        "amax > 0.0f ? amax / 240.0f : 1.0f;"),
    "quant_amax_over_whole_row": (
        "for (int64_t i = g * group; i < (g + 1) * group; ++i) {\n                float v = x_is_bf16",
        "for (int64_t i = 0; i < h; ++i) {\n                float v = x_is_bf16"),
    "quant_multiplies_by_scale": (
        "float q = v / scale;",
        "float q = v * scale;"),
    # grouped GEMM
    "gemm_next_expert_weight": (
        "const uint16_t *we = w + (int64_t)e * n_out * k_in;",
        "const uint16_t *we = w + (int64_t)((e + 1) % num_experts) * n_out * k_in;"),
    "gemm_weight_transposed": (
        "* oracle_bf16_to_double(we[n * k_in + k]);",
        "* oracle_bf16_to_double(we[k * n_out + n]);"),
    "gemm_drops_last_k": (
        "for (int64_t k = 0; k < k_in; ++k)\n                    acc +=",
        "for (int64_t k = 0; k < k_in - 1; ++k)\n                    acc +="),
    # int64 ids
    "int64_ids_truncated": (
        "if (ids64[i] < 0 || ids64[i] >= (int64_t)num_experts)",
        "if ((int32_t)ids64[i] < 0 || (int32_t)ids64[i] >= num_experts)"),
    # local-expert filter
    "local_remote_rows_get_slot_zero": (
        "inv_permuted_idx[r] = -1;\n                continue;",
        "inv_permuted_idx[r] = 0;\n                continue;"),
    "local_map_assumed_prefix": (
        "int32_t l = expert_map[id];",
        "int32_t l = id < num_local_experts ? id : -1;"),
    "local_order_not_stable": (
        "for (int64_t r = 0; r < num_rows; ++r) {\n            if (local[r] < 0) {",
        "for (int64_t r = num_rows - 1; r >= 0; --r) {\n            if (local[r] < 0) {"),
    "local_gathers_with_expert_id": (
        "expert_first_token_offset[num_local_experts], topk,",
        "expert_first_token_offset[num_local_experts], 1,"),
    "unpermute_minus_one_wraps_to_last_row": (
        "if (j < 0)\n                    continue;",
        "if (j < 0)\n                    j = num_rows - 1;"),
    "unpermute_wrong_sign": (
        "acc += (double)topk_weights[r] *\n                       oracle_bf16_to_double",
        "acc -= (double)topk_weights[r] *\n                       oracle_bf16_to_double"),
    "bf16_truncates": (
        "double q = nearbyint(a / quantum);",
        "double q = floor(a / quantum);"),
    "bf16_rounds_ties_away": (
        "double q = nearbyint(a / quantum);",
        "double q = round(a / quantum);"),
    "bf16_wrong_bias": (
        "mag = ldexp(128.0 + (double)frac, expo - 127 - 7);",
        "mag = ldexp(128.0 + (double)frac, expo - 126 - 7);"),
}


def _run_pins(lib_path):
    env = dict(os.environ, MOE_ORACLE_LIB=lib_path, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def _build(tmp_path, name, source):
    c = tmp_path / (name + ".c")
    c.write_text(source)
    so = tmp_path / ("lib" + name + ".so")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    return str(so)


def test_unmodified_oracle_passes_pins(tmp_path):
    res = _run_pins(_build(tmp_path, "clean", open(SRC).read()))
    assert res.returncode == 0, res.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    before, after = MUTANTS[name]
    source = open(SRC).read()
    assert source.count(before) >= 1, "mutation anchor not found: " + name
    res = _run_pins(_build(tmp_path, name, source.replace(before, after, 1)))
    assert res.returncode != 0, "pins did not notice mutant " + name
