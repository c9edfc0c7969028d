"""Planted mistakes in copies of the oracle must each trip at least one pin.

Each mutant is a textual edit of oracle.c (a dropped term, a wrong index, a
transposed operand, a wrong sign ...), compiled into a temporary library and
checked by the fast pins in a child process.  The real oracle is untouched.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

MUTANTS = {
    "padding_rounds_down": ("(c + block_m - 1) / block_m * block_m", "c / block_m * block_m"),
    "sentinel_off_by_one": ("= (int32_t)numel;", "= (int32_t)numel - 1;"),
    "group_start_after_group": (
        "start[(int64_t)l * E + e] = offset;\n            offset += padded;",
        "offset += padded;\n            start[(int64_t)l * E + e] = offset - c;"),
    "pairs_walked_downwards": (
        "    for (int64_t p = 0; p < numel; ++p) {\n        int64_t m = p / topk;\n"
        "        int32_t l = token_lora_mapping[m];\n        int32_t e = topk_ids[p];\n"
        "        if (l < 0 || l >= L || e < 0 || e >= E)\n            continue;\n"
        "        int64_t g",
        "    for (int64_t p = numel - 1; p >= 0; --p) {\n        int64_t m = p / topk;\n"
        "        int32_t l = token_lora_mapping[m];\n        int32_t e = topk_ids[p];\n"
        "        if (l < 0 || l >= L || e < 0 || e >= E)\n            continue;\n"
        "        int64_t g"),
    "expert_ids_reversed": ("expert_ids[(int64_t)l * nb + b] = e;",
                            "expert_ids[(int64_t)l * nb + b] = E - 1 - e;"),
    "empty_slot_counted_active": ("if (num_tokens_post_padded[l] > 0)",
                                  "if (num_tokens_post_padded[l] >= 0)"),
    "lora_a_transposed": ("A[(int64_t)j * K + t]", "A[(int64_t)t * r + j]"),
    "lora_b_transposed": ("B[(int64_t)n * r + j]", "B[(int64_t)j * Ns + n]"),
    "routed_weight_dropped": ("if (mul)\n                d *= (double)topk_weights[p];",
                              "if (0)\n                d *= (double)topk_weights[p];"),
    "routed_weight_by_token": ("d *= (double)topk_weights[p];",
                               "d *= (double)topk_weights[m];"),
    "add_inputs_ignored": ("double base = add ? bf16_to_double(y_in_row[col]) : 0.0;",
                           "double base = bf16_to_double(y_in_row[col]);"),
    "x_row_always_token": ("int64_t row = x_per_pair ? p : m;", "int64_t row = m;"),
    "slice_offset_dropped": ("int64_t col = (int64_t)s * Ns + n;", "int64_t col = n;"),
    "wrong_slot_weights": ("lora_a + (((int64_t)s * L + l) * E + e)",
                           "lora_a + (((int64_t)s * L + (l + 1) % L) * E + e)"),
    "shrink_sign_flipped": ("acc += bf16_to_double(xr[t])", "acc -= bf16_to_double(xr[t])"),
    "bf16_widening_wrong": ("((uint32_t)h) << 16", "((uint32_t)h) << 15"),
    "last_rank_dropped": ("for (int32_t j = 0; j < r; ++j)\n                d +=",
                          "for (int32_t j = 0; j < r - 1; ++j)\n                d +="),
    "last_k_dropped": ("for (int32_t t = 0; t < K; ++t)", "for (int32_t t = 0; t < K - 1; ++t)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert old in src, f"mutation site for {name} no longer in oracle.c"
    mutant_src = tmp_path / "oracle_mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(src=str(mutant_src), out=str(tmp_path / "libmutant.so"),
                       extra=("-w",))
    proc = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                          capture_output=True, text=True, timeout=300)
    if proc.returncode < 0:
        return  # the mutant crashed: caught
    assert proc.returncode == 0, proc.stderr[-2000:]
    res = json.loads(proc.stdout.strip().splitlines()[-1])
    failed = [k for k, v in res.items() if v != "pass"]
    assert failed, f"mutant {name} passed every pin"
