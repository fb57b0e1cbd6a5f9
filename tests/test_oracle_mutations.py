"""Plant plausible mistakes in a copy of the oracle's C source and check that
the pins catch every one of them (the mistakes live only in temporary copies
built for this test; the oracle itself is untouched)."""
import os

import pytest

import oracle
import oracle_pins

MUTATIONS = {
    "scale_dropped": ("logit[j] = s * dot;", "logit[j] = dot;"),
    "stage2_uses_seeds": (
        "/* stage 2: the routing queries compress the same tokens */\n"
        "            rc |= oracle_sdpa(qd, ORACLE_F64, M, Kbh, dtype, Vbh, dtype, N, D, D, s, z);",
        "/* stage 2: the routing queries compress the same tokens */\n"
        "            rc |= oracle_sdpa(Sh, dtype, M, Kbh, dtype, Vbh, dtype, N, D, D, s, z);",
    ),
    "decode_keys_values_swapped": (
        "rc |= oracle_sdpa(Kbh, dtype, N, qd, ORACLE_F64, z, ORACLE_F64, M, D, D,",
        "rc |= oracle_sdpa(Kbh, dtype, N, z, ORACLE_F64, qd, ORACLE_F64, M, D, D,",
    ),
    "dot_skips_first_dim": (
        "for (int64_t e = 0; e < d; ++e)\n                dot += oracle_load(q, q_dtype, i * d + e) *\n"
        "                       oracle_load(k, k_dtype, j * d + e);\n            logit[j]",
        "for (int64_t e = 1; e < d; ++e)\n                dot += oracle_load(q, q_dtype, i * d + e) *\n"
        "                       oracle_load(k, k_dtype, j * d + e);\n            logit[j]",
    ),
    "denominator_drops_last_key": ("denom += logit[j];", "denom += (j + 1 < nk) ? logit[j] : 0.0;"),
    "no_max_subtraction": ("logit[j] = exp(logit[j] - lmax);", "logit[j] = exp(logit[j]);"),
    "value_operand_transposed": (
        "acc += logit[j] * oracle_load(v, v_dtype, j * dv + e);",
        "acc += logit[j] * oracle_load(v, v_dtype, e * nk + j);",
    ),
    "bf16_widened_wrong": ("[idx]) << 16;", "[idx]) << 15;"),
    "head_offset_ignores_head": (
        "const void *Kbh = oracle_offset(K, dtype, bh * N * D);\n            const void *Vbh = oracle_offset(V, dtype, bh * N * D);\n            /* stage 1",
        "const void *Kbh = oracle_offset(K, dtype, b * N * D);\n            const void *Vbh = oracle_offset(V, dtype, b * N * D);\n            /* stage 1",
    ),
    "per_head_seeds_ignored": (
        "const void *Sh = oracle_offset(S, dtype, h * q_head_stride);\n"
        "            const void *Kbh = oracle_offset(K, dtype, bh * N * D);\n"
        "            const void *Vbh = oracle_offset(V, dtype, bh * N * D);\n            /* stage 1",
        "const void *Sh = oracle_offset(S, dtype, 0);\n"
        "            const void *Kbh = oracle_offset(K, dtype, bh * N * D);\n"
        "            const void *Vbh = oracle_offset(V, dtype, bh * N * D);\n            /* stage 1",
    ),
    "stage3_scale_is_one": (
        "rc |= oracle_sdpa(Kbh, dtype, N, qd, ORACLE_F64, z, ORACLE_F64, M, D, D,\n"
        "                              s, Y",
        "rc |= oracle_sdpa(Kbh, dtype, N, qd, ORACLE_F64, z, ORACLE_F64, M, D, D,\n"
        "                              1.0, Y",
    ),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.compile_oracle(str(mutated), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"
