"""The oracle's backward against its pins, and planted mistakes in copies of
its C source that the pins must catch."""
import pytest

import oracle
import oracle_pins_backward as pins


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    pin(oracle.default())


MUTATIONS = {
    "softmax_jacobian_sign": ("double dl = p[j] * (dp[j] - pdp);", "double dl = p[j] * (dp[j] + pdp);"),
    "softmax_jacobian_no_centering": ("double dl = p[j] * (dp[j] - pdp);", "double dl = p[j] * dp[j];"),
    "query_grad_drops_scale": (
        "dq[i * d + e] += s * dl * oracle_load(k, k_dtype, j * d + e);",
        "dq[i * d + e] += dl * oracle_load(k, k_dtype, j * d + e);",
    ),
    "key_grad_uses_key": (
        "dk[j * d + e] += s * dl * oracle_load(q, q_dtype, i * d + e);",
        "dk[j * d + e] += s * dl * oracle_load(k, k_dtype, j * d + e);",
    ),
    "value_grad_unweighted": (
        "dvv[j * dv + e] += p[j] * dout[i * dv + e];",
        "dvv[j * dv + e] += dout[i * dv + e];",
    ),
    "decode_key_grad_dropped": (
        "s, dY + bh * N * D, dKbh, dqd, dz);",
        "s, dY + bh * N * D, dKbh, NULL, dz);",
    ),
    "stage2_query_grad_dropped": (
        "s, dz, dqd, dKbh, dVbh);",
        "s, dz, NULL, dKbh, dVbh);",
    ),
    "shared_seed_grad_not_summed": (
        "double *dSh = dS + (q_head_stride ? h * M * D : 0);",
        "double *dSh = dS + (q_head_stride ? h * M * D : 0);\n            if (!q_head_stride)\n                memset(dS, 0, (size_t)(M * D) * sizeof(double));",
    ),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_pins_catch_mutation(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.compile_oracle(str(mutated), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no backward pin catches the planted mistake '{name}'"
