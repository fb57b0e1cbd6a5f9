"""The spectral oracle against its pins, and planted mistakes in copies of its
source that the pins must catch."""
import importlib.util
import os

import pytest

import oracle
from oracle import spectral
import oracle_pins_spectral as pins


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_spectral_pin(pin):
    pin(spectral, oracle.default())


MUTATIONS = {
    "scale_dropped": ('L = s * np.einsum("bhmd,bhnd->bhmn", Qd, Kw)', 'L = np.einsum("bhmd,bhnd->bhmn", Qd, Kw)'),
    "decode_softmax_over_tokens": ("W_dec[b, h] = _softmax_rows(L[b, h].T)", "W_dec[b, h] = _softmax_rows(L[b, h]).T"),
    "encode_weights_unnormalised": ("W_enc[b, h] = _softmax_rows(L[b, h])", "W_enc[b, h] = np.exp(L[b, h])"),
    "product_order_swapped_and_truncated": (
        "ev = np.linalg.eigvals(W_enc[b, h] @ W_dec[b, h])",
        "ev = np.linalg.eigvals((W_dec[b, h] @ W_enc[b, h])[:M, :M])",
    ),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_spectral_pins_catch_mutation(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(spectral.__file__).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "spectral_mutant.py"
    path.write_text(src.replace(old, new).replace("from . import route as _route", "from oracle import route as _route"))
    spec = importlib.util.spec_from_file_location("spectral_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for pin in pins.PINS:
        try:
            pin(mod, oracle.default())
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no spectral pin catches the planted mistake '{name}'"
