"""The spike inputs of the fp16-overflow parity tests reach the path they are
meant to test (a model of the encode's tile rule on the CPU)."""
import pytest

from spike_inputs import overflowing_tiles, spike_problem


@pytest.mark.parametrize("N,chunk", [(4096, 128), (4096, 4096), (16384, 128), (16384, 16384)])
def test_spikes_overflow_an_unchecked_tile(N, chunk):
    spikes = [(300, 0), (2000, 5)] + ([(9000, 9)] if N > 9000 else [])
    p = spike_problem(N, spikes)
    over = overflowing_tiles(p, chunk)
    assert len(over) == len(spikes), over
    assert all(d > 17 for _, d in over)


def test_no_spikes_no_overflow():
    assert overflowing_tiles(spike_problem(4096, []), 4096) == []
