"""Plants one mistake at a time in a copy of the oracle's index projection
(on the CPU) and checks that its pin catches each: the key head taken first,
the heads shifted by one, truncation instead of rounding to nearest even, and
the weight used untransposed."""
import numpy as np
import pytest

import oracle
import oracle_pins as pins


def _mutant(kind):
    def project(hidden, w, groups, index_dim=128):
        h64 = oracle._bf16_bits_to_f64(hidden)
        w64 = oracle._bf16_bits_to_f64(w)
        G, dI = groups, index_dim
        if kind == "untransposed":
            c = h64 @ w64.reshape(h64.shape[-1], -1)
        else:
            c = h64 @ w64.T
        if kind == "key_head_first":
            c = np.concatenate([c[:, G * dI:], c[:, :G * dI]], axis=1)
        if kind == "heads_shifted":
            c = np.roll(c, -dI, axis=1)
        q = c[:, :G * dI].reshape(-1, G, dI)
        k = c[:, G * dI:]
        if kind == "truncation":
            to_bits = lambda x: (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
        else:
            to_bits = oracle._f64_to_bf16_bits
        return q, k, to_bits(q), to_bits(k)
    return project


@pytest.mark.parametrize("kind", ["key_head_first", "heads_shifted", "truncation",
                                  "untransposed"])
def test_project_mutant_is_caught(monkeypatch, kind):
    monkeypatch.setattr(oracle, "index_project", _mutant(kind))
    with pytest.raises(Exception):
        pins.pin_index_project(None)


def test_project_pin_passes_on_the_oracle():
    pins.pin_index_project(None)
