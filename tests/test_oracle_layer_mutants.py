"""Planted mistakes in the encoder-layer oracle (on the CPU) must each fail at least one
pin of tests/test_oracle_layer.py: the tanh GELU, an unbiased or mis-placed LayerNorm
variance, a dropped residual, LN2 applied to the layer input, reversed or shifted
convolution taps and a missing positional embedding.
"""
import math

import numpy as np
import pytest

import oracle.encoder_layer as L
from tests import test_oracle_layer as P

ORIG = {name: getattr(L, name) for name in ("layer_norm", "gelu", "conv1d_k3", "encoder_stem",
                                             "encoder_layer")}


def _gelu_tanh(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))


def _ln_unbiased(x, gamma, beta, eps=L.LN_EPS):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(-1, keepdims=True)
    var = x.var(-1, ddof=1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def _ln_eps_outside(x, gamma, beta, eps=L.LN_EPS):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(-1, keepdims=True)
    return (x - mu) / (np.sqrt(((x - mu) ** 2).mean(-1, keepdims=True)) + eps) * gamma + beta


def _conv_taps_reversed(x, w, b, stride):
    return ORIG["conv1d_k3"](x, np.asarray(w)[:, :, ::-1], b, stride)


def _conv_shifted(x, w, b, stride):
    x = np.asarray(x, dtype=np.float64)
    xs = np.vstack([x[1:], np.zeros((1, x.shape[1]))])  # reads frame stride*t + tap
    return ORIG["conv1d_k3"](xs, w, b, stride)


def _stem_without_positions(mel, c1w, c1b, c2w, c2b, pos):
    return ORIG["encoder_stem"](mel, c1w, c1b, c2w, c2b, np.zeros_like(np.asarray(pos, dtype=np.float64)))


def _layer_without_mlp_residual(x, w, batch, seq_len, chunk_len, valid_len, n_heads, rows=None):
    out = ORIG["encoder_layer"](x, w, batch, seq_len, chunk_len, valid_len, n_heads, rows)
    out["y"] = out["y"] - out["x1"]
    return out


def _layer_ln2_on_input(x, w, batch, seq_len, chunk_len, valid_len, n_heads, rows=None):
    out = ORIG["encoder_layer"](x, w, batch, seq_len, chunk_len, valid_len, n_heads, rows)
    xs = np.asarray(x, dtype=np.float64)[out["rows"]]
    out["y"] = out["x1"] + L.mlp(L.layer_norm(xs, w.ln2_g, w.ln2_b), w.w_fc1, w.b_fc1, w.w_fc2, w.b_fc2)
    return out


MUTANTS = {
    "gelu_tanh": ("gelu", _gelu_tanh),
    "ln_unbiased": ("layer_norm", _ln_unbiased),
    "ln_eps_outside": ("layer_norm", _ln_eps_outside),
    "conv_taps_reversed": ("conv1d_k3", _conv_taps_reversed),
    "conv_shifted": ("conv1d_k3", _conv_shifted),
    "stem_without_positions": ("encoder_stem", _stem_without_positions),
    "no_mlp_residual": ("encoder_layer", _layer_without_mlp_residual),
    "ln2_on_input": ("encoder_layer", _layer_ln2_on_input),
}


def run_pins():
    P.test_layer_norm_against_torch()
    P.test_layer_norm_brute_force()
    P.test_layer_norm_invariants()
    P.test_gelu_exact_values()
    P.test_gelu_against_torch_and_odd_identity()
    P.test_linear_and_mlp_brute_force()
    for stride in (1, 2):
        P.test_conv_against_torch(stride, 5)
    P.test_conv_brute_force_taps()
    P.test_stem_against_torch_and_shape()
    P.test_layer_against_torch(8, 4, 7, 1)
    P.test_layer_closed_forms()


def test_unmutated_pins_pass():
    run_pins()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    target, fn = MUTANTS[name]
    monkeypatch.setattr(L, target, fn)
    with pytest.raises(AssertionError):
        run_pins()
