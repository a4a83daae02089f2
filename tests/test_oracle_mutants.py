"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

This shows the pins in test_oracle.py are strong enough: a dropped term, a wrong
scale, an off-by-one mask bound, a transposed head layout, a missing
normalisation or an un-rescaled merge cannot pass them unnoticed.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as OA
from tests import test_oracle as P

ORIG = {name: getattr(OA, name) for name in (
    "qkv_projection", "key_interval", "split_heads", "softmax_probabilities", "causal_rows",
    "merge_partials", "attention_head")}


def _wrong_scale(q, k, admit, scale):
    return ORIG["softmax_probabilities"](q, k, admit, scale * scale)


def _no_normalisation(q, k, admit, scale):
    s = np.where(admit, (np.asarray(q, float) @ np.asarray(k, float).T) * scale, -np.inf)
    m = np.where(admit.any(1, keepdims=True), s.max(1, keepdims=True), 0.0)
    return np.where(admit, np.exp(s - m), 0.0)


def _keys_as_queries(q, k, admit, scale):
    qq = np.asarray(q, float)
    kk = np.resize(qq, np.shape(k))  # uses the query rows in place of keys
    return ORIG["softmax_probabilities"](q, kk, admit, scale)


def _dropped_bias(x, w_qkv, b_qkv=None):
    return ORIG["qkv_projection"](x, w_qkv, None)


def _chunk_off_by_one(i, chunk_len, valid_len):
    lo, hi = ORIG["key_interval"](i, chunk_len, valid_len)
    return lo, max(lo, hi - 1) if chunk_len else hi


def _valid_ignored(i, chunk_len, valid_len):
    return ORIG["key_interval"](i, chunk_len, 10 ** 9)


def _interleaved_heads(block, n_heads):
    rows, width = block.shape
    return block.reshape(rows, width // n_heads, n_heads).transpose(2, 0, 1)


def _causal_without_diagonal(n_q, n_kv):
    m = ORIG["causal_rows"](n_q, n_kv)
    for t in range(n_q):
        m[t, n_kv - n_q + t] = False
    return m


def _merge_without_rescale(parts):
    l = sum(p[1] for p in parts)
    o = sum(p[2] for p in parts)
    out = np.zeros_like(o)
    nz = l > 0
    out[nz] = o[nz] / l[nz][:, None]
    return out


def _head_ignores_value_bias(q, k, v, admit, scale):
    vv = np.asarray(v, float)
    return ORIG["attention_head"](q, k, vv - vv.mean(axis=0, keepdims=True), admit, scale)


MUTANTS = {
    "wrong_scale": ("softmax_probabilities", _wrong_scale),
    "no_normalisation": ("softmax_probabilities", _no_normalisation),
    "keys_as_queries": ("softmax_probabilities", _keys_as_queries),
    "dropped_bias": ("qkv_projection", _dropped_bias),
    "chunk_off_by_one": ("key_interval", _chunk_off_by_one),
    "valid_ignored": ("key_interval", _valid_ignored),
    "interleaved_heads": ("split_heads", _interleaved_heads),
    "causal_without_diagonal": ("causal_rows", _causal_without_diagonal),
    "merge_without_rescale": ("merge_partials", _merge_without_rescale),
    "value_centred": ("attention_head", _head_ignores_value_bias),
}


def run_pins():
    P.test_brute_force_encoder(6, 2, 5)
    P.test_brute_force_encoder(6, 0, 4)
    P.test_brute_force_verify(4, 7, "causal")
    P.test_causal_rows_brute()
    P.test_softmax_rows_sum_to_one_and_respect_mask()
    P.test_against_torch_sdpa_float64()
    P.test_merge_of_any_partition_equals_full_softmax([0, 13, 40])
    P.test_k_bias_invariance_and_v_bias_pass_through()


def test_unmutated_pins_pass():
    run_pins()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    target, fn = MUTANTS[name]
    monkeypatch.setattr(OA, target, fn)
    if hasattr(oracle, target):
        monkeypatch.setattr(oracle, target, fn)
    with pytest.raises(AssertionError):
        run_pins()
