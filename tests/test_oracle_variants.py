"""Pins for the attention-variant oracle (sinks, block masks), independent of its own code:
float64 torch scaled_dot_product_attention with the sink as an extra zero-value key carrying an
additive logit, the no-sink limit against the pinned verification oracle, closed forms, and
planted mistakes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.variants as V

F = torch.nn.functional


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def rand(seed, n_q=5, n_kv=9, h=3, dh=8):
    r = np.random.default_rng(seed)
    return (r.standard_normal((n_q, h, dh)), r.standard_normal((n_kv, h, dh)) * 1.3, r.standard_normal((n_kv, h, dh)),
            r.standard_normal(h) * 2)


def sdpa_with_sinks(q, k, v, mask, sinks):
    """torch SDPA over the keys plus one extra key per head with q.k = 0, value 0, and an
    additive bias equal to the sink (the extra column is always admitted)."""
    n_q, h, dh = q.shape
    n_kv = k.shape[0]
    K = torch.cat([t64(k), torch.zeros(1, h, dh, dtype=torch.float64)])
    Vv = torch.cat([t64(v), torch.zeros(1, h, dh, dtype=torch.float64)])
    bias = torch.zeros(h, n_q, n_kv + 1, dtype=torch.float64)
    if mask is not None:
        bias[:, :, :n_kv] = torch.where(t64(mask).bool(), 0.0, -math.inf)[None]
    bias[:, :, n_kv] = t64(sinks)[:, None]
    o = F.scaled_dot_product_attention(t64(q).transpose(0, 1), K.transpose(0, 1), Vv.transpose(0, 1),
                                       attn_mask=bias)
    return o.transpose(0, 1).numpy()


@pytest.mark.parametrize("seed,masked", [(1, False), (2, True), (3, True)])
def test_sinks_against_torch_sdpa(seed, masked):
    q, k, v, sinks = rand(seed)
    mask = V.block_mask(5, 9, causal=True) if masked else None
    assert np.abs(V.verify_attention_sinks(q, k, v, mask, sinks) - sdpa_with_sinks(q, k, v, mask, sinks)).max() < 1e-12


def test_no_sink_limit_is_plain_verification():
    q, k, v, _ = rand(4)
    mask = np.random.default_rng(4).random((5, 9)) < 0.6
    ref = oracle.verify_attention(q, k, v, mask)
    assert np.abs(V.verify_attention_sinks(q, k, v, mask, None) - ref).max() < 1e-12
    assert np.abs(V.verify_attention_sinks(q, k, v, mask, np.full(3, -np.inf)) - ref).max() < 1e-12


def test_sink_closed_forms():
    q, k, v, _ = rand(5, n_q=1, n_kv=1, h=1)
    s = float(q[0, 0] @ k[0, 0]) / math.sqrt(8)
    for sink in (s, s + math.log(3.0), -2.0):
        got = V.verify_attention_sinks(q, k, v, None, np.array([sink]))[0, 0]
        assert np.abs(got - v[0, 0] * math.exp(s) / (math.exp(s) + math.exp(sink))).max() < 1e-12
    # A sink equal to the only score halves the output; a row with no admitted key stays 0.
    assert np.abs(V.verify_attention_sinks(q, k, v, None, np.array([s]))[0, 0] - v[0, 0] / 2).max() < 1e-12
    none = np.zeros((1, 1), dtype=bool)
    assert not V.verify_attention_sinks(q, k, v, none, np.array([1.0])).any()


def test_block_masks():
    assert V.block_mask(3, 7, causal=False).all()
    np.testing.assert_array_equal(V.block_mask(3, 7, causal=True), oracle.causal_rows(3, 7))


ORIG = V.verify_attention_sinks


def _sink_unscaled(q, k, v, mask=None, sinks=None):
    return ORIG(q, k, v, mask, None if sinks is None else np.asarray(sinks) * math.sqrt(q.shape[2]))


def _sink_with_value(q, k, v, mask=None, sinks=None):
    out = ORIG(q, k, v, mask, sinks)
    return out + 0.01 * np.asarray(v).mean(axis=0)[None]


def _sink_ignored(q, k, v, mask=None, sinks=None):
    return ORIG(q, k, v, mask, None)


@pytest.mark.parametrize("fn", [_sink_unscaled, _sink_with_value, _sink_ignored])
def test_planted_mistake_is_caught(fn, monkeypatch):
    monkeypatch.setattr(V, "verify_attention_sinks", fn)
    with pytest.raises(AssertionError):
        test_sinks_against_torch_sdpa(1, False)
        test_sink_closed_forms()
