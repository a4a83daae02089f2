"""fp64 CPU oracle for the drafter's attention variants (test infrastructure only, under the
same rules as attention.py).

llama.cpp DSpark diff ("model: add DSpark support for Nemotron3.5"):
* common/speculative.cpp hunks: block-internal drafter attention is non-causal unless the model
  sets the causal flag ("dflash.attention.causal"). Within a verification block of n_q tokens
  in the last n_q cache slots, the non-causal block admits every slot 0..n_kv-1 for each
  token; the causal block admits slots 0..n_kv-n_q+t for token t.
* src/models/dflash.cpp hunks: optional per-head attention sinks (one value per head) are
  passed into the attention call. Reading (listed in the design notes): a sink is one extra
  logit per head, in the units of the scaled scores, that joins the softmax denominator with a
  zero value vector:  O = sum_j e^(s_j - m) v_j / (e^(sink - m) + sum_j e^(s_j - m)),
  m = max(sink, max_j s_j).  A sink of -inf is no sink.

Pinned in tests/test_oracle_variants.py.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import as_f64, causal_rows


def block_mask(n_q: int, n_kv: int, causal: bool) -> np.ndarray:
    """Mask rows of a block in the last n_q of n_kv slots: causal, or every slot (non-causal)."""
    if causal:
        return causal_rows(n_q, n_kv)
    return np.ones((n_q, n_kv), dtype=bool)


def verify_attention_sinks(q, k, v, mask=None, sinks=None) -> np.ndarray:
    """O [n_q, H, dh] for q [n_q, H, dh], k/v [n_kv, H, dh], mask bool [n_q, n_kv] or None,
    sinks [H] (logits in scaled-score units) or None; scale 1/sqrt(dh)."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    n_q, n_heads, dh = q.shape
    admit = np.ones((n_q, k.shape[0]), dtype=bool) if mask is None else np.asarray(mask, dtype=bool)
    out = np.zeros((n_q, n_heads, dh))
    for h in range(n_heads):
        sink = -math.inf if sinks is None else float(sinks[h])
        s = (q[:, h, :] @ k[:, h, :].T) / math.sqrt(dh)
        for i in range(n_q):
            cols = np.nonzero(admit[i])[0]
            m = max([sink] + [s[i, j] for j in cols])
            if m == -math.inf:
                continue  # nothing admitted and no sink: O = 0
            e = np.exp(s[i, cols] - m)
            denom = e.sum() + (math.exp(sink - m) if sink > -math.inf else 0.0)
            out[i, h, :] = (e @ v[cols, h, :]) / denom
    return out
