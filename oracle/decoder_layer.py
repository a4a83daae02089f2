"""fp64 CPU oracle for the decoder's verification layer (test infrastructure only, under the
same rules as attention.py).

"audio.cpp PR #1223, Add Edda ASR" (PR description and commit messages): the target decoder
verifies an anchor plus up to 15 drafted tokens in one pass, with KV slots indexed by position;
beam search shares one token-tree KV cache whose mask row for a beam admits only its
ancestors; the decoder also attends to the encoder output (cross-attention). The pages do
not spell out the decoder layer; it follows the public Whisper-large-v3 decoder (a reading,
listed in the design notes): pre-norm residual sublayers

    x1 = x  + SelfAttn(LN1(x))     (the block's K/V rows are written into the cache first)
    x2 = x1 + CrossAttn(LN2(x1))   (K/V of the encoder output, projected once per utterance)
    y  = x2 + MLP(LN3(x2))

with the same LayerNorm, GELU MLP and 1/sqrt(64) score scale as the encoder. Weights are in
the math layout (y = x w): w [in, out]. Pinned in tests/test_oracle_decoder.py.
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64, verify_attention
from .encoder_layer import layer_norm, linear, mlp

N_HEADS, HEAD_DIM = 20, 64


def heads(a, n_heads: int = N_HEADS) -> np.ndarray:
    """[rows, n_heads * dh] -> [rows, n_heads, dh]."""
    a = as_f64(a)
    return a.reshape(a.shape[0], n_heads, -1)


def append_kv(k_cache, v_cache, slots, k_new, v_new):
    """Copies of the caches [slots_total, H, dh] with row slots[t] replaced by k_new[t], v_new[t]."""
    k, v = as_f64(k_cache).copy(), as_f64(v_cache).copy()
    for t, s in enumerate(slots):
        k[s] = as_f64(k_new)[t]
        v[s] = as_f64(v_new)[t]
    return k, v


def cross_kv(enc, w_k, w_v, b_v=None, n_heads: int = N_HEADS):
    """Cross-attention K and V of the encoder output enc [frames, d]: enc W_k (no bias) and
    enc W_v + b_v, each [frames, H, dh]."""
    return heads(linear(enc, w_k), n_heads), heads(linear(enc, w_v, b_v), n_heads)


def decoder_verify_layer(x, w, slots, k_cache, v_cache, n_kv: int, mask, cross_k, cross_v,
                         n_heads: int = N_HEADS) -> dict:
    """One decoder layer for the n_q block tokens x [n_q, d].

    w: object with ln1_g, ln1_b, w_qkv [d, 3d], b_qkv, w_o, b_o (self-attention), ln2_g, ln2_b,
    w_qc [d, d], b_qc, w_oc, b_oc (cross-attention), ln3_g, ln3_b, w_fc1, b_fc1, w_fc2, b_fc2.
    slots [n_q]: cache slot of each block token; the self-attention reads slots 0..n_kv-1 of
    the caches after the append, under mask [n_q, n_kv] (None = every slot).
    Returns {"k_cache", "v_cache" (after the append), "x1", "x2", "y"}.
    """
    x = as_f64(x)
    d = x.shape[1]
    h = layer_norm(x, w.ln1_g, w.ln1_b)
    qkv = linear(h, w.w_qkv, w.b_qkv)
    q, k_new, v_new = (heads(qkv[:, :d], n_heads), heads(qkv[:, d:2 * d], n_heads),
                       heads(qkv[:, 2 * d:], n_heads))
    kc, vc = append_kv(k_cache, v_cache, slots, k_new, v_new)
    o = verify_attention(q, kc[:n_kv], vc[:n_kv], mask).reshape(x.shape[0], d)
    x1 = x + linear(o, w.w_o, w.b_o)
    qc = heads(linear(layer_norm(x1, w.ln2_g, w.ln2_b), w.w_qc, w.b_qc), n_heads)
    oc = verify_attention(qc, cross_k, cross_v, None).reshape(x.shape[0], d)
    x2 = x1 + linear(oc, w.w_oc, w.b_oc)
    y = x2 + mlp(layer_norm(x2, w.ln3_g, w.ln3_b), w.w_fc1, w.b_fc1, w.w_fc2, w.b_fc2)
    return {"k_cache": kc, "v_cache": vc, "x1": x1, "x2": x2, "y": y}
