"""fp64 CPU oracle for the rest of a Whisper-large-v3 encoder around the attention path.

TEST INFRASTRUCTURE ONLY, under the same rules as attention.py: only the tests, the
smoke check and the benchmark's CPU-baseline leg use it; it shares no code with the HIP
library and computes the plain definitions in float64 with no rounding of intermediates.

The pages place the attention sublayer inside a Whisper-large-v3 encoder ("audio.cpp
PR #1223, Add Edda ASR": the encoder commit message times a whole 30 s window, and the
PR description names the model), and "BuzzASR/danish discussion #1" counts its 32
layers. They do not spell out the rest of the layer. It is taken here from the public
Whisper-large-v3 architecture (a reading, listed in the design notes):

* pre-norm residual layer:  x1 = x + Attn(LN1(x));  y = x1 + MLP(LN2(x1)),
  MLP(h) = GELU(h W1 + b1) W2 + b2 with a 4x (5120-wide) hidden layer;
* LayerNorm over the 1280 features with a learned scale and shift, eps = 1e-5;
* GELU in its exact form x * Phi(x), Phi the standard normal CDF (via erf);
* the convolutional stem: conv1 (128 mel bins -> 1280, kernel 3, padding 1), GELU,
  conv2 (1280 -> 1280, kernel 3, stride 2, padding 1), GELU, plus a [1500, 1280]
  positional embedding; a final LayerNorm after the last layer.

Weights are in the math layout (y = x W): w [in, out]. The convolution weight is
[out, in, 3] (output channel, input channel, tap) and reads input frame
stride * t + tap - 1 (zero outside the input).

Parity pins: tests/test_oracle_layer.py (library routines in float64, closed forms,
invariants, brute force on tiny shapes).
"""
from __future__ import annotations

import math

import numpy as np

from .attention import as_f64, encoder_attention

LN_EPS = 1e-5


def layer_norm(x, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """Per row: (x - mean) / sqrt(var + eps) * gamma + beta, var the biased variance."""
    x = as_f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * as_f64(gamma) + as_f64(beta)


def gelu(x) -> np.ndarray:
    """x * Phi(x) with Phi(x) = (1 + erf(x / sqrt 2)) / 2."""
    x = as_f64(x)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return x * 0.5 * (1.0 + erf(x / math.sqrt(2.0)))


def linear(x, w, b=None) -> np.ndarray:
    """x [rows, in] times w [in, out] plus b [out]."""
    y = as_f64(x) @ as_f64(w)
    if b is not None:
        y = y + as_f64(b)[None, :]
    return y


def mlp(h, w1, b1, w2, b2) -> np.ndarray:
    return linear(gelu(linear(h, w1, b1)), w2, b2)


def conv1d_k3(x, w, b, stride: int) -> np.ndarray:
    """x [T_in, C_in] (time-major), w [C_out, C_in, 3], b [C_out]; padding 1.
    Output frame t reads input frames stride*t - 1, stride*t, stride*t + 1."""
    x, w = as_f64(x), as_f64(w)
    t_in = x.shape[0]
    t_out = (t_in + 2 - 3) // stride + 1
    xp = np.zeros((t_in + 2, x.shape[1]))
    xp[1:t_in + 1] = x
    y = np.zeros((t_out, w.shape[0]))
    for tap in range(3):
        frames = xp[stride * np.arange(t_out) + tap]     # padded index = input index + 1
        y += frames @ w[:, :, tap].T
    return y + as_f64(b)[None, :]


def encoder_stem(mel, conv1_w, conv1_b, conv2_w, conv2_b, pos_emb) -> np.ndarray:
    """mel [n_mels, n_frames] (channel-major, as a log-mel spectrogram is stored) ->
    [n_frames // 2, d] = GELU(conv2(GELU(conv1(mel)))) + pos_emb."""
    x = as_f64(mel).T
    h = gelu(conv1d_k3(x, conv1_w, conv1_b, stride=1))
    h = gelu(conv1d_k3(h, conv2_w, conv2_b, stride=2))
    return h + as_f64(pos_emb)[: h.shape[0]]


def encoder_layer(x, w, batch: int, seq_len: int, chunk_len: int, valid_len, n_heads: int,
                  rows=None) -> dict:
    """One pre-norm encoder layer over `batch` windows of `seq_len` rows.

    w: object with ln1_g, ln1_b, w_qkv [d, 3d], b_qkv, w_o [d, d], b_o, ln2_g, ln2_b,
    w_fc1 [d, 4d], b_fc1, w_fc2 [4d, d], b_fc2. `rows`: optional sorted global row
    indices to return (the attention still sees every key of their windows).
    Returns {"x1": [rows_sel, d], "y": [rows_sel, d], "rows": rows}.
    """
    x = as_f64(x)
    h = layer_norm(x, w.ln1_g, w.ln1_b)
    att = encoder_attention(h, w.w_qkv, w.b_qkv, w.w_o, w.b_o, batch, seq_len, chunk_len, valid_len,
                            n_heads, rows=rows)
    sel = att["rows"]
    x1 = x[sel] + att["y"]
    y = x1 + mlp(layer_norm(x1, w.ln2_g, w.ln2_b), w.w_fc1, w.b_fc1, w.w_fc2, w.b_fc2)
    return {"x1": x1, "y": y, "rows": sel}
