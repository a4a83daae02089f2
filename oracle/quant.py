"""CPU oracle for 8-bit block-quantized weights (test infrastructure only, under the same
rules as attention.py: nothing in the product path imports it).

"audio.cpp PR #1223, Add Edda ASR" (PR description, results table): the decoder runs with
Q8_0 weights beside an F16 encoder. The pages name the format without defining it; the
reading (listed in the design notes) is GGML's Q8_0 block format:

* a weight row (one output feature, its input features in order) is cut into blocks of 32;
* each block stores one scale d = max|x| / 127 and 32 int8 codes q = round(x / d), rounding
  half away from zero, so that x ~ d q; an all-zero block has d = 0 and q = 0;
* d is computed in fp32 (d = amax / 127 rounded to fp32; its reciprocal 1/d rounded to
  fp32; each code from x * (1/d) rounded to fp32, then to an integer) and stored in fp16.

Because a code is an integer decided by fp32 arithmetic, the quantizer here takes those
decisions in fp32 exactly as stated (NumPy float32 operations round to nearest even), and
only the final integer rounding is done in fp64, where x * (1/d) + 1/2 is exact.
Dequantized weights are fp16(d) * q, exact in fp64. Pinned in tests/test_oracle_quant.py.
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64
from .encoder_layer import linear

QK = 32  # values per block


def quantize_q8_0(w_out_in):
    """w [N, K] (K % 32 == 0; fp16 values) -> (q int8 [N, K], d fp16 [N, K / 32])."""
    x = np.asarray(w_out_in, dtype=np.float32)
    n, k = x.shape
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(n, k // QK, QK)
    amax = np.abs(blocks).max(axis=2)                       # exact in fp32
    d = (amax / np.float32(127)).astype(np.float32)        # fp32 division
    inv = np.zeros_like(d)
    nz = d != 0
    inv[nz] = (np.float32(1) / d[nz]).astype(np.float32)   # fp32 reciprocal
    y = (blocks * inv[..., None]).astype(np.float32)       # fp32 products
    y64 = y.astype(np.float64)
    q = np.trunc(y64 + np.copysign(0.5, y64))              # half away from zero, exact in fp64
    return q.reshape(n, k).astype(np.int8), d.astype(np.float16)


def dequantize_q8_0(q, d):
    """fp64 [N, K] = fp16(d) * q, block by block."""
    q = np.asarray(q, dtype=np.float64)
    n, k = q.shape
    scale = np.repeat(np.asarray(d, dtype=np.float64), QK, axis=1)
    return q * scale.reshape(n, k)


def linear_q8(x, q, d, b=None):
    """x [rows, K] times the dequantized weight [N, K] transposed, plus b [N]: [rows, N] in fp64."""
    return linear(as_f64(x), dequantize_q8_0(q, d).T, b)


class DequantizedDecoderWeights:
    """A decoder layer's weights with every projection matrix replaced by its Q8_0
    dequantization (math layout [in, out], as the decoder oracle takes them); LayerNorm
    parameters, biases and the cross K/V projection are kept in fp16."""

    MATRICES = ("w_qkv", "w_o", "w_qc", "w_oc", "w_fc1", "w_fc2")

    def __init__(self, w, codes):
        """codes[name] = (q [out, in], d) from quantize_q8_0 of the matrix in [out, in] order."""
        for name in vars(w):
            setattr(self, name, getattr(w, name))
        for name in self.MATRICES:
            q, d = codes[name]
            setattr(self, name, dequantize_q8_0(q, d).T)


def quantize_decoder_weights(w):
    """Q8_0 codes of every projection matrix of a decoder layer (each as [out, in])."""
    return {name: quantize_q8_0(np.asarray(getattr(w, name)).T) for name in DequantizedDecoderWeights.MATRICES}
