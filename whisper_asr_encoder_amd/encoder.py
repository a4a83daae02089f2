"""Device-resident encoder attention stack and verification helper.

Holds per-layer weights on the GPU in the library's layout and runs the
sublayer sequence (edda_qkv_pack -> edda_encoder_attn) on one stream. All
arithmetic runs in libedda.so; this module only allocates device buffers
(through torch) and issues the C-ABI calls.
"""
from __future__ import annotations

import numpy as np

from . import _lib


class EncoderAttention:
    """Encoder self-attention sublayers for `batch` windows of `seq_len` rows."""

    def __init__(self, layer_weights, batch: int, seq_len: int, chunk_len: int = 0, valid_len=None,
                 device="cuda"):
        import torch
        self.torch = torch
        self.batch, self.seq_len, self.chunk_len = int(batch), int(seq_len), int(chunk_len)
        self.valid_len = None if valid_len is None else np.asarray(valid_len, dtype=np.int32).reshape(-1)
        self.rows = self.batch * self.seq_len
        self.device = device
        self.w_qkv, self.b_qkv, self.w_o, self.b_o = [], [], [], []
        for w in layer_weights:
            self.w_qkv.append(self._dev(_lib.linear_layout(w.w_qkv)))
            self.b_qkv.append(None if w.b_qkv is None else self._dev(w.b_qkv))
            self.w_o.append(self._dev(_lib.linear_layout(w.w_o)))
            self.b_o.append(None if w.b_o is None else self._dev(w.b_o))
        self.qkv = torch.empty((self.rows, _lib.QKV_COLS), dtype=torch.float16, device=device)
        ws = _lib.encoder_workspace_bytes(self.batch, self.seq_len)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)

    def _dev(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.device)

    @property
    def layers(self) -> int:
        return len(self.w_qkv)

    def sublayer(self, x, layer: int, y, stream=None):
        """y[rows, 1280] = attention sublayer `layer` applied to x[rows, 1280] (device fp16)."""
        _lib.edda_qkv_pack(x, self.w_qkv[layer], self.b_qkv[layer], self.qkv, stream)
        _lib.edda_encoder_attn(self.qkv, self.batch, self.seq_len, self.chunk_len, self.valid_len,
                               self.w_o[layer], self.b_o[layer], y, self.workspace, stream)

    def all_layers(self, x, ys, stream=None):
        """Every layer reads the same x; ys[layer] receives that layer's output."""
        for layer in range(self.layers):
            self.sublayer(x, layer, ys[layer], stream)


class VerifyAttention:
    """Block-verification attention with a reusable workspace sized for n_kv <= max_kv."""

    def __init__(self, max_kv: int, device="cuda"):
        import torch
        self.torch = torch
        nbytes = max(_lib.verify_workspace_bytes(_lib.MAX_VERIFY_QUERIES, max_kv), _lib.VERIFY_COUNTER_BYTES)
        # Zero-filled once: the leading arrival counters must start at zero (calls keep them so).
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.device = device

    def mask_rows(self, mask):
        if mask is None:
            return None
        return self.torch.from_numpy(_lib.pack_mask_rows(mask).view(np.int32)).to(self.device)

    def __call__(self, q, k, v, mask_rows, o, stream=None):
        _lib.edda_verify_attn(q, k, v, mask_rows, o, self.workspace, stream)
