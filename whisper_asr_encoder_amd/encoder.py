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


class FullEncoder:
    """Whole encoder: convolutional stem, pre-norm layers and the final LayerNorm, for
    `batch` windows of `seq_len` positions (2 * seq_len mel frames each). Weights are held on
    the device in the library's layout; every step runs in libedda.so."""

    def __init__(self, layer_weights, stem=None, batch: int = 1, seq_len: int = 1500, chunk_len: int = 0,
                 valid_len=None, n_mels: int = 128, device="cuda"):
        import torch
        self.torch = torch
        self.batch, self.seq_len, self.chunk_len = int(batch), int(seq_len), int(chunk_len)
        self.valid_len = None if valid_len is None else [int(v) for v in np.asarray(valid_len).reshape(-1)]
        self.rows = self.batch * self.seq_len
        self.device = device
        self._keep = []          # device tensors the pointer structs refer to
        self.structs = []
        for w in layer_weights:
            t = dict(ln1_gamma=self._dev(w.ln1_g), ln1_beta=self._dev(w.ln1_b),
                     w_qkv=self._dev(_lib.linear_layout(w.w_qkv)), b_qkv=self._dev(w.b_qkv),
                     w_o=self._dev(_lib.linear_layout(w.w_o)), b_o=self._opt(w.b_o),
                     ln2_gamma=self._dev(w.ln2_g), ln2_beta=self._dev(w.ln2_b),
                     w_fc1=self._dev(_lib.linear_layout(w.w_fc1)), b_fc1=self._opt(w.b_fc1),
                     w_fc2=self._dev(_lib.linear_layout(w.w_fc2)), b_fc2=self._opt(w.b_fc2))
            self._keep.append(t)
            self.structs.append(_lib.LayerWeights(**{k: (None if v is None else v.data_ptr()) for k, v in t.items()}))
        self.stem_w = None
        if stem is not None:
            self.n_mels = int(n_mels)
            self.stem_w = dict(c1w=self._dev(_lib.conv_layout(stem.conv1_w)), c1b=self._dev(stem.conv1_b),
                               c2w=self._dev(_lib.conv_layout(stem.conv2_w)), c2b=self._dev(stem.conv2_b),
                               pos=self._dev(stem.pos_emb[:self.seq_len]), lnp_g=self._dev(stem.lnp_g),
                               lnp_b=self._dev(stem.lnp_b))
            sb = _lib.encoder_stem_workspace_bytes(self.batch, self.n_mels, 2 * self.seq_len)
            self.stem_ws = torch.empty(max(sb, 16), dtype=torch.uint8, device=device)
        lb = _lib.encoder_layer_workspace_bytes(self.batch, self.seq_len)
        self.workspace = torch.empty(max(lb, 16), dtype=torch.uint8, device=device)
        self.x = torch.empty((self.rows, _lib.D_MODEL), dtype=torch.float16, device=device)

    def _dev(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.device)

    def _opt(self, a):
        return None if a is None else self._dev(a)

    @property
    def layers(self) -> int:
        return len(self.structs)

    def layer(self, x, layer: int, y, stream=None):
        """y = encoder layer `layer` applied to x (device fp16 [rows, 1280]); y may be x."""
        _lib.edda_encoder_layer(x, self.batch, self.seq_len, self.chunk_len, self.valid_len, self.structs[layer], y,
                                self.workspace, stream)

    def stem(self, mel, y, stream=None):
        s = self.stem_w
        _lib.edda_encoder_stem(mel, s["c1w"], s["c1b"], s["c2w"], s["c2b"], s["pos"], y, self.stem_ws, stream)

    def forward(self, mel, out, stream=None):
        """out[rows, 1280] = LN_post(layers(stem(mel))); mel [batch, n_mels, 2*seq_len] device fp16."""
        self.stem(mel, self.x, stream)
        for layer in range(self.layers):
            self.layer(self.x, layer, self.x, stream)
        _lib.edda_layer_norm(self.x, self.stem_w["lnp_g"], self.stem_w["lnp_b"], out, stream)


class DecoderVerifier:
    """Decoder verification layers with device-resident weights, per-layer cross K/V of one
    encoder output and a shared workspace (zero-filled once: its leading arrival counters
    must start at zero). Every step runs in libedda.so."""

    MATRICES = ("w_qkv", "w_o", "w_q_cross", "w_o_cross", "w_fc1", "w_fc2")

    def __init__(self, layer_weights, max_kv: int, n_frames: int = 1500, device="cuda", q8: bool = False):
        """q8: the six projection matrices of every layer are quantized to Q8_0 on the device
        (edda_quantize_q8_0) and the layers run edda_decoder_verify_layer_q8."""
        import torch
        self.torch = torch
        self.device = device
        self.q8 = bool(q8)
        self.n_frames = int(n_frames)
        self._keep, self.structs, self.codes = [], [], []
        for w in layer_weights:
            t = dict(ln1_gamma=self._dev(w.ln1_g), ln1_beta=self._dev(w.ln1_b),
                     w_qkv=self._dev(_lib.linear_layout(w.w_qkv)), b_qkv=self._dev(w.b_qkv),
                     w_o=self._dev(_lib.linear_layout(w.w_o)), b_o=self._dev(w.b_o),
                     ln2_gamma=self._dev(w.ln2_g), ln2_beta=self._dev(w.ln2_b),
                     w_q_cross=self._dev(_lib.linear_layout(w.w_qc)), b_q_cross=self._dev(w.b_qc),
                     w_o_cross=self._dev(_lib.linear_layout(w.w_oc)), b_o_cross=self._dev(w.b_oc),
                     ln3_gamma=self._dev(w.ln3_g), ln3_beta=self._dev(w.ln3_b),
                     w_fc1=self._dev(_lib.linear_layout(w.w_fc1)), b_fc1=self._dev(w.b_fc1),
                     w_fc2=self._dev(_lib.linear_layout(w.w_fc2)), b_fc2=self._dev(w.b_fc2),
                     w_ck=self._dev(_lib.linear_layout(w.w_ck)), w_cv=self._dev(_lib.linear_layout(w.w_cv)),
                     b_cv=self._dev(w.b_cv))
            self._keep.append(t)
            fields = {k: v.data_ptr() for k, v in t.items() if k not in ("w_ck", "w_cv", "b_cv")}
            if not self.q8:
                self.structs.append(_lib.DecoderLayerWeights(**fields))
                continue
            codes = {}
            for name in self.MATRICES:
                w = t[name]
                c = torch.empty(w.shape, dtype=torch.int8, device=device)
                d = torch.empty((w.shape[1] // 32, w.shape[0]), dtype=torch.float16, device=device)
                _lib.edda_quantize_q8_0(w, c, d)
                codes[name] = (c, d)
                fields[name] = _lib.Q8Matrix(c.data_ptr(), d.data_ptr())
            self.codes.append(codes)
            self.structs.append(_lib.DecoderLayerWeightsQ8(**fields))
        shape = (self.n_frames, _lib.N_HEADS, _lib.HEAD_DIM)
        self.cross_k = [torch.empty(shape, dtype=torch.float16, device=device) for _ in self._keep]
        self.cross_v = [torch.empty(shape, dtype=torch.float16, device=device) for _ in self._keep]
        nb = _lib.decoder_verify_workspace_bytes(_lib.MAX_VERIFY_QUERIES, max_kv, self.n_frames)
        self.workspace = torch.zeros(max(nb, _lib.VERIFY_COUNTER_BYTES), dtype=torch.uint8, device=device)
        self._stack, self.stack_workspace = None, None

    def _dev(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.device)

    @property
    def layers(self) -> int:
        return len(self.structs)

    def set_encoder_output(self, enc, stream=None):
        """Project the encoder output [n_frames, 1280] into every layer's cross K/V."""
        for l, t in enumerate(self._keep):
            _lib.edda_cross_kv(enc, t["w_ck"], t["w_cv"], t["b_cv"], self.cross_k[l], self.cross_v[l], stream)

    def layer(self, x, layer: int, slots, k_cache, v_cache, n_kv, mask_rows, y, stream=None):
        _lib.edda_decoder_verify_layer(x, slots, k_cache, v_cache, n_kv, mask_rows, self.cross_k[layer],
                                       self.cross_v[layer], self.structs[layer], y, self.workspace, stream)

    def stack(self, x, slots, caches, n_kv, mask_rows, y, stream=None):
        """Every layer in order over the block x (edda_decoder_verify_stack, or _q8 for Q8_0
        weights): caches[l] = (k_cache, v_cache) of layer l; y receives the last layer's output."""
        cache_slots = caches[0][0].shape[0]
        if self._stack is None or self._stack[0] != [(k.data_ptr(), v.data_ptr()) for k, v in caches]:
            kind = _lib.DecoderStackLayerQ8 if self.q8 else _lib.DecoderStackLayer
            arr = (kind * len(self.structs))()
            for l, w in enumerate(self.structs):
                k, v = caches[l]
                arr[l] = kind(w, k.data_ptr(), v.data_ptr(), self.cross_k[l].data_ptr(), self.cross_v[l].data_ptr())
            self._stack = ([(k.data_ptr(), v.data_ptr()) for k, v in caches], arr)
        if self.stack_workspace is None:
            nb = _lib.decoder_verify_stack_workspace_bytes(_lib.MAX_VERIFY_QUERIES, _lib.DECODER_STACK_MAX_KV,
                                                           self.n_frames)
            self.stack_workspace = self.torch.zeros(nb, dtype=self.torch.uint8, device=self.device)
        _lib.edda_decoder_verify_stack(x, slots, cache_slots, n_kv, mask_rows, self.n_frames, self._stack[1], y,
                                       self.stack_workspace, stream)
