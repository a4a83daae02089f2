"""ctypes binding of libedda.so (argument marshalling only).

Every computation runs in the library's HIP kernels; this module turns torch
tensors into device pointers, passes the current HIP stream, and raises on a
non-zero status with the library's error text. PyTorch provides device memory
and streams and nothing else. There is no fallback: if the library is missing
or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# EDDA_LIBRARY names another build of the same library (e.g. the host-sanitizer build the ABI
# tests run against); default: the in-tree libedda.so.
LIB_PATH = os.environ.get("EDDA_LIBRARY") or os.path.join(HERE, "libedda.so")

D_MODEL = 1280
N_HEADS = 20
HEAD_DIM = 64
QKV_COLS = 3 * D_MODEL
MAX_VERIFY_QUERIES = 16
NOALLOC_MAX_KV = 8192  # most keys edda_verify_attn_noalloc takes (its static scratch)
VERIFY_COUNTER_BYTES = 16384  # leading workspace bytes of edda_verify_attn: zero before first use
DECODER_STACK_MAX_KV = 512  # largest cache edda_decoder_verify_stack serves
DECODER_STACK_ZERO_BYTES = 40960  # leading bytes of its workspace: zero before first use

STATUS = {0: "EDDA_OK", 1: "EDDA_ERR_INVALID_ARGUMENT", 2: "EDDA_ERR_UNSUPPORTED",
          3: "EDDA_ERR_MISALIGNED", 4: "EDDA_ERR_WORKSPACE", 5: "EDDA_ERR_HIP"}

# Every symbol include/edda.h declares.
EXPORTS = ("edda_qkv_pack", "edda_encoder_attn", "edda_flash_attn", "edda_encoder_workspace_bytes", "edda_verify_attn",
           "edda_verify_attn_noalloc",
           "edda_verify_workspace_bytes", "edda_linear", "edda_layer_norm", "edda_encoder_layer",
           "edda_encoder_layer_workspace_bytes", "edda_encoder_stem", "edda_encoder_stem_workspace_bytes",
           "edda_decoder_verify_layer", "edda_decoder_verify_workspace_bytes", "edda_cross_kv",
           "edda_verify_attn_ex", "edda_verify_workspace_bytes_ex",
           "edda_quantize_q8_0", "edda_linear_q8", "edda_decoder_verify_layer_q8",
           "edda_decoder_verify_stack", "edda_decoder_verify_stack_q8", "edda_decoder_verify_stack_workspace_bytes",
           "edda_last_error", "edda_version")

D_FF = 5120
ACT_NONE, ACT_GELU = 0, 1


class LayerWeights(ctypes.Structure):
    """edda_encoder_layer_weights: device pointers (Linear layout)."""
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "ln1_gamma", "ln1_beta", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_gamma", "ln2_beta",
        "w_fc1", "b_fc1", "w_fc2", "b_fc2")]


class DecoderLayerWeights(ctypes.Structure):
    """edda_decoder_layer_weights: device pointers (Linear layout)."""
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "ln1_gamma", "ln1_beta", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_gamma", "ln2_beta", "w_q_cross",
        "b_q_cross", "w_o_cross", "b_o_cross", "ln3_gamma", "ln3_beta", "w_fc1", "b_fc1", "w_fc2", "b_fc2")]


class Q8Matrix(ctypes.Structure):
    """edda_q8_matrix: Q8_0 codes int8 [out, in] and scales fp16 [in / 32, out] (device)."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class DecoderLayerWeightsQ8(ctypes.Structure):
    """edda_decoder_layer_weights_q8: projection matrices as Q8Matrix, the rest fp16 pointers."""
    _fields_ = [(name, Q8Matrix if name.startswith("w_") else ctypes.c_void_p) for name in (
        "ln1_gamma", "ln1_beta", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_gamma", "ln2_beta", "w_q_cross",
        "b_q_cross", "w_o_cross", "b_o_cross", "ln3_gamma", "ln3_beta", "w_fc1", "b_fc1", "w_fc2", "b_fc2")]


class DecoderStackLayer(ctypes.Structure):
    """edda_decoder_stack_layer: a layer's weights, its caches and its cross K/V (device)."""
    _fields_ = [("weights", DecoderLayerWeights), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("cross_k", ctypes.c_void_p), ("cross_v", ctypes.c_void_p)]


class DecoderStackLayerQ8(ctypes.Structure):
    """edda_decoder_stack_layer_q8: as DecoderStackLayer with Q8_0 projection weights."""
    _fields_ = [("weights", DecoderLayerWeightsQ8), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("cross_k", ctypes.c_void_p), ("cross_v", ctypes.c_void_p)]


class EddaError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libedda.so (once) and declare its prototypes. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or "
                           "python -m whisper_asr_encoder_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.edda_qkv_pack.argtypes = [vp, i64, vp, vp, vp, vp]
    lib.edda_encoder_attn.argtypes = [vp, i32, i32, i32, ctypes.POINTER(i32), vp, vp, vp, vp, sz, vp]
    lib.edda_flash_attn.argtypes = [vp, i32, i32, i32, ctypes.POINTER(i32), vp, vp]
    lib.edda_encoder_workspace_bytes.argtypes = [i32, i32]
    lib.edda_encoder_workspace_bytes.restype = sz
    lib.edda_verify_attn.argtypes = [vp, i32, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.edda_verify_attn_noalloc.argtypes = [vp, i32, vp, vp, i32, vp, vp, vp]
    lib.edda_verify_workspace_bytes.argtypes = [i32, i32]
    lib.edda_verify_workspace_bytes.restype = sz
    lib.edda_linear.argtypes = [vp, i64, i32, vp, i32, vp, i32, vp, i64, vp, vp]
    lib.edda_layer_norm.argtypes = [vp, i64, i32, vp, vp, vp, vp]
    lib.edda_encoder_layer.argtypes = [vp, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(LayerWeights), vp,
                                       vp, sz, vp]
    lib.edda_encoder_layer_workspace_bytes.argtypes = [i32, i32]
    lib.edda_encoder_layer_workspace_bytes.restype = sz
    lib.edda_encoder_stem.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.edda_encoder_stem_workspace_bytes.argtypes = [i32, i32, i32]
    lib.edda_encoder_stem_workspace_bytes.restype = sz
    lib.edda_decoder_verify_layer.argtypes = [vp, i32, ctypes.POINTER(i32), vp, vp, i32, i32, vp, vp, vp, i32,
                                              ctypes.POINTER(DecoderLayerWeights), vp, vp, sz, vp]
    lib.edda_decoder_verify_layer_q8.argtypes = [vp, i32, ctypes.POINTER(i32), vp, vp, i32, i32, vp, vp, vp, i32,
                                                 ctypes.POINTER(DecoderLayerWeightsQ8), vp, vp, sz, vp]
    lib.edda_decoder_verify_stack.argtypes = [vp, i32, ctypes.POINTER(i32), i32, i32, vp, i32,
                                              ctypes.POINTER(DecoderStackLayer), i32, vp, vp, sz, vp]
    lib.edda_decoder_verify_stack_q8.argtypes = [vp, i32, ctypes.POINTER(i32), i32, i32, vp, i32,
                                                 ctypes.POINTER(DecoderStackLayerQ8), i32, vp, vp, sz, vp]
    lib.edda_decoder_verify_stack_workspace_bytes.argtypes = [i32, i32, i32]
    lib.edda_decoder_verify_stack_workspace_bytes.restype = sz
    lib.edda_quantize_q8_0.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.edda_linear_q8.argtypes = [vp, ctypes.c_int64, i32, vp, vp, i32, vp, i32, vp, ctypes.c_int64, vp, vp]
    lib.edda_decoder_verify_workspace_bytes.argtypes = [i32, i32, i32]
    lib.edda_decoder_verify_workspace_bytes.restype = sz
    lib.edda_cross_kv.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
    lib.edda_verify_attn_ex.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.edda_verify_workspace_bytes_ex.argtypes = [i32, i32, i32]
    lib.edda_verify_workspace_bytes_ex.restype = sz
    lib.edda_last_error.restype = ctypes.c_char_p
    lib.edda_version.restype = ctypes.c_char_p
    for name in ("edda_qkv_pack", "edda_encoder_attn", "edda_flash_attn", "edda_verify_attn", "edda_verify_attn_noalloc",
                 "edda_linear",
                 "edda_layer_norm", "edda_encoder_layer", "edda_encoder_stem", "edda_decoder_verify_layer",
                 "edda_cross_kv", "edda_verify_attn_ex", "edda_quantize_q8_0", "edda_linear_q8",
                 "edda_decoder_verify_layer_q8", "edda_decoder_verify_stack", "edda_decoder_verify_stack_q8"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def last_error() -> str:
    return load().edda_last_error().decode()


def _check(status: int):
    if status != 0:
        raise EddaError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require(t, name, shape=None, dtype=None):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return torch


# ---------------------------------------------------------------------------
# Host-side layout helpers (load time, not part of the timed path).
# ---------------------------------------------------------------------------

def linear_layout(w_in_out: np.ndarray) -> np.ndarray:
    """Weight packing: a [in, out] matrix W (y = x W) -> its output-feature-major
    copy [out, in] (the layout the library reads; rows of a stacked q/k/v Linear weight)."""
    return np.ascontiguousarray(np.asarray(w_in_out, dtype=np.float16).T)


def conv_layout(w_out_in_tap: np.ndarray) -> np.ndarray:
    """Convolution weight [out, in, 3] -> [out, 3*in] with column tap*in + c (the layout of
    the stem's column-gathered GEMM)."""
    w = np.asarray(w_out_in_tap, dtype=np.float16)
    return np.ascontiguousarray(w.transpose(0, 2, 1).reshape(w.shape[0], -1))


def pack_mask_rows(mask: np.ndarray) -> np.ndarray:
    """bool [n_q, n_kv] -> uint32 [n_q, ceil(n_kv/32)], bit j % 32 of word j // 32 = slot j admitted."""
    mask = np.asarray(mask, dtype=bool)
    n_q, n_kv = mask.shape
    words = (n_kv + 31) // 32
    padded = np.zeros((n_q, words * 32), dtype=bool)
    padded[:, :n_kv] = mask
    packed = np.packbits(padded.reshape(n_q, words, 32), axis=2, bitorder="little")
    return np.ascontiguousarray(packed).view("<u4").reshape(n_q, words).astype(np.uint32)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI).
# ---------------------------------------------------------------------------

def edda_qkv_pack(x, w_qkv, b_qkv, qkv, stream=None):
    """qkv[rows, 3840] = x[rows, 1280] * w_qkv^T + b_qkv; w_qkv is [3840, 1280] (Linear layout)."""
    lib = load()
    torch = _require(x, "x", dtype=None)
    rows = x.shape[0]
    _require(x, "x", (rows, D_MODEL), torch.float16)
    _require(w_qkv, "w_qkv", (QKV_COLS, D_MODEL), torch.float16)
    if b_qkv is not None:
        _require(b_qkv, "b_qkv", (QKV_COLS,), torch.float16)
    _require(qkv, "qkv", (rows, QKV_COLS), torch.float16)
    _check(lib.edda_qkv_pack(_ptr(x), rows, _ptr(w_qkv), _ptr(b_qkv), _ptr(qkv), _stream(stream)))


def encoder_workspace_bytes(batch: int, seq_len: int) -> int:
    return int(load().edda_encoder_workspace_bytes(batch, seq_len))


def edda_encoder_attn(qkv, batch, seq_len, chunk_len, valid_len, w_o, b_o, y, workspace, stream=None):
    """y = attention(qkv) * w_o^T + b_o over `batch` windows of `seq_len` rows.
    valid_len: host sequence of ints (or None); workspace: device uint8 tensor."""
    lib = load()
    torch = _require(qkv, "qkv", (batch * seq_len, QKV_COLS))
    _require(w_o, "w_o", (D_MODEL, D_MODEL), torch.float16)
    if b_o is not None:
        _require(b_o, "b_o", (D_MODEL,), torch.float16)
    _require(y, "y", (batch * seq_len, D_MODEL), torch.float16)
    _require(workspace, "workspace")
    _require(qkv, "qkv", dtype=torch.float16)
    keep, vl = _valid_arg(valid_len, batch)
    _check(lib.edda_encoder_attn(_ptr(qkv), batch, seq_len, chunk_len, vl, _ptr(w_o), _ptr(b_o), _ptr(y),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))
    del keep


def _valid_arg(valid_len, batch):
    if valid_len is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(valid_len, dtype=np.int32).reshape(-1))
    if arr.size != batch:
        raise ValueError(f"valid_len must have {batch} entries")
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def edda_flash_attn(qkv, batch, seq_len, chunk_len, valid_len, o, stream=None):
    """o[rows, 1280] = per-head masked softmax attention of qkv (no output projection)."""
    lib = load()
    torch = _require(qkv, "qkv", (batch * seq_len, QKV_COLS))
    _require(qkv, "qkv", dtype=torch.float16)
    _require(o, "o", (batch * seq_len, D_MODEL), torch.float16)
    keep, vl = _valid_arg(valid_len, batch)
    _check(lib.edda_flash_attn(_ptr(qkv), batch, seq_len, chunk_len, vl, _ptr(o), _stream(stream)))
    del keep


def verify_workspace_bytes(n_q: int, n_kv: int) -> int:
    return int(load().edda_verify_workspace_bytes(n_q, n_kv))


def edda_verify_attn(q, k, v, mask_rows, o, workspace=None, stream=None):
    """o[n_q,20,64] = softmax over admitted slots of (q.k/8) times v. mask_rows: device uint32
    tensor [n_q, ceil(n_kv/32)] (see pack_mask_rows) or None for every slot admitted."""
    lib = load()
    torch = _require(q, "q")
    n_q, n_kv = q.shape[0], k.shape[0]
    _require(q, "q", (n_q, N_HEADS, HEAD_DIM), torch.float16)
    _require(k, "k", (n_kv, N_HEADS, HEAD_DIM), torch.float16)
    _require(v, "v", (n_kv, N_HEADS, HEAD_DIM), torch.float16)
    _require(o, "o", (n_q, N_HEADS, HEAD_DIM), torch.float16)
    if mask_rows is not None:
        _require(mask_rows, "mask_rows", (n_q, (n_kv + 31) // 32))
        if mask_rows.dtype not in (torch.int32, torch.uint32):
            raise ValueError("mask_rows must hold 32-bit words")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.edda_verify_attn(_ptr(q), n_q, _ptr(k), _ptr(v), n_kv, _ptr(mask_rows), _ptr(o),
                                _ptr(workspace), ws_bytes, _stream(stream)))


def edda_verify_attn_noalloc(q, k, v, mask_rows, o, stream=None):
    """edda_verify_attn with the library's static scratch instead of a workspace (n_kv up to
    NOALLOC_MAX_KV; calls on one GPU must not overlap)."""
    lib = load()
    torch = _require(q, "q")
    n_q, n_kv = q.shape[0], k.shape[0]
    _require(q, "q", (n_q, N_HEADS, HEAD_DIM), torch.float16)
    _require(k, "k", (n_kv, N_HEADS, HEAD_DIM), torch.float16)
    _require(v, "v", (n_kv, N_HEADS, HEAD_DIM), torch.float16)
    _require(o, "o", (n_q, N_HEADS, HEAD_DIM), torch.float16)
    if mask_rows is not None:
        _require(mask_rows, "mask_rows", (n_q, (n_kv + 31) // 32))
        if mask_rows.dtype not in (torch.int32, torch.uint32):
            raise ValueError("mask_rows must hold 32-bit words")
    _check(lib.edda_verify_attn_noalloc(_ptr(q), n_q, _ptr(k), _ptr(v), n_kv, _ptr(mask_rows), _ptr(o),
                                        _stream(stream)))


def edda_linear(x, w, bias, y, activation=ACT_NONE, residual=None, residual_rows=None, stream=None):
    """y[rows, out] = act(x[rows, in] * w^T + bias) + residual[row % residual_rows]; w is [out, in]."""
    lib = load()
    torch = _require(x, "x")
    rows, k = x.shape
    n = w.shape[0]
    _require(x, "x", (rows, k), torch.float16)
    _require(w, "w", (n, k), torch.float16)
    if bias is not None:
        _require(bias, "bias", (n,), torch.float16)
    _require(y, "y", (rows, n), torch.float16)
    if residual is not None:
        residual_rows = residual.shape[0] if residual_rows is None else residual_rows
        _require(residual, "residual", (residual.shape[0], n), torch.float16)
        if residual.shape[0] < min(residual_rows, rows):
            raise ValueError("residual has fewer rows than residual_rows")
    _check(lib.edda_linear(_ptr(x), rows, k, _ptr(w), n, _ptr(bias), activation, _ptr(residual),
                           residual_rows or 0, _ptr(y), _stream(stream)))


def edda_layer_norm(x, gamma, beta, y, stream=None):
    lib = load()
    torch = _require(x, "x")
    rows, f = x.shape
    _require(x, "x", (rows, f), torch.float16)
    _require(gamma, "gamma", (f,), torch.float16)
    _require(beta, "beta", (f,), torch.float16)
    _require(y, "y", (rows, f), torch.float16)
    _check(lib.edda_layer_norm(_ptr(x), rows, f, _ptr(gamma), _ptr(beta), _ptr(y), _stream(stream)))


def encoder_layer_workspace_bytes(batch: int, seq_len: int) -> int:
    return int(load().edda_encoder_layer_workspace_bytes(batch, seq_len))


def edda_encoder_layer(x, batch, seq_len, chunk_len, valid_len, weights: "LayerWeights", y, workspace,
                       stream=None):
    """One pre-norm encoder layer; weights: a LayerWeights of device pointers (kept alive by the caller)."""
    lib = load()
    torch = _require(x, "x")
    rows = batch * seq_len
    _require(x, "x", (rows, D_MODEL), torch.float16)
    _require(y, "y", (rows, D_MODEL), torch.float16)
    vl = None
    if valid_len is not None:
        arr = (ctypes.c_int32 * batch)(*[int(v) for v in valid_len])
        vl = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.edda_encoder_layer(_ptr(x), batch, seq_len, chunk_len, vl, ctypes.byref(weights), _ptr(y),
                                  _ptr(workspace), ws_bytes, _stream(stream)))


def encoder_stem_workspace_bytes(batch: int, n_mels: int, n_frames: int) -> int:
    return int(load().edda_encoder_stem_workspace_bytes(batch, n_mels, n_frames))


def edda_encoder_stem(mel, conv1_w, conv1_b, conv2_w, conv2_b, pos, y, workspace, stream=None):
    """mel [batch, n_mels, n_frames] -> y [batch * ((n_frames + 1) // 2), 1280]; conv weights in
    conv_layout ([1280, 3 * in])."""
    lib = load()
    torch = _require(mel, "mel")
    batch, n_mels, n_frames = mel.shape
    t2 = (n_frames - 1) // 2 + 1
    _require(mel, "mel", (batch, n_mels, n_frames), torch.float16)
    _require(conv1_w, "conv1_w", (D_MODEL, 3 * n_mels), torch.float16)
    _require(conv2_w, "conv2_w", (D_MODEL, 3 * D_MODEL), torch.float16)
    _require(pos, "pos", (t2, D_MODEL), torch.float16)
    _require(y, "y", (batch * t2, D_MODEL), torch.float16)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.edda_encoder_stem(_ptr(mel), batch, n_mels, n_frames, _ptr(conv1_w), _ptr(conv1_b), _ptr(conv2_w),
                                 _ptr(conv2_b), _ptr(pos), _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)))


def decoder_verify_workspace_bytes(n_q: int, n_kv: int, n_frames: int) -> int:
    return int(load().edda_decoder_verify_workspace_bytes(n_q, n_kv, n_frames))


def edda_decoder_verify_layer(x, slots, k_cache, v_cache, n_kv, mask_rows, cross_k, cross_v,
                              weights, y, workspace, stream=None):
    """One decoder layer over the block rows x [n_q, 1280]; slots: host ints; caches
    [cache_slots, 20, 64] updated in place; mask_rows as for edda_verify_attn (or None).
    weights: DecoderLayerWeights (fp16) or DecoderLayerWeightsQ8 (Q8_0 projections)."""
    lib = load()
    torch = _require(x, "x")
    n_q = x.shape[0]
    _require(x, "x", (n_q, D_MODEL), torch.float16)
    _require(y, "y", (n_q, D_MODEL), torch.float16)
    cache_slots = k_cache.shape[0]
    _require(k_cache, "k_cache", (cache_slots, N_HEADS, HEAD_DIM), torch.float16)
    _require(v_cache, "v_cache", (cache_slots, N_HEADS, HEAD_DIM), torch.float16)
    n_frames = cross_k.shape[0]
    _require(cross_k, "cross_k", (n_frames, N_HEADS, HEAD_DIM), torch.float16)
    _require(cross_v, "cross_v", (n_frames, N_HEADS, HEAD_DIM), torch.float16)
    if mask_rows is not None:
        _require(mask_rows, "mask_rows", (n_q, (n_kv + 31) // 32))
    arr = (ctypes.c_int32 * n_q)(*[int(v) for v in slots])
    ws_bytes = workspace.numel() * workspace.element_size()
    fn = lib.edda_decoder_verify_layer_q8 if isinstance(weights, DecoderLayerWeightsQ8) else lib.edda_decoder_verify_layer
    _check(fn(_ptr(x), n_q, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), _ptr(k_cache), _ptr(v_cache),
              cache_slots, n_kv, _ptr(mask_rows), _ptr(cross_k), _ptr(cross_v), n_frames, ctypes.byref(weights),
              _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)))


def decoder_verify_stack_workspace_bytes(n_q: int, n_kv: int, n_frames: int) -> int:
    return int(load().edda_decoder_verify_stack_workspace_bytes(n_q, n_kv, n_frames))


def edda_decoder_verify_stack(x, slots, cache_slots, n_kv, mask_rows, n_frames, layers, y, workspace, stream=None):
    """Consecutive decoder layers over the block rows x [n_q, 1280] into y; layers: a ctypes
    array of DecoderStackLayer (fp16 weights) or DecoderStackLayerQ8 (Q8_0 projections), with
    caches [cache_slots, 20, 64] updated in place and cross K/V [n_frames, 20, 64]; slots host
    ints; mask_rows as for edda_verify_attn (or None)."""
    lib = load()
    torch = _require(x, "x")
    n_q = x.shape[0]
    _require(x, "x", (n_q, D_MODEL), torch.float16)
    _require(y, "y", (n_q, D_MODEL), torch.float16)
    if mask_rows is not None:
        _require(mask_rows, "mask_rows", (n_q, (n_kv + 31) // 32))
    arr = (ctypes.c_int32 * n_q)(*[int(v) for v in slots])
    ws_bytes = workspace.numel() * workspace.element_size()
    fn = lib.edda_decoder_verify_stack_q8 if layers._type_ is DecoderStackLayerQ8 else lib.edda_decoder_verify_stack
    _check(fn(_ptr(x), n_q, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), cache_slots, n_kv, _ptr(mask_rows),
              n_frames, layers, len(layers), _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)))


def edda_cross_kv(enc, w_k, w_v, b_v, cross_k, cross_v, stream=None):
    """cross_k = enc w_k^T, cross_v = enc w_v^T + b_v; enc [n_frames, 1280], outputs [n_frames, 20, 64]."""
    lib = load()
    torch = _require(enc, "enc")
    n = enc.shape[0]
    _require(enc, "enc", (n, D_MODEL), torch.float16)
    _require(w_k, "w_k", (D_MODEL, D_MODEL), torch.float16)
    _require(w_v, "w_v", (D_MODEL, D_MODEL), torch.float16)
    _require(cross_k, "cross_k", (n, N_HEADS, HEAD_DIM), torch.float16)
    _require(cross_v, "cross_v", (n, N_HEADS, HEAD_DIM), torch.float16)
    _check(lib.edda_cross_kv(_ptr(enc), n, _ptr(w_k), _ptr(w_v), _ptr(b_v), _ptr(cross_k), _ptr(cross_v),
                             _stream(stream)))


MASK_ROWS, MASK_NONE, MASK_CAUSAL_BLOCK = 0, 1, 2
MAX_VERIFY_HEADS = 64


def verify_workspace_bytes_ex(n_q: int, n_kv: int, n_heads: int) -> int:
    return int(load().edda_verify_workspace_bytes_ex(n_q, n_kv, n_heads))


def edda_verify_attn_ex(q, k, v, o, mask_mode=MASK_NONE, mask_rows=None, sinks=None, workspace=None, stream=None):
    """Verification attention with n_heads = q.shape[1] (head_dim 64), a mask mode and optional
    fp32 sinks [n_heads] (device)."""
    lib = load()
    torch = _require(q, "q")
    n_q, n_heads, _ = q.shape
    n_kv = k.shape[0]
    _require(q, "q", (n_q, n_heads, HEAD_DIM), torch.float16)
    _require(k, "k", (n_kv, n_heads, HEAD_DIM), torch.float16)
    _require(v, "v", (n_kv, n_heads, HEAD_DIM), torch.float16)
    _require(o, "o", (n_q, n_heads, HEAD_DIM), torch.float16)
    if sinks is not None:
        _require(sinks, "sinks", (n_heads,), torch.float32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.edda_verify_attn_ex(_ptr(q), n_q, _ptr(k), _ptr(v), n_kv, n_heads, mask_mode, _ptr(mask_rows),
                                   _ptr(sinks), _ptr(o), _ptr(workspace), ws_bytes, _stream(stream)))


def edda_quantize_q8_0(w, codes, scales, stream=None):
    """Q8_0 codes int8 [rows, cols] and scales fp16 [cols / 32, rows] of fp16 w [rows, cols]."""
    lib = load()
    torch = _require(w, "w")
    rows, cols = w.shape
    _require(w, "w", (rows, cols), torch.float16)
    _require(codes, "codes", (rows, cols), torch.int8)
    _require(scales, "scales", (cols // 32, rows), torch.float16)
    _check(lib.edda_quantize_q8_0(_ptr(w), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))


def edda_linear_q8(x, codes, scales, bias, y, activation=ACT_NONE, residual=None, residual_rows=None, stream=None):
    """edda_linear with Q8_0 weights (codes [out, in], scales [in / 32, out]); rows <= 16."""
    lib = load()
    torch = _require(x, "x")
    rows, k = x.shape
    n = codes.shape[0]
    _require(x, "x", (rows, k), torch.float16)
    _require(codes, "codes", (n, k), torch.int8)
    _require(scales, "scales", (k // 32, n), torch.float16)
    if bias is not None:
        _require(bias, "bias", (n,), torch.float16)
    _require(y, "y", (rows, n), torch.float16)
    if residual is not None:
        residual_rows = residual.shape[0] if residual_rows is None else residual_rows
        _require(residual, "residual", (residual.shape[0], n), torch.float16)
    _check(lib.edda_linear_q8(_ptr(x), rows, k, _ptr(codes), _ptr(scales), n, _ptr(bias), activation,
                              _ptr(residual), residual_rows or 0, _ptr(y), _stream(stream)))
