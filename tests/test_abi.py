"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects every invalid argument with its
documented status before any HIP call (fake, never-dereferenced addresses are
passed; validation must fail first)."""
import ctypes
import os
import re

import pytest

from whisper_asr_encoder_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "edda.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, HIP = range(6)
A = 1 << 20           # a 16-byte aligned fake device address (never dereferenced here)
B = A + 0x10000
ODD = A + 2           # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libedda.so not built")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(edda_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_error_text(lib):
    assert b"gfx950" in lib.edda_version()
    assert lib.edda_qkv_pack(None, 10, None, None, None, None) == INVALID
    assert b"non-null" in lib.edda_last_error()


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (EDDA_\w+) (\d+)", text))
    assert int(consts["EDDA_VERIFY_COUNTER_BYTES"]) == _lib.VERIFY_COUNTER_BYTES
    assert int(consts["EDDA_MAX_VERIFY_QUERIES"]) == _lib.MAX_VERIFY_QUERIES
    assert int(consts["EDDA_MAX_VERIFY_HEADS"]) == _lib.MAX_VERIFY_HEADS
    enum = dict(re.findall(r"(EDDA_MASK_\w+) = (\d+)", text))
    assert {k: int(v) for k, v in enum.items()} == {"EDDA_MASK_ROWS": _lib.MASK_ROWS, "EDDA_MASK_NONE": _lib.MASK_NONE,
                                                     "EDDA_MASK_CAUSAL_BLOCK": _lib.MASK_CAUSAL_BLOCK}
    assert int(consts["EDDA_D_MODEL"]) == _lib.D_MODEL


def test_workspace_sizes(lib):
    assert lib.edda_encoder_workspace_bytes(1, 1500) == 1500 * 1280 * 2
    assert lib.edda_encoder_workspace_bytes(16, 1500) == 16 * 1500 * 1280 * 2
    assert lib.edda_encoder_workspace_bytes(0, 1500) == 0
    assert lib.edda_encoder_workspace_bytes(1, -3) == 0
    assert lib.edda_verify_workspace_bytes(16, 100) == 0      # one split: no workspace
    assert lib.edda_verify_workspace_bytes(16, 128) == 0
    assert lib.edda_verify_workspace_bytes(16, 512) == 0      # still one workgroup per head
    C = _lib.VERIFY_COUNTER_BYTES
    assert lib.edda_verify_workspace_bytes(16, 513) == C + 5 * 16 * 20 * 66 * 4  # counters + partials
    assert lib.edda_verify_workspace_bytes(3, 1500) == C + 12 * 3 * 20 * 66 * 4
    assert lib.edda_verify_workspace_bytes(17, 1500) == 0      # invalid n_q
    assert lib.edda_verify_workspace_bytes(1, 0) == 0


@pytest.mark.parametrize("args,status", [
    ((None, 10, A, None, B, None), INVALID),
    ((A, 0, A, None, B, None), INVALID),
    ((A, -1, A, None, B, None), INVALID),
    ((A, 1 << 40, A, None, B, None), INVALID),
    ((ODD, 10, A, None, B, None), MISALIGNED),
    ((A, 10, A, ODD, B, None), MISALIGNED),
    ((A, 10, A, None, ODD, None), MISALIGNED),
])
def test_qkv_pack_rejects(lib, args, status):
    assert lib.edda_qkv_pack(*args) == status


def enc(lib, qkv=A, batch=1, seq=200, chunk=0, valid=None, w_o=A, b_o=None, y=B, ws=B + (1 << 24),
        ws_bytes=1 << 30):
    vl = None
    if valid is not None:
        arr = (ctypes.c_int32 * len(valid))(*valid)
        vl = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return lib.edda_encoder_attn(qkv, batch, seq, chunk, vl, w_o, b_o, y, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=None), INVALID), (dict(w_o=None), INVALID), (dict(y=None), INVALID),
    (dict(batch=0), INVALID), (dict(seq=0), INVALID), (dict(chunk=-1), INVALID),
    (dict(chunk=201), INVALID), (dict(batch=2, valid=[200, 0]), INVALID),
    (dict(batch=2, valid=[201, 5]), INVALID), (dict(valid=[-4]), INVALID),
    (dict(batch=1 << 20, seq=1500), INVALID),
    (dict(qkv=ODD), MISALIGNED), (dict(b_o=ODD), MISALIGNED), (dict(ws=ODD), MISALIGNED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=200 * 1280 * 2 - 1), WORKSPACE),
])
def test_encoder_attn_rejects(lib, kw, status):
    assert enc(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=None), INVALID), (dict(o=None), INVALID), (dict(batch=0), INVALID), (dict(seq=-1), INVALID),
    (dict(chunk=300), INVALID), (dict(valid=[0]), INVALID), (dict(qkv=ODD), MISALIGNED), (dict(o=ODD), MISALIGNED),
])
def test_flash_attn_rejects(lib, kw, status):
    args = dict(qkv=A, batch=1, seq=200, chunk=0, valid=None, o=B)
    args.update(kw)
    vl = None
    if args["valid"] is not None:
        arr = (ctypes.c_int32 * len(args["valid"]))(*args["valid"])
        vl = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    assert lib.edda_flash_attn(args["qkv"], args["batch"], args["seq"], args["chunk"], vl, args["o"], None) == status


def ver(lib, q=A, n_q=16, k=A, v=A, n_kv=448, mask=None, o=B, ws=B + (1 << 24), ws_bytes=1 << 30):
    return lib.edda_verify_attn(q, n_q, k, v, n_kv, mask, o, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(n_q=0), INVALID), (dict(n_q=17), INVALID), (dict(n_kv=0), INVALID), (dict(n_kv=-5), INVALID),
    (dict(q=ODD), MISALIGNED), (dict(o=ODD), MISALIGNED), (dict(mask=A + 2), MISALIGNED),
    (dict(ws=None, n_kv=1500), WORKSPACE), (dict(ws_bytes=16, n_kv=513), WORKSPACE),
])
def test_verify_attn_rejects(lib, kw, status):
    assert ver(lib, **kw) == status


def ver_ex(lib, q=A, n_q=16, k=A, v=A, n_kv=448, h=8, mode=1, mask=None, sinks=None, o=B, ws=B + (1 << 24),
           ws_bytes=1 << 30):
    return lib.edda_verify_attn_ex(q, n_q, k, v, n_kv, h, mode, mask, sinks, o, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(n_q=0), INVALID), (dict(n_q=17), INVALID),
    (dict(h=0), INVALID), (dict(h=65), INVALID), (dict(n_kv=0), INVALID), (dict(n_kv=1 << 20, h=64), INVALID),
    (dict(mode=3), INVALID), (dict(mode=-1), INVALID), (dict(mode=0), INVALID),
    (dict(mode=2, n_q=16, n_kv=15), INVALID), (dict(q=ODD), MISALIGNED), (dict(sinks=A + 2), MISALIGNED),
    (dict(mode=0, mask=A + 2), MISALIGNED), (dict(ws=None, n_kv=1500), WORKSPACE),
    (dict(ws_bytes=16, n_kv=513), WORKSPACE),
])
def test_verify_attn_ex_rejects(lib, kw, status):
    assert ver_ex(lib, **kw) == status


def test_verify_workspace_bytes_ex(lib):
    C = _lib.VERIFY_COUNTER_BYTES
    assert lib.edda_verify_workspace_bytes_ex(16, 512, 64) == 0
    assert lib.edda_verify_workspace_bytes_ex(16, 513, 64) == C + 5 * 16 * 64 * 66 * 4
    assert lib.edda_verify_workspace_bytes_ex(4, 1500, 20) == lib.edda_verify_workspace_bytes(4, 1500)
    assert lib.edda_verify_workspace_bytes_ex(4, 1500, 0) == 0
    assert lib.edda_verify_workspace_bytes_ex(4, 1500, 65) == 0


def test_mask_packing_bit_order():
    import numpy as np
    m = np.zeros((2, 40), dtype=bool)
    m[0, [0, 5, 31, 32, 39]] = True
    m[1, :] = True
    w = _lib.pack_mask_rows(m)
    assert w.shape == (2, 2) and w.dtype == np.uint32
    assert w[0, 0] == (1 | (1 << 5) | (1 << 31)) and w[0, 1] == (1 | (1 << 7))
    assert w[1, 0] == 0xFFFFFFFF and w[1, 1] == 0xFF


# ---------------------------------------------------------------------------
# The rest of the encoder: linear, LayerNorm, encoder layer, stem.
# ---------------------------------------------------------------------------

def lin(lib, x=A, rows=100, k=1280, w=A, n=1280, bias=None, act=0, res=None, res_rows=0, y=B):
    return lib.edda_linear(x, rows, k, w, n, bias, act, res, res_rows, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID), (dict(rows=0), INVALID),
    (dict(k=0), INVALID), (dict(n=-64), INVALID), (dict(act=2), INVALID), (dict(res=A, res_rows=0), INVALID),
    (dict(rows=1 << 30), INVALID), (dict(k=100), UNSUPPORTED), (dict(n=1000), UNSUPPORTED),
    (dict(x=ODD), MISALIGNED), (dict(y=ODD), MISALIGNED), (dict(bias=ODD), MISALIGNED),
    (dict(res=ODD, res_rows=10), MISALIGNED),
])
def test_linear_rejects(lib, kw, status):
    assert lin(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(g=None), INVALID), (dict(rows=0), INVALID), (dict(f=1000), UNSUPPORTED),
    (dict(f=8192), UNSUPPORTED), (dict(x=ODD), MISALIGNED), (dict(b=ODD), MISALIGNED),
])
def test_layer_norm_rejects(lib, kw, status):
    a = dict(x=A, rows=10, f=1280, g=A, b=A, y=B)
    a.update(kw)
    assert lib.edda_layer_norm(a["x"], a["rows"], a["f"], a["g"], a["b"], a["y"], None) == status


def layer_weights(**over):
    w = _lib.LayerWeights(*([A] * 12))
    for k, v in over.items():
        setattr(w, k, v)
    return w


@pytest.mark.parametrize("kw,wover,status", [
    (dict(x=None), {}, INVALID), (dict(batch=0), {}, INVALID), (dict(chunk=500), {}, INVALID),
    (dict(), dict(w_fc1=None), INVALID), (dict(), dict(ln2_gamma=None), INVALID),
    (dict(), dict(w_o=ODD), MISALIGNED), (dict(y=ODD), {}, MISALIGNED),
    (dict(ws=None), {}, WORKSPACE), (dict(ws_bytes=200 * 7680 * 2 - 1), {}, WORKSPACE),
])
def test_encoder_layer_rejects(lib, kw, wover, status):
    a = dict(x=A, batch=1, seq=200, chunk=0, y=B, ws=B + (1 << 24), ws_bytes=1 << 30)
    a.update(kw)
    w = layer_weights(**wover)
    assert lib.edda_encoder_layer(a["x"], a["batch"], a["seq"], a["chunk"], None, ctypes.byref(w), a["y"],
                                  a["ws"], a["ws_bytes"], None) == status


def test_encoder_layer_allows_null_biases_in_validation(lib):
    # Biases may be NULL: with a too-small workspace the call still fails on the workspace only.
    w = layer_weights(b_qkv=None, b_o=None, b_fc1=None, b_fc2=None)
    assert lib.edda_encoder_layer(A, 1, 200, 0, None, ctypes.byref(w), B, None, 0, None) == WORKSPACE


@pytest.mark.parametrize("kw,status", [
    (dict(mel=None), INVALID), (dict(pos=None), INVALID), (dict(batch=0), INVALID), (dict(frames=0), INVALID),
    (dict(mels=100), UNSUPPORTED), (dict(mel=ODD), MISALIGNED), (dict(c1b=ODD), MISALIGNED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=1000), WORKSPACE),
])
def test_encoder_stem_rejects(lib, kw, status):
    a = dict(mel=A, batch=1, mels=128, frames=3000, c1w=A, c1b=None, c2w=A, c2b=None, pos=A, y=B,
             ws=B + (1 << 24), ws_bytes=1 << 30)
    a.update(kw)
    assert lib.edda_encoder_stem(a["mel"], a["batch"], a["mels"], a["frames"], a["c1w"], a["c1b"], a["c2w"],
                                 a["c2b"], a["pos"], a["y"], a["ws"], a["ws_bytes"], None) == status


def test_layer_and_stem_workspace_sizes(lib):
    assert lib.edda_encoder_layer_workspace_bytes(1, 1500) == 1500 * (5120 + 2 * 1280) * 2
    assert lib.edda_encoder_layer_workspace_bytes(0, 1500) == 0
    assert lib.edda_encoder_stem_workspace_bytes(1, 128, 3000) == (3000 * 384 + 3000 * 1280 + 1500 * 3840) * 2
    assert lib.edda_encoder_stem_workspace_bytes(2, 128, 7) == (14 * 384 + 14 * 1280 + 8 * 3840) * 2
    assert lib.edda_encoder_stem_workspace_bytes(1, 128, 0) == 0


# ---------------------------------------------------------------------------
# Decoder verification layer and cross K/V.
# ---------------------------------------------------------------------------

def dec(lib, x=A, n_q=16, slots=tuple(range(24, 40)), kc=A, vc=A, cap=448, n_kv=40, mask=None, ck=A, cv=A,
        frames=1500, wover=None, y=B, ws=B + (1 << 24), ws_bytes=1 << 30):
    w = _lib.DecoderLayerWeights(*([A] * 18))
    for k, v in (wover or {}).items():
        setattr(w, k, v)
    arr = None
    if slots is not None:
        arr = ctypes.cast((ctypes.c_int32 * max(len(slots), 1))(*slots), ctypes.POINTER(ctypes.c_int32))
    return lib.edda_decoder_verify_layer(x, n_q, arr, kc, vc, cap, n_kv, mask, ck, cv, frames, ctypes.byref(w), y,
                                         ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(slots=None), INVALID), (dict(kc=None), INVALID), (dict(ck=None), INVALID),
    (dict(n_q=0, slots=(1,)), INVALID), (dict(n_q=17, slots=tuple(range(17))), INVALID),
    (dict(n_kv=0), INVALID), (dict(n_kv=500), INVALID), (dict(frames=0), INVALID),
    (dict(n_q=2, slots=(3, 40)), INVALID), (dict(n_q=2, slots=(-1, 3)), INVALID), (dict(n_q=2, slots=(5, 5)), INVALID),
    (dict(wover=dict(w_fc2=None)), INVALID), (dict(wover=dict(ln3_beta=None)), INVALID),
    (dict(x=ODD), MISALIGNED), (dict(wover=dict(b_o_cross=ODD)), MISALIGNED), (dict(mask=A + 2), MISALIGNED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=1000), WORKSPACE),
])
def test_decoder_verify_layer_rejects(lib, kw, status):
    assert dec(lib, **kw) == status


def stack(lib, x=A, n_q=16, slots=tuple(range(24, 40)), cap=448, n_kv=40, mask=None, frames=1500, n_layers=3,
          lover=None, wover=None, y=B, ws=B + (1 << 24), ws_bytes=1 << 30, layers="default"):
    arr = (_lib.DecoderStackLayer * max(n_layers, 1))()
    for l in range(max(n_layers, 1)):
        arr[l] = _lib.DecoderStackLayer(_lib.DecoderLayerWeights(*([A] * 18)), A, A, A, A)
    for k, v in (wover or {}).items():
        setattr(arr[n_layers - 1].weights, k, v)
    for k, v in (lover or {}).items():
        setattr(arr[n_layers - 1], k, v)
    sl = None
    if slots is not None:
        sl = ctypes.cast((ctypes.c_int32 * max(len(slots), 1))(*slots), ctypes.POINTER(ctypes.c_int32))
    return lib.edda_decoder_verify_stack(x, n_q, sl, cap, n_kv, mask, frames, arr if layers == "default" else layers,
                                         n_layers, y, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(slots=None), INVALID), (dict(layers=None), INVALID), (dict(y=None), INVALID),
    (dict(n_layers=0), INVALID), (dict(n_q=17, slots=tuple(range(17))), INVALID), (dict(n_kv=500), INVALID),
    (dict(frames=0), INVALID), (dict(n_q=2, slots=(5, 5)), INVALID), (dict(n_q=2, slots=(3, 40)), INVALID),
    (dict(cap=600, n_kv=513), UNSUPPORTED), (dict(frames=6145), UNSUPPORTED),
    (dict(wover=dict(w_fc1=None)), INVALID), (dict(lover=dict(cross_v=None)), INVALID),
    (dict(lover=dict(k_cache=None)), INVALID), (dict(wover=dict(b_fc2=ODD)), MISALIGNED),
    (dict(lover=dict(v_cache=ODD)), MISALIGNED), (dict(ws=B + 16), MISALIGNED), (dict(x=ODD), MISALIGNED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=1 << 20), WORKSPACE),
])
def test_decoder_verify_stack_rejects(lib, kw, status):
    assert stack(lib, **kw) == status
    assert lib.edda_last_error()


def test_decoder_verify_stack_q8_rejects(lib):
    arr = (_lib.DecoderStackLayerQ8 * 2)()
    for l in range(2):
        w = _lib.DecoderLayerWeightsQ8()
        for name, kind in _lib.DecoderLayerWeightsQ8._fields_:
            setattr(w, name, _lib.Q8Matrix(A, A) if kind is _lib.Q8Matrix else A)
        arr[l] = _lib.DecoderStackLayerQ8(w, A, A, A, A)
    sl = ctypes.cast((ctypes.c_int32 * 16)(*range(24, 40)), ctypes.POINTER(ctypes.c_int32))
    call = lambda: lib.edda_decoder_verify_stack_q8(A, 16, sl, 448, 40, None, 1500, arr, 2, B, B + (1 << 24), 1 << 30,
                                                     None)
    arr[1].weights.w_fc2 = _lib.Q8Matrix(A, None)
    assert call() == INVALID and b"scales" in lib.edda_last_error()
    arr[1].weights.w_fc2 = _lib.Q8Matrix(A, ODD)
    assert call() == MISALIGNED
    arr[1].weights.w_fc2 = _lib.Q8Matrix(None, A)
    assert call() == INVALID


def test_decoder_stack_workspace_bytes(lib):
    n = lib.edda_decoder_verify_stack_workspace_bytes(16, 448, 1500)
    # zeroed counters and flags, cross partials (3 splits of 512 frames), carry rows, 8 blocks of
    # per-layer rows
    block = 16 * 2 * (3840 + 6 * 1280 + 5120)
    assert n == _lib.DECODER_STACK_ZERO_BYTES + 3 * 16 * 20 * 66 * 4 + 16 * 1280 * 2 + 8 * block
    assert lib.edda_decoder_verify_stack_workspace_bytes(16, 513, 1500) == 0
    assert lib.edda_decoder_verify_stack_workspace_bytes(17, 448, 1500) == 0
    assert lib.edda_decoder_verify_stack_workspace_bytes(1, 448, 6145) == 0


@pytest.mark.parametrize("args,status", [
    ((None, 1500, A, A, None, B, B), INVALID), ((A, 0, A, A, None, B, B), INVALID),
    ((A, 1500, A, None, None, B, B), INVALID), ((A, 1500, A, A, ODD, B, B), MISALIGNED),
    ((A, 1500, A, A, None, B, ODD), MISALIGNED),
])
def test_cross_kv_rejects(lib, args, status):
    assert lib.edda_cross_kv(*args, None) == status


def test_decoder_workspace_sizes(lib):
    n = lib.edda_decoder_verify_workspace_bytes(16, 360, 1500)
    verify = max(lib.edda_verify_workspace_bytes(16, 360), lib.edda_verify_workspace_bytes(16, 1500))
    assert n >= verify + 16 * (4 * 1280 + 3840 + 5120) * 2  # h, o, x1, x2, qkv, MLP hidden
    assert lib.edda_decoder_verify_workspace_bytes(17, 360, 1500) == 0
    assert lib.edda_decoder_verify_workspace_bytes(1, 0, 1500) == 0


def q8(lib, w=A, rows=64, cols=128, codes=B, scales=B + 4096):
    return lib.edda_quantize_q8_0(w, rows, cols, codes, scales, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), INVALID), (dict(codes=None), INVALID), (dict(scales=None), INVALID), (dict(rows=0), INVALID),
    (dict(cols=16), INVALID), (dict(cols=48), UNSUPPORTED), (dict(rows=1 << 20, cols=4096), INVALID),
    (dict(w=ODD), MISALIGNED), (dict(codes=B + 8), MISALIGNED), (dict(scales=B + 1), MISALIGNED),
])
def test_quantize_q8_0_rejects(lib, kw, status):
    assert q8(lib, **kw) == status


def lin_q8(lib, x=A, rows=16, k=1280, codes=B, scales=B + 65536, n=1280, bias=None, act=0, res=None, res_rows=0, y=A + 65536):
    return lib.edda_linear_q8(x, rows, k, codes, scales, n, bias, act, res, res_rows, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(codes=None), INVALID), (dict(scales=None), INVALID), (dict(y=None), INVALID),
    (dict(rows=0), INVALID), (dict(act=2), INVALID), (dict(res=A, res_rows=0), INVALID),
    (dict(rows=17), UNSUPPORTED), (dict(k=48), UNSUPPORTED), (dict(n=24), UNSUPPORTED),
    (dict(x=ODD), MISALIGNED), (dict(scales=B + 8), MISALIGNED), (dict(codes=B + 8), MISALIGNED),
])
def test_linear_q8_rejects(lib, kw, status):
    assert lin_q8(lib, **kw) == status


def test_decoder_layer_q8_rejects_missing_scales(lib):
    w = _lib.DecoderLayerWeightsQ8()
    for name, _ in w._fields_:
        if name.startswith("w_"):
            setattr(w, name, _lib.Q8Matrix(A, A + 4096))
        elif not name.startswith("b_"):
            setattr(w, name, A)
    slots = (ctypes.c_int32 * 1)(0)
    args = lambda: (A, 1, ctypes.cast(slots, ctypes.POINTER(ctypes.c_int32)), A, A, 64, 8, None, A, A, 1500,
                    ctypes.byref(w), A, B, 1 << 30, None)
    w.w_fc2 = _lib.Q8Matrix(A, None)
    assert lib.edda_decoder_verify_layer_q8(*args()) == INVALID
    w.w_fc2 = _lib.Q8Matrix(A, A + 8)
    assert lib.edda_decoder_verify_layer_q8(*args()) == MISALIGNED
    assert lib.edda_decoder_verify_layer_q8(A, 17, ctypes.cast(slots, ctypes.POINTER(ctypes.c_int32)), A, A, 64, 8,
                                            None, A, A, 1500, ctypes.byref(w), A, B, 1 << 30, None) == INVALID


def test_weight_structs_match_the_c_layout(tmp_path):
    """sizeof / offsetof of the header's weight structs, compiled with the host C compiler,
    equal the binding's ctypes layouts."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"edda_decoder_layer_weights": _lib.DecoderLayerWeights,
               "edda_decoder_layer_weights_q8": _lib.DecoderLayerWeightsQ8,
               "edda_q8_matrix": _lib.Q8Matrix}
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "edda.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in py._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {(l.split()[0], l.split()[1]): int(l.split()[2]) for l in out if l}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for field, _ in py._fields_:
            assert got[(cname, field)] == getattr(py, field).offset, (cname, field)


@pytest.mark.parametrize("args,status", [
    ((None, 16, A, A, 100, None, B, None), INVALID),
    ((A, 0, A, A, 100, None, B, None), INVALID),
    ((A, 17, A, A, 100, None, B, None), INVALID),
    ((A, 16, A, A, 0, None, B, None), INVALID),
    ((A, 16, A, A, 8193, None, B, None), UNSUPPORTED),   # beyond the static scratch
    ((A, 16, A, A, 1 << 30, None, B, None), UNSUPPORTED),
    ((ODD, 16, A, A, 100, None, B, None), MISALIGNED),
    ((A, 16, A, A, 100, A + 1, B, None), MISALIGNED),
])
def test_verify_noalloc_rejects(lib, args, status):
    assert lib.edda_verify_attn_noalloc(*args) == status
    if status == UNSUPPORTED:
        assert b"8192" in lib.edda_last_error()


def test_noalloc_limits_match_header():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (EDDA_\w+) (\d+)", text))
    assert int(consts["EDDA_NOALLOC_MAX_KV"]) == _lib.NOALLOC_MAX_KV
    # The scratch holds the counters and the partials of 16 queries x 20 heads x 64 splits.
    assert _lib.load().edda_verify_workspace_bytes(16, _lib.NOALLOC_MAX_KV) == 16384 + 64 * 16 * 20 * 66 * 4
