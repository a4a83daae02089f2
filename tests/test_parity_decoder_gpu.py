"""GPU parity of the decoder's verification layer (skinny GEMMs, cache append, self and cross
verification attention, MLP) and of the cross K/V projection against the fp64 oracle,
through the C ABI. Bar as for the encoder layer: |delta| <= 3e-3 + 1e-3 |ref| per element,
relative Frobenius <= 1e-3, all outputs finite; the appended cache rows are fp16 results of
the QKV projection (same bar) and every other cache slot must be bit-identical.
"""
import sys

import numpy as np
import pytest

import oracle.decoder_layer as DL
import oracle.encoder_layer as L
from whisper_asr_encoder_amd import _lib
from whisper_asr_encoder_amd import inputs as I

pytestmark = pytest.mark.gpu

ATOL, RTOL, REL_FRO = 3e-3, 1e-3, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    say(f"  {what}: max|d| {np.abs(got - ref).max():.3e}  worst excess {excess.max():.3e}  rel_fro {rel:.3e}")
    assert excess.max() <= 0, f"{what}: |delta| beyond 3e-3 + 1e-3|ref| by {excess.max():.3e}"
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e}"


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    return t


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.float().cpu().numpy()


# ---------------------------------------------------------------------------
# Block-sized GEMMs (M <= 16 rows take the skinny kernel).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,k,n,act,res", [
    (16, 1280, 3840, 0, False), (1, 1280, 1280, 0, True), (5, 1280, 5120, 1, False), (16, 5120, 1280, 0, True),
    (7, 64, 64, 1, True), (16, 1280, 2560, 0, False)])
def test_skinny_linear(torch, rows, k, n, act, res):
    say(f"skinny linear rows={rows} in={k} out={n} act={act} residual={res}")
    r = np.random.default_rng(rows * 3 + k + n)
    x = r.standard_normal((rows, k)).astype(np.float16)
    w = (r.standard_normal((k, n)) / np.sqrt(k)).astype(np.float16)
    b = (r.standard_normal(n) * 0.1).astype(np.float16)
    ref = L.linear(x, w, b)
    if act:
        ref = L.gelu(ref)
    residual = None
    if res:
        rr = r.standard_normal((rows, n)).astype(np.float16)
        residual = dev(torch, rr)
        ref = ref + rr.astype(np.float64)
    y = torch.full((rows, n), float("nan"), dtype=torch.float16, device="cuda")
    _lib.edda_linear(dev(torch, x), dev(torch, _lib.linear_layout(w)), dev(torch, b), y, activation=act,
                     residual=residual)
    torch.cuda.synchronize()
    check(host(y), ref, "y")


# ---------------------------------------------------------------------------
# Cross K/V and the decoder layer.
# ---------------------------------------------------------------------------

def test_cross_kv(torch):
    say("cross K/V of a 1500-frame encoder output")
    w = I.decoder_layer_weights(0)
    enc = I.encoder_workload(1, layers=1).x
    from whisper_asr_encoder_amd.encoder import DecoderVerifier
    dv = DecoderVerifier([w], max_kv=64)
    dv.set_encoder_output(dev(torch, enc))
    torch.cuda.synchronize()
    k, v = DL.cross_kv(enc, w.w_ck, w.w_cv, w.b_cv)
    check(host(dv.cross_k[0]), k, "cross K")
    check(host(dv.cross_v[0]), v, "cross V")


def run_layer(torch, layer, trial, kind, n_kv=None, in_place=False):
    """One decoder layer on GPU and oracle; kind = 'causal' (chain of 16) or 'tree' (5 beams)."""
    from whisper_asr_encoder_amd.encoder import DecoderVerifier
    w = I.decoder_layer_weights(layer)
    if kind == "causal":
        case = I.verify_self_case(trial, layer, n_kv=n_kv)
        n_q, nk = 16, case.n_kv
        slots = list(range(nk - n_q, nk))
    else:
        case = I.verify_tree_case(trial, layer, n_kv=n_kv)
        n_q, nk = case.q.shape[0], case.n_kv
        slots = [int(s) for s in case.query_slots]
    cap = nk + 8
    r = np.random.default_rng(1000 + layer)
    kc = np.zeros((cap, 20, 64), dtype=np.float16)
    vc = np.zeros((cap, 20, 64), dtype=np.float16)
    kc[:nk], vc[:nk] = case.k, case.v
    kc[nk:] = r.standard_normal((cap - nk, 20, 64)).astype(np.float16)   # beyond n_kv: must stay
    x = I.decoder_block_input(trial, n_q)
    enc = I.encoder_workload(1, layers=1).x
    dv = DecoderVerifier([w], max_kv=cap)
    dv.set_encoder_output(dev(torch, enc))
    ck, cv = DL.cross_kv(enc, w.w_ck, w.w_cv, w.b_cv)
    ck16, cv16 = host(dv.cross_k[0]).astype(np.float16), host(dv.cross_v[0]).astype(np.float16)
    k_d, v_d = dev(torch, kc), dev(torch, vc)
    xd = dev(torch, x)
    y = xd if in_place else torch.full((n_q, 1280), float("nan"), dtype=torch.float16, device="cuda")
    mask = case.mask
    dv.layer(xd, 0, slots, k_d, v_d, nk, None if mask is None else VerifyRows(torch, mask), y)
    torch.cuda.synchronize()
    # The oracle reads the GPU's own cross K/V (fp16, checked separately above).
    ref = DL.decoder_verify_layer(x, w, slots, kc, vc, nk, mask, ck16, cv16)
    assert not dv.workspace[:_lib.VERIFY_COUNTER_BYTES].any().item(), "arrival counters not returned to zero"
    return host(y), host(k_d), host(v_d), ref, kc, vc, slots


def VerifyRows(torch, mask):
    return torch.from_numpy(_lib.pack_mask_rows(mask).view(np.int32)).cuda()


@pytest.mark.parametrize("trial,layer,kind", [(0, 0, "causal"), (3, 31, "causal"), (1, 5, "tree"), (6, 17, "tree")])
def test_decoder_layer(torch, trial, layer, kind):
    say(f"decoder verification layer trial {trial} layer {layer} {kind}")
    y, kd, vd, ref, kc, vc, slots = run_layer(torch, layer, trial, kind)
    check(y, ref["y"], "y")
    others = np.setdiff1d(np.arange(kc.shape[0]), slots)
    assert np.array_equal(kd[others], kc[others].astype(np.float32)), "cache rows outside the block changed"
    assert np.array_equal(vd[others], vc[others].astype(np.float32)), "cache rows outside the block changed"
    check(kd[slots], ref["k_cache"][slots], "appended K rows")
    check(vd[slots], ref["v_cache"][slots], "appended V rows")


def test_decoder_layer_short_cache_in_place(torch):
    say("decoder layer: cache of 16 slots (the block alone), y = x in place")
    y, _, _, ref, _, _, _ = run_layer(torch, 2, 4, "causal", n_kv=16, in_place=True)
    check(y, ref["y"], "y")
