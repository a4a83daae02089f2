"""GPU parity of the Q8_0 decoder weights against the oracle in oracle/quant.py, through the
C ABI: the quantizer's codes and scales bit for bit (integers decided in fp32 on both sides),
edda_linear_q8 and the Q8 decoder layer to the layer bar (|delta| <= 3e-3 + 1e-3 |ref|,
relative Frobenius <= 1e-3) against the oracle on its own dequantized weights. The distance
between the Q8 and the fp16 decoder layer is printed (and loosely bounded): it is the
quantization of the weights, not an error of the kernels.
"""
import sys

import numpy as np
import pytest

import oracle.decoder_layer as DL
import oracle.encoder_layer as L
import oracle.quant as Q
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


def gpu_quantize(torch, w_out_in):
    w = dev(torch, w_out_in)
    n, k = w.shape
    codes = torch.full((n, k), 99, dtype=torch.int8, device="cuda")
    scales = torch.full((k // 32, n), float("nan"), dtype=torch.float16, device="cuda")
    _lib.edda_quantize_q8_0(w, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def weights_with_edges(seed, n, k):
    """N(0, 1/k) weights with per-row magnitudes over four decades, some all-zero blocks, and
    blocks whose codes fall on exact ties (amax 127/8, values (j + 1/2)/8)."""
    r = np.random.default_rng(seed)
    w = r.standard_normal((n, k)) / np.sqrt(k) * 10.0 ** r.uniform(-2, 2, (n, 1))
    tie = np.zeros(32)
    tie[0] = 127 / 8
    tie[1:] = (np.arange(31) - 15 + 0.5) / 8
    w[3 % n, (64 % k):(64 % k) + 32] = 0
    w[7 % n, :32] = 0
    w[11 % n, (32 % k):(32 % k) + 32] = tie
    w[12 % n, 0:32] = -tie
    return w.astype(np.float16)


@pytest.mark.parametrize("n,k", [(3840, 1280), (1280, 5120), (16, 32), (48, 96)])
def test_quantizer_bit_exact(torch, n, k):
    say(f"Q8_0 quantizer [{n}, {k}]")
    w = weights_with_edges(n + k, n, k)
    codes, scales = gpu_quantize(torch, w)
    q_ref, d_ref = Q.quantize_q8_0(w)
    assert np.array_equal(codes.cpu().numpy(), q_ref), "codes differ"
    got_d = scales.cpu().numpy().T
    assert np.array_equal(got_d.view(np.uint16), d_ref.view(np.uint16)), "scales differ"


@pytest.mark.parametrize("rows,k,n,act,res", [
    (16, 1280, 3840, 0, False), (1, 1280, 1280, 0, True), (5, 1280, 5120, 1, False), (16, 5120, 1280, 0, True),
    (7, 64, 32, 1, True), (16, 1280, 1280, 0, False)])
def test_linear_q8(torch, rows, k, n, act, res):
    say(f"linear_q8 rows={rows} in={k} out={n} act={act} residual={res}")
    r = np.random.default_rng(rows * 5 + k + n)
    x = r.standard_normal((rows, k)).astype(np.float16)
    w = (r.standard_normal((n, k)) / np.sqrt(k)).astype(np.float16)   # [out, in]
    b = (r.standard_normal(n) * 0.1).astype(np.float16)
    q_ref, d_ref = Q.quantize_q8_0(w)
    ref = Q.linear_q8(x, q_ref, d_ref, b)
    if act:
        ref = L.gelu(ref)
    residual = None
    if res:
        rr = r.standard_normal((rows, n)).astype(np.float16)
        residual = dev(torch, rr)
        ref = ref + rr.astype(np.float64)
    codes, scales = gpu_quantize(torch, w)
    y = torch.full((rows, n), float("nan"), dtype=torch.float16, device="cuda")
    _lib.edda_linear_q8(dev(torch, x), codes, scales, dev(torch, b), y, activation=act, residual=residual)
    torch.cuda.synchronize()
    check(y.float().cpu().numpy(), ref, "y")


def run_layer(torch, layer, trial, kind, q8, frames=1500, n_kv=None):
    from whisper_asr_encoder_amd.encoder import DecoderVerifier
    w = I.decoder_layer_weights(layer)
    case = (I.verify_self_case(trial, layer, n_kv=n_kv) if kind == "causal"
            else I.verify_tree_case(trial, layer, n_kv=n_kv))
    n_q, nk = case.q.shape[0], case.n_kv
    slots = list(range(nk - n_q, nk)) if kind == "causal" else [int(s) for s in case.query_slots]
    cap = nk + 8
    kc = np.zeros((cap, 20, 64), dtype=np.float16)
    vc = np.zeros((cap, 20, 64), dtype=np.float16)
    kc[:nk], vc[:nk] = case.k, case.v
    x = I.decoder_block_input(trial, n_q)
    dv = DecoderVerifier([w], max_kv=cap, q8=q8, n_frames=frames)
    # Cross K/V from the oracle, rounded once to fp16 on the host, feed both sides.
    enc = np.ascontiguousarray(I.encoder_workload(1, layers=1).x[:frames])
    ck, cv = DL.cross_kv(enc, w.w_ck, w.w_cv, w.b_cv)
    ck16, cv16 = ck.astype(np.float16), cv.astype(np.float16)
    dv.cross_k[0].copy_(dev(torch, ck16))
    dv.cross_v[0].copy_(dev(torch, cv16))
    k_d, v_d = dev(torch, kc), dev(torch, vc)
    y = torch.full((n_q, 1280), float("nan"), dtype=torch.float16, device="cuda")
    mask = None if case.mask is None else torch.from_numpy(_lib.pack_mask_rows(case.mask).view(np.int32)).cuda()
    dv.layer(dev(torch, x), 0, slots, k_d, v_d, nk, mask, y)
    torch.cuda.synchronize()
    return w, x, slots, kc, vc, nk, case.mask, ck16, cv16, y.float().cpu().numpy(), k_d.float().cpu().numpy()


@pytest.mark.parametrize("trial,layer,kind,frames,n_kv", [(0, 0, "causal", 1500, None), (3, 31, "causal", 1500, None),
                                                         (1, 5, "tree", 1500, None), (2, 11, "causal", 300, None),
                                                         (4, 2, "causal", 1500, 600)])
def test_decoder_layer_q8(torch, trial, layer, kind, frames, n_kv):
    """Caches up to 512 keys take the single-launch layer, a 600-key cache the eight launches."""
    say(f"Q8 decoder verification layer trial {trial} layer {layer} {kind}, {frames} frames, n_kv {n_kv}")
    w, x, slots, kc, vc, nk, mask, ck16, cv16, y, kd = run_layer(torch, layer, trial, kind, q8=True, frames=frames,
                                                                 n_kv=n_kv)
    wq = Q.DequantizedDecoderWeights(w, Q.quantize_decoder_weights(w))
    ref = DL.decoder_verify_layer(x, wq, slots, kc, vc, nk, mask, ck16, cv16)
    check(y, ref["y"], "y")
    check(kd[slots], ref["k_cache"][slots], "appended K rows")
    y16 = run_layer(torch, layer, trial, kind, q8=False, frames=frames, n_kv=n_kv)[9]
    rel = np.linalg.norm(y - y16) / np.linalg.norm(y16)
    say(f"  Q8 vs fp16 weights: y relative Frobenius distance {rel:.3e} (weight quantization)")
    assert rel < 2e-2


def test_decoder_stack_q8_matches_layer_by_layer(torch):
    """edda_decoder_verify_stack_q8 over 9 layers (two launches) against the Q8 layer entry point
    layer by layer: y and every cache bit for bit (the per-layer form is held to the oracle above)."""
    from whisper_asr_encoder_amd.encoder import DecoderVerifier
    say("Q8 decoder stack of 9 layers vs layer by layer")
    n_layers = 9
    weights = [I.decoder_layer_weights(l) for l in range(n_layers)]
    cases = [I.verify_tree_case(2, l) for l in range(n_layers)]
    n_q, nk = cases[0].q.shape[0], cases[0].n_kv
    slots = [int(s) for s in cases[0].query_slots]
    cap = nk + 4
    dv = DecoderVerifier(weights, max_kv=cap, q8=True)
    dv.set_encoder_output(dev(torch, I.encoder_workload(1, layers=1).x))
    host = []
    for c in cases:
        kc = np.zeros((cap, 20, 64), dtype=np.float16)
        vc = np.zeros((cap, 20, 64), dtype=np.float16)
        kc[:nk], vc[:nk] = c.k, c.v
        host.append((kc, vc))
    mask = torch.from_numpy(_lib.pack_mask_rows(cases[0].mask).view(np.int32)).cuda()
    x0 = I.decoder_block_input(2, n_q)
    ca = [(dev(torch, k), dev(torch, v)) for k, v in host]
    ya = torch.empty((n_q, 1280), dtype=torch.float16, device="cuda")
    cur = dev(torch, x0)
    for l in range(n_layers):
        dv.layer(cur, l, slots, ca[l][0], ca[l][1], nk, mask, ya)
        cur = ya
    cb = [(dev(torch, k), dev(torch, v)) for k, v in host]
    yb = torch.full((n_q, 1280), float("nan"), dtype=torch.float16, device="cuda")
    dv.stack(dev(torch, x0), slots, cb, nk, mask, yb)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb), "Q8 stack output differs from layer-by-layer"
    for l in range(n_layers):
        assert torch.equal(ca[l][0], cb[l][0]) and torch.equal(ca[l][1], cb[l][1]), f"layer {l} caches differ"
    assert not dv.stack_workspace[:_lib.DECODER_STACK_ZERO_BYTES].any().item()
