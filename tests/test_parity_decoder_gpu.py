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


def run_layer(torch, layer, trial, kind, n_kv=None, in_place=False, frames=1500, no_mask=False):
    """One decoder layer on GPU and oracle; kind = 'causal' (chain of 16), 'tree' (5 beams) or
    'single' (one token: a plain decoding step); `frames` rows of the encoder output feed the
    cross-attention; no_mask: the self-attention admits every slot (mask_rows NULL)."""
    from whisper_asr_encoder_amd.encoder import DecoderVerifier
    w = I.decoder_layer_weights(layer)
    if kind == "single":
        case = I.verify_self_case(trial, layer, n_kv=n_kv, n_q=1)
        n_q, nk = 1, case.n_kv
        slots = [nk - 1]
    elif kind == "causal":
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
    enc = np.ascontiguousarray(I.encoder_workload(1, layers=1).x[:frames])
    dv = DecoderVerifier([w], max_kv=cap, n_frames=frames)
    # The oracle's own cross K/V, rounded once to fp16 on the host, feed both sides (the
    # projection on the device, edda_cross_kv, is checked on its own in test_cross_kv).
    ck, cv = DL.cross_kv(enc, w.w_ck, w.w_cv, w.b_cv)
    ck16, cv16 = ck.astype(np.float16), cv.astype(np.float16)
    dv.cross_k[0].copy_(dev(torch, ck16))
    dv.cross_v[0].copy_(dev(torch, cv16))
    k_d, v_d = dev(torch, kc), dev(torch, vc)
    xd = dev(torch, x)
    y = xd if in_place else torch.full((n_q, 1280), float("nan"), dtype=torch.float16, device="cuda")
    mask = None if no_mask else case.mask
    dv.layer(xd, 0, slots, k_d, v_d, nk, None if mask is None else VerifyRows(torch, mask), y)
    torch.cuda.synchronize()
    ref = DL.decoder_verify_layer(x, w, slots, kc, vc, nk, mask, ck16, cv16)
    assert not dv.workspace[:_lib.VERIFY_COUNTER_BYTES].any().item(), "arrival counters not returned to zero"
    return host(y), host(k_d), host(v_d), ref, kc, vc, slots


def VerifyRows(torch, mask):
    return torch.from_numpy(_lib.pack_mask_rows(mask).view(np.int32)).cuda()


@pytest.mark.parametrize("trial,layer,kind", [(0, 0, "causal"), (3, 31, "causal"), (1, 5, "tree"), (6, 17, "tree"),
                                             (4, 12, "single")])
def test_decoder_layer(torch, trial, layer, kind):
    say(f"decoder verification layer trial {trial} layer {layer} {kind}")
    y, kd, vd, ref, kc, vc, slots = run_layer(torch, layer, trial, kind)
    check(y, ref["y"], "y")
    others = np.setdiff1d(np.arange(kc.shape[0]), slots)
    assert np.array_equal(kd[others], kc[others].astype(np.float32)), "cache rows outside the block changed"
    assert np.array_equal(vd[others], vc[others].astype(np.float32)), "cache rows outside the block changed"
    check(kd[slots], ref["k_cache"][slots], "appended K rows")
    check(vd[slots], ref["v_cache"][slots], "appended V rows")


@pytest.mark.parametrize("frames", [300, 100])
def test_decoder_layer_short_encoder_output(torch, frames):
    """Cross-attention over fewer frames: one workgroup per head (the 1500-frame layers split
    the frames over twelve workgroups per head)."""
    say(f"decoder layer: {frames} encoder frames")
    y, kd, _, ref, _, _, slots = run_layer(torch, 7, 5, "causal", frames=frames)
    check(y, ref["y"], "y")
    check(kd[slots], ref["k_cache"][slots], "appended K rows")


@pytest.mark.parametrize("n_kv,kind,no_mask", [(256, "causal", False), (257, "tree", False), (512, "causal", False),
                                              (300, "causal", True), (40, "single", False), (513, "causal", False),
                                              (700, "tree", False)])
def test_decoder_layer_cache_lengths(torch, n_kv, kind, no_mask):
    """Caches at the chunk boundaries of the single-launch layer's self-attention (one 32-key
    chunk per wave up to 256 keys, two up to 512), an unmasked self-attention, and caches
    beyond 512 keys, which take the eight-launch form of the layer."""
    say(f"decoder layer: n_kv {n_kv} {kind}{' no mask' if no_mask else ''}")
    y, kd, vd, ref, kc, vc, slots = run_layer(torch, 11, 2, kind, n_kv=n_kv, no_mask=no_mask)
    check(y, ref["y"], "y")
    others = np.setdiff1d(np.arange(kc.shape[0]), slots)
    assert np.array_equal(kd[others], kc[others].astype(np.float32)), "cache rows outside the block changed"
    check(kd[slots], ref["k_cache"][slots], "appended K rows")
    check(vd[slots], ref["v_cache"][slots], "appended V rows")


def test_decoder_layer_repeatable_and_graph_replay(torch):
    """The layer's result does not depend on which workgroup takes which work item: two eager
    calls on fresh copies of the caches, and three replays of a captured graph (with eager work
    between them), all bit-identical; the counters are zero after each."""
    from whisper_asr_encoder_amd.encoder import DecoderVerifier
    say("decoder layer: repeat and graph replay")
    w = I.decoder_layer_weights(6)
    case = I.verify_tree_case(3, 6)
    n_q, nk = case.q.shape[0], case.n_kv
    slots = [int(s) for s in case.query_slots]
    cap = nk + 4
    kc = np.zeros((cap, 20, 64), dtype=np.float16)
    vc = np.zeros((cap, 20, 64), dtype=np.float16)
    kc[:nk], vc[:nk] = case.k, case.v
    dv = DecoderVerifier([w], max_kv=cap)
    dv.set_encoder_output(dev(torch, I.encoder_workload(1, layers=1).x))
    x = dev(torch, I.decoder_block_input(3, n_q))
    mask = VerifyRows(torch, case.mask)
    outs = []
    for _ in range(2):
        k_d, v_d = dev(torch, kc), dev(torch, vc)
        y = torch.full((n_q, 1280), float("nan"), dtype=torch.float16, device="cuda")
        dv.layer(x, 0, slots, k_d, v_d, nk, mask, y)
        torch.cuda.synchronize()
        assert not dv.workspace[:_lib.VERIFY_COUNTER_BYTES].any().item(), "counters not returned to zero"
        outs.append((y.clone(), k_d.clone(), v_d.clone()))
    assert all(torch.equal(a, b) for a, b in zip(*outs)), "two eager calls differ"
    k_g, v_g = dev(torch, kc), dev(torch, vc)
    y_g = torch.full((n_q, 1280), float("nan"), dtype=torch.float16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dv.layer(x, 0, slots, k_g, v_g, nk, mask, y_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dv.layer(x, 0, slots, k_g, v_g, nk, mask, y_g)
    for i in range(3):
        y_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, outs[0][0]), f"graph replay {i} differs from the eager result"
        assert torch.equal(k_g, outs[0][1]) and torch.equal(v_g, outs[0][2]), f"replay {i}: caches differ"
        assert not dv.workspace[:_lib.VERIFY_COUNTER_BYTES].any().item(), "counters not returned to zero"
        torch.mul(x, 1.0)  # eager work between replays


def test_decoder_layer_short_cache_in_place(torch):
    say("decoder layer: cache of 16 slots (the block alone), y = x in place")
    y, _, _, ref, _, _, _ = run_layer(torch, 2, 4, "causal", n_kv=16, in_place=True)
    check(y, ref["y"], "y")


@pytest.mark.parametrize("trial,layer,kind", [(0, 3, "causal"), (2, 9, "tree")])
def test_decoder_layer_matches_composition_of_public_entries(torch, trial, layer, kind):
    """The layer's fused launches (LayerNorm inside the block GEMMs, the cache append in the
    QKV epilogue, split K for the 1280-wide outputs) against the public entry points step by
    step (edda_layer_norm, edda_linear, edda_verify_attn, the append done by indexing): the
    cache rows bit for bit (LayerNorm and QKV arithmetic are the same code), y to the layer
    bar (split K groups the fp32 sums differently)."""
    from whisper_asr_encoder_amd.encoder import DecoderVerifier, VerifyAttention
    say(f"decoder layer vs composed public entries: trial {trial} layer {layer} {kind}")
    w = I.decoder_layer_weights(layer)
    case = I.verify_self_case(trial, layer) if kind == "causal" else I.verify_tree_case(trial, layer)
    n_q, nk = case.q.shape[0], case.n_kv
    slots = list(range(nk - n_q, nk)) if kind == "causal" else [int(s) for s in case.query_slots]
    cap = nk + 4
    kc = np.zeros((cap, 20, 64), dtype=np.float16)
    vc = np.zeros((cap, 20, 64), dtype=np.float16)
    kc[:nk], vc[:nk] = case.k, case.v
    x = dev(torch, I.decoder_block_input(trial, n_q))
    dv = DecoderVerifier([w], max_kv=cap)
    dv.set_encoder_output(dev(torch, I.encoder_workload(1, layers=1).x))
    mask = None if case.mask is None else VerifyRows(torch, case.mask)
    # Fused layer.
    k_f, v_f = dev(torch, kc), dev(torch, vc)
    y_f = torch.empty((n_q, 1280), dtype=torch.float16, device="cuda")
    dv.layer(x, 0, slots, k_f, v_f, nk, mask, y_f)
    # The same layer from public entry points.
    t = dv._keep[0]
    k_c, v_c = dev(torch, kc), dev(torch, vc)
    va = VerifyAttention(max(cap, 1500))
    e = lambda *shape: torch.empty(shape, dtype=torch.float16, device="cuda")
    h1, qkv = e(n_q, 1280), e(n_q, 3840)
    _lib.edda_layer_norm(x, t["ln1_gamma"], t["ln1_beta"], h1)
    _lib.edda_linear(h1, t["w_qkv"], t["b_qkv"], qkv)
    idx = torch.tensor(slots, device="cuda")
    k_c.view(cap, 1280)[idx] = qkv[:, 1280:2560]
    v_c.view(cap, 1280)[idx] = qkv[:, 2560:]
    o = e(n_q, 20, 64)
    va(qkv[:, :1280].contiguous().view(n_q, 20, 64), k_c[:nk], v_c[:nk], mask, o)
    x1, h2, qc, oc, x2, h3, f, y_c = (e(n_q, 1280), e(n_q, 1280), e(n_q, 1280), e(n_q, 20, 64), e(n_q, 1280),
                                      e(n_q, 1280), e(n_q, 5120), e(n_q, 1280))
    _lib.edda_linear(o.view(n_q, 1280), t["w_o"], t["b_o"], x1, residual=x)
    _lib.edda_layer_norm(x1, t["ln2_gamma"], t["ln2_beta"], h2)
    _lib.edda_linear(h2, t["w_q_cross"], t["b_q_cross"], qc)
    va(qc.view(n_q, 20, 64), dv.cross_k[0], dv.cross_v[0], None, oc)
    _lib.edda_linear(oc.view(n_q, 1280), t["w_o_cross"], t["b_o_cross"], x2, residual=x1)
    _lib.edda_layer_norm(x2, t["ln3_gamma"], t["ln3_beta"], h3)
    _lib.edda_linear(h3, t["w_fc1"], t["b_fc1"], f, activation=_lib.ACT_GELU)
    _lib.edda_linear(f, t["w_fc2"], t["b_fc2"], y_c, residual=x2)
    torch.cuda.synchronize()
    assert torch.equal(k_f, k_c) and torch.equal(v_f, v_c), "cache contents differ"
    check(host(y_f), host(y_c).astype(np.float64), "y, fused vs composed")


@pytest.mark.parametrize("n_layers,kind,in_place", [(4, "causal", False), (10, "tree", True)])
def test_decoder_stack_matches_layer_by_layer(torch, n_layers, kind, in_place):
    """edda_decoder_verify_stack (several layers per launch: 4 in one launch, 10 in two) against
    edda_decoder_verify_layer called layer by layer: y and every layer's caches bit for bit.
    The per-layer entry point is held to the oracle by the tests above; the first layers of the
    stack are also checked against the oracle chain here."""
    from whisper_asr_encoder_amd.encoder import DecoderVerifier
    say(f"decoder stack of {n_layers} layers ({kind}{', y = x' if in_place else ''}) vs layer by layer")
    weights = [I.decoder_layer_weights(l) for l in range(n_layers)]
    cases = [I.verify_self_case(1, l) if kind == "causal" else I.verify_tree_case(1, l) for l in range(n_layers)]
    n_q, nk = cases[0].q.shape[0], cases[0].n_kv
    slots = list(range(nk - n_q, nk)) if kind == "causal" else [int(s) for s in cases[0].query_slots]
    cap = nk + 4
    dv = DecoderVerifier(weights, max_kv=cap)
    enc = I.encoder_workload(1, layers=1).x
    cross = [DL.cross_kv(enc, w.w_ck, w.w_cv, w.b_cv) for w in weights[:2]]
    dv.set_encoder_output(dev(torch, enc))
    for l in range(2):  # the oracle's own cross K/V (fp16) for the layers checked against it
        dv.cross_k[l].copy_(dev(torch, cross[l][0].astype(np.float16)))
        dv.cross_v[l].copy_(dev(torch, cross[l][1].astype(np.float16)))
    host_caches = []
    for c in cases:
        kc = np.zeros((cap, 20, 64), dtype=np.float16)
        vc = np.zeros((cap, 20, 64), dtype=np.float16)
        kc[:nk], vc[:nk] = c.k, c.v
        host_caches.append((kc, vc))
    mask = VerifyRows(torch, cases[0].mask)
    x0 = I.decoder_block_input(1, n_q)
    # Layer by layer.
    caches_a = [(dev(torch, k), dev(torch, v)) for k, v in host_caches]
    xa = dev(torch, x0)
    ya = torch.empty_like(xa)
    cur = xa
    for l in range(n_layers):
        dv.layer(cur, l, slots, caches_a[l][0], caches_a[l][1], nk, mask, ya)
        cur = ya
    # The stack.
    caches_b = [(dev(torch, k), dev(torch, v)) for k, v in host_caches]
    xb = dev(torch, x0)
    yb = xb if in_place else torch.full_like(xb, float("nan"))
    dv.stack(xb, slots, caches_b, nk, mask, yb)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb), "stack output differs from layer-by-layer"
    for l in range(n_layers):
        assert torch.equal(caches_a[l][0], caches_b[l][0]) and torch.equal(caches_a[l][1], caches_b[l][1]), \
            f"layer {l} caches differ"
    assert not dv.stack_workspace[:_lib.DECODER_STACK_ZERO_BYTES].any().item(), "counters or flags not cleared"
    # The first two layers of the stack against the oracle chain.
    dv2 = DecoderVerifier(weights[:2], max_kv=cap)
    for l in range(2):
        dv2.cross_k[l].copy_(dv.cross_k[l])
        dv2.cross_v[l].copy_(dv.cross_v[l])
    caches_c = [(dev(torch, k), dev(torch, v)) for k, v in host_caches[:2]]
    yc = torch.empty_like(xb)
    dv2.stack(dev(torch, x0), slots, caches_c, nk, mask, yc)
    torch.cuda.synchronize()
    ref_x = x0
    for l in range(2):
        kc, vc = host_caches[l]
        ck, cv = cross[l]
        ref = DL.decoder_verify_layer(ref_x, weights[l], slots, kc, vc, nk, cases[0].mask, ck.astype(np.float16),
                                      cv.astype(np.float16))
        ref_x = ref["y"]
    check(host(yc), ref_x, "y after two layers")
