"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs. Bar: max |delta| <= 3e-3 and relative Frobenius error
<= 1e-3 on every compared output, all outputs finite.

Small cases compare every element; full-size workloads (the launch
configuration the benchmark times) compare whole layers or sampled windows and
rows that the oracle computes one by one.
"""
import sys

import numpy as np
import pytest

import oracle
from whisper_asr_encoder_amd import _lib
from whisper_asr_encoder_amd import inputs as I

pytestmark = pytest.mark.gpu

ATOL = 3e-3
REL_FRO = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(got, ref, what, atol=ATOL, rel_fro=REL_FRO):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    diff = np.abs(got - ref)
    mx = float(diff.max()) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    fro = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got - ref))
    say(f"  {what}: max|d| = {mx:.3e}, rel_fro = {fro:.3e}")
    assert mx <= atol, f"{what}: max |delta| {mx:.3e} > {atol}"
    assert fro <= rel_fro, f"{what}: relative Frobenius {fro:.3e} > {rel_fro}"


@pytest.fixture(scope="module")
def torch():
    import torch
    from whisper_asr_encoder_amd import _lib
    _lib.load()
    return torch


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.float().cpu().numpy()


def run_encoder(torch, x, weights, batch, seq_len, chunk_len, valid_len, poison=True, keep=None):
    """Run every sublayer through the C ABI; return host copies of y (and qkv) for the
    layers in `keep` (default all). Every layer's output is checked finite on the device."""
    from whisper_asr_encoder_amd.encoder import EncoderAttention
    enc = EncoderAttention(weights, batch, seq_len, chunk_len, valid_len)
    keep = set(range(len(weights))) if keep is None else set(keep)
    xd = dev(torch, x)
    y = torch.empty((batch * seq_len, I.D_MODEL), dtype=torch.float16, device="cuda")
    ys, qkvs = {}, {}
    for layer in range(len(weights)):
        y.fill_(float("nan") if poison else 0.0)
        enc.qkv.fill_(float("nan"))
        enc.workspace.fill_(255)
        enc.sublayer(xd, layer, y)
        assert bool(torch.isfinite(y).all()), f"layer {layer}: non-finite output"
        if layer in keep:
            ys[layer] = host(y)
            qkvs[layer] = host(enc.qkv)
    torch.cuda.synchronize()
    return ys, qkvs


def oracle_layer(x, w, batch, seq_len, chunk_len, valid_len, rows=None):
    return oracle.encoder_attention(x, w.w_qkv, w.b_qkv, w.w_o, w.b_o, batch, seq_len, chunk_len,
                                    valid_len, I.N_HEADS, rows=rows)


# ---------------------------------------------------------------------------
# Encoder: small cases, every element.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("batch,seq_len,chunk_len,valid", [
    (1, 200, 0, None),          # one 4 s chunk (the small workload)
    (1, 1, 0, None),            # a single frame
    (1, 37, 0, None),           # ragged: shorter than every tile
    (1, 300, 0, [129]),         # key tail cut mid-tile
    (2, 150, 0, [1, 150]),      # one key only / full
    (1, 450, 200, None),        # chunks 200, 200, 50
    (1, 450, 200, [260]),       # last chunk fully padded -> zero rows
    (1, 130, 1, None),          # chunk of one frame: O = V row
    (1, 200, 65, [199]),        # chunk just above a key tile
    (3, 96, 32, [96, 40, 33]),  # several windows, chunked and padded
    # More windows than one launch takes (256): the second launch's windows and their valid
    # lengths are indexed from its first window.
    (300, 8, 0, [1 + b % 8 for b in range(300)]),
    (260, 24, 8, [24 - b % 24 for b in range(260)]),
])
def test_encoder_small(torch, batch, seq_len, chunk_len, valid):
    say(f"encoder small batch={batch} seq={seq_len} chunk={chunk_len} valid={valid if batch <= 16 else '...'}")
    wl = I.encoder_workload(0, batch=batch, seq_len=seq_len, chunk_len=chunk_len, layers=1, valid_len=valid)
    w = wl.weights(0)
    ys, qkvs = run_encoder(torch, wl.x, [w], batch, seq_len, chunk_len, wl.valid_len)
    ref = oracle_layer(wl.x, w, batch, seq_len, chunk_len, wl.valid_len)
    check(qkvs[0], ref["qkv"], "qkv")
    check(ys[0], ref["y"], "y")


def test_encoder_bias_variants(torch):
    say("encoder with output bias and without QKV bias")
    wl = I.encoder_workload(0, seq_len=77, layers=1)
    w = wl.weights(0)
    r = np.random.default_rng(7)
    w.b_o = (r.standard_normal(I.D_MODEL) * 0.1).astype(np.float16)
    ys, _ = run_encoder(torch, wl.x, [w], 1, 77, 0, None)
    check(ys[0], oracle_layer(wl.x, w, 1, 77, 0, [77])["y"], "y with b_o")
    w.b_qkv = None
    w.b_o = None
    ys, qkvs = run_encoder(torch, wl.x, [w], 1, 77, 0, None)
    ref = oracle_layer(wl.x, w, 1, 77, 0, [77])
    check(qkvs[0], ref["qkv"], "qkv without bias")
    check(ys[0], ref["y"], "y without bias")


def test_encoder_deterministic(torch):
    say("encoder determinism")
    wl = I.encoder_workload(1, layers=1)
    w = wl.weights(0)
    a, _ = run_encoder(torch, wl.x, [w], 1, 1500, 0, None)
    b, _ = run_encoder(torch, wl.x, [w], 1, 1500, 0, None, poison=False)
    assert np.array_equal(a[0], b[0])


# ---------------------------------------------------------------------------
# Encoder: the full-size workloads (32 sublayers, as timed).
# ---------------------------------------------------------------------------

def test_config_small_chunk(torch):
    say("workload: one 4 s chunk, one sublayer")
    wl = I.encoder_workload(0)
    w = wl.weights(0)
    ys, qkvs = run_encoder(torch, wl.x, [w], 1, 200, 0, None)
    ref = oracle_layer(wl.x, w, 1, 200, 0, [200])
    check(qkvs[0], ref["qkv"], "qkv")
    check(ys[0], ref["y"], "y")


def test_config_30s_window(torch):
    say("workload: 30 s window, 32 sublayers (layers 0, 13, 31 compared in full)")
    wl = I.encoder_workload(1)
    weights = [wl.weights(l) for l in range(wl.layers)]
    ys, qkvs = run_encoder(torch, wl.x, weights, 1, 1500, 0, None, keep=(0, 13, 31))
    for l in (0, 13, 31):
        ref = oracle_layer(wl.x, weights[l], 1, 1500, 0, [1500])
        check(qkvs[l], ref["qkv"], f"layer {l} qkv")
        check(ys[l], ref["y"], f"layer {l} y")


def test_config_chunked_45s(torch):
    say("workload: 45 s in 4 s chunks, 32 sublayers (layers 0, 31 in full)")
    wl = I.encoder_workload(2)
    weights = [wl.weights(l) for l in range(wl.layers)]
    ys, _ = run_encoder(torch, wl.x, weights, 1, wl.seq_len, wl.chunk_len, wl.valid_len, keep=(0, 31))
    for l in (0, 31):
        ref = oracle_layer(wl.x, weights[l], 1, wl.seq_len, wl.chunk_len, wl.valid_len)
        check(ys[l], ref["y"], f"layer {l} y")


def test_config_batched_windows(torch):
    """All 16 windows at layer 0 (each with its own drawn valid length, so its own masked tail
    tile), rows around every valid length; layers 17 and 31 on a spread of windows."""
    say("workload: 16 windows with padded key tails, 32 sublayers (sampled rows of every window)")
    wl = I.encoder_workload(3)
    weights = [wl.weights(l) for l in range(wl.layers)]
    ys, _ = run_encoder(torch, wl.x, weights, wl.batch, wl.seq_len, 0, wl.valid_len, keep=(0, 17, 31))
    order = np.argsort(wl.valid_len)
    rng = np.random.default_rng(11)
    S = wl.seq_len
    plan = ((0, list(range(wl.batch))),
            (17, [int(order[0]), int(order[5]), int(order[10]), int(order[-1])]),
            (31, [int(order[2]), int(order[8]), int(order[13])]))
    for l, wins in plan:
        for b in wins:
            v = int(wl.valid_len[b])
            near = [r for r in range(v - 3, v + 3) if 0 <= r < S]  # both sides of the valid length
            tile = [r for r in (128 * (v // 128), 128 * (v // 128) + 127) if r < S]  # its query tile
            local = np.unique(np.concatenate([rng.choice(S, size=48, replace=False), [0, S - 1], near, tile]))
            rows = b * S + local
            ref = oracle_layer(wl.x, weights[l], wl.batch, S, 0, wl.valid_len, rows=rows)
            check(ys[l][rows], ref["y"], f"layer {l} window {b} (valid {v}) y")


# ---------------------------------------------------------------------------
# Verification attention.
# ---------------------------------------------------------------------------

def run_verify(torch, case, mask=None, use_mask=True):
    from whisper_asr_encoder_amd.encoder import VerifyAttention
    va = VerifyAttention(max(case.n_kv, 1))
    m = case.mask if use_mask else None
    if mask is not None:
        m = mask
    o = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    C = _lib.VERIFY_COUNTER_BYTES
    va.workspace[C:].fill_(255)  # poison the partials; the arrival counters start at zero
    va(dev(torch, case.q), dev(torch, case.k), dev(torch, case.v), va.mask_rows(m), o)
    torch.cuda.synchronize()
    assert not va.workspace[:C].any().item(), "arrival counters not returned to zero"
    return host(o), m


@pytest.mark.parametrize("trial", range(8))
def test_verify_workload(torch, trial):
    L = I.cache_length(trial)
    say(f"verify trial {trial}: causal self-attention over L={L}, cross over 1500, beam tree")
    for layer in (0, 31):
        c = I.verify_self_case(trial, layer)
        got, m = run_verify(torch, c)
        check(got, oracle.verify_attention(c.q, c.k, c.v, m), f"L{layer} causal")
        x = I.verify_cross_case(trial, layer)
        got, _ = run_verify(torch, x)
        check(got, oracle.verify_attention(x.q, x.k, x.v, None), f"L{layer} cross")
        t = I.verify_tree_case(trial, layer)
        got, m = run_verify(torch, t)
        check(got, oracle.verify_attention(t.q, t.k, t.v, m), f"L{layer} tree")


@pytest.mark.parametrize("n_q,n_kv,kind", [
    (1, 1, "none"), (1, 33, "causal"), (16, 16, "causal"), (16, 31, "causal"), (16, 32, "causal"),
    (16, 33, "causal"), (16, 127, "random"), (16, 128, "none"), (16, 129, "causal"),
    (5, 300, "random"), (16, 256, "causal"), (3, 257, "random"), (16, 384, "none"), (16, 385, "causal"),
    (16, 448, "random"), (16, 512, "causal"), (16, 513, "causal"), (2, 511, "empty_rows"), (16, 1500, "none"),
    (7, 4096, "random"), (16, 200, "empty_rows"),
    (16, 4097, "causal"), (9, 6000, "random"), (16, 5000, "empty_rows")])
def test_verify_edges(torch, n_q, n_kv, kind):
    say(f"verify edge n_q={n_q} n_kv={n_kv} {kind}")
    r = np.random.default_rng(n_q * 7919 + n_kv)
    q = r.standard_normal((n_q, 20, 64)).astype(np.float16)
    k = (r.standard_normal((n_kv, 20, 64)) * 1.5).astype(np.float16)
    v = r.standard_normal((n_kv, 20, 64)).astype(np.float16)
    if kind == "causal":
        mask = oracle.causal_rows(n_q, n_kv) if n_kv >= n_q else r.random((n_q, n_kv)) < 0.5
    elif kind == "none":
        mask = None
    else:
        mask = r.random((n_q, n_kv)) < 0.3
        empty = [i for i in (0, 5, 15) if i < n_q]
        if kind == "empty_rows":
            mask[empty] = False
    case = I.VerifyCase(q=q, k=k, v=v, mask=mask, kind=kind)
    got, m = run_verify(torch, case)
    ref = oracle.verify_attention(q, k, v, m)
    check(got, ref, "o")
    if kind == "empty_rows":
        assert np.all(got[empty] == 0)


def test_verify_graph_replay(torch):
    """The verification launches captured in a HIP graph (as a decoder replays them) give the
    eager results on every replay, with eager work between replays, and leave the workspace's
    arrival counters at zero (the graph's arguments, counters included, are fixed)."""
    from whisper_asr_encoder_amd.encoder import VerifyAttention
    say("verify graph replay: causal L=360, cross 1500, random mask 5000")
    r = np.random.default_rng(4242)
    va = VerifyAttention(5000)
    cases = []
    for n_kv, kind in ((360, "causal"), (1500, "none"), (5000, "random")):
        q = r.standard_normal((16, 20, 64)).astype(np.float16)
        k = r.standard_normal((n_kv, 20, 64)).astype(np.float16)
        v = r.standard_normal((n_kv, 20, 64)).astype(np.float16)
        mask = {"causal": oracle.causal_rows(16, n_kv), "none": None,
                "random": r.random((16, n_kv)) < 0.3}[kind]
        cases.append((dev(torch, q), dev(torch, k), dev(torch, v), va.mask_rows(mask),
                      torch.empty((16, 20, 64), dtype=torch.float16, device="cuda"), (q, k, v, mask)))

    def run():
        for q, k, v, m, o, _ in cases:
            va(q, k, v, m, o)

    run()
    torch.cuda.synchronize()
    eager = [host(c[4]) for c in cases]
    for got, c in zip(eager, cases):
        check(got, oracle.verify_attention(*c[5]), "eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for c in cases:
            c[4].fill_(float("nan"))
        va.workspace[_lib.VERIFY_COUNTER_BYTES:].fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, c in enumerate(cases):
            assert np.array_equal(host(c[4]), eager[i]), f"replay {rep} case {i}"
        assert not va.workspace[:_lib.VERIFY_COUNTER_BYTES].any().item(), f"replay {rep}: arrival counters not zero"
        run()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [1, 2])
def test_encoder_graph_replay(torch, cfg):
    """Sublayers captured in a HIP graph (as the benchmark replays them) give the eager
    results bit for bit on every replay, with eager work and synchronisations in between."""
    from whisper_asr_encoder_amd.encoder import EncoderAttention
    say(f"encoder graph replay, workload {cfg}, 2 sublayers")
    wl = I.encoder_workload(cfg, layers=2)
    weights = [wl.weights(l) for l in range(2)]
    enc = EncoderAttention(weights, wl.batch, wl.seq_len, wl.chunk_len, None if cfg == 1 else wl.valid_len)
    x = dev(torch, wl.x)
    ys = [torch.empty((wl.rows, I.D_MODEL), dtype=torch.float16, device="cuda") for _ in range(2)]

    def step():
        for l in range(2):
            enc.sublayer(x, l, ys[l])

    step()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        enc.qkv.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(2):
            assert torch.equal(ys[l], eager[l]), f"replay {rep}, layer {l} differs from eager"
        step()  # eager work between replays
        torch.cuda.synchronize()
