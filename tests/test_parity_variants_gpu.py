"""GPU parity of the drafter's attention variants (edda_verify_attn_ex) against the fp64
oracle in oracle/variants.py, through the C ABI: head counts other than 20, the causal or
non-causal block mask computed in the kernel, explicit mask rows, and per-head sinks, over
caches of one 128-key split, several splits, and more than 16 splits (the merge's batches).
Bar as for verification attention: max |delta| <= 3e-3, relative Frobenius <= 1e-3, every
output finite, the arrival counters back at zero after each call.
"""
import sys

import numpy as np
import pytest

import oracle.variants as V
from whisper_asr_encoder_amd import _lib

pytestmark = pytest.mark.gpu

ATOL, REL_FRO = 3e-3, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx = float(np.abs(got - ref).max())
    nrm = float(np.linalg.norm(ref))
    fro = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got - ref))
    say(f"  {what}: max|d| = {mx:.3e}, rel_fro = {fro:.3e}")
    assert mx <= ATOL, f"{what}: max |delta| {mx:.3e} > {ATOL}"
    assert fro <= REL_FRO, f"{what}: relative Frobenius {fro:.3e} > {REL_FRO}"


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    return t


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def make(seed, n_q, n_kv, h, sink_kind):
    r = np.random.default_rng(seed)
    q = r.standard_normal((n_q, h, 64)).astype(np.float16)
    k = (r.standard_normal((n_kv, h, 64)) * 1.5).astype(np.float16)
    v = r.standard_normal((n_kv, h, 64)).astype(np.float16)
    sinks = None
    if sink_kind == "random":
        sinks = (r.standard_normal(h) * 2).astype(np.float32)
    elif sink_kind == "mixed":  # some heads without a sink, one sink far above every score
        sinks = (r.standard_normal(h) * 2).astype(np.float32)
        sinks[::3] = -np.inf
        sinks[1] = 40.0
    return q, k, v, sinks


def run(torch, q, k, v, mode, mask=None, sinks=None):
    n_q, h, _ = q.shape
    n_kv = k.shape[0]
    nbytes = max(_lib.verify_workspace_bytes_ex(n_q, n_kv, h), _lib.VERIFY_COUNTER_BYTES)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ws[_lib.VERIFY_COUNTER_BYTES:].fill_(255)  # poison the partials; the counters start at zero
    o = torch.full(q.shape, float("nan"), dtype=torch.float16, device="cuda")
    rows = None if mask is None else torch.from_numpy(_lib.pack_mask_rows(mask).view(np.int32)).cuda()
    _lib.edda_verify_attn_ex(dev(torch, q), dev(torch, k), dev(torch, v), o, mask_mode=mode, mask_rows=rows,
                             sinks=None if sinks is None else dev(torch, sinks), workspace=ws)
    torch.cuda.synchronize()
    assert not ws[:_lib.VERIFY_COUNTER_BYTES].any().item(), "arrival counters not returned to zero"
    return o.float().cpu().numpy()


CASES = [
    # n_q, n_kv, heads, mask, sinks
    (16, 16, 8, "causal", None), (16, 16, 8, "none", "random"), (1, 1, 1, "causal", "random"),
    (5, 100, 32, "causal", "mixed"), (16, 128, 64, "none", "mixed"), (16, 129, 20, "causal", "random"),
    (16, 360, 20, "causal", None), (16, 360, 20, "none", None), (9, 1500, 12, "none", "random"),
    (16, 1500, 20, "rows", "mixed"), (3, 2200, 40, "causal", "random"), (16, 4097, 64, "causal", "mixed"),
    (16, 2100, 4, "rows", "random"), (7, 33, 2, "causal", "mixed"), (16, 300, 64, "rows", "mixed"),
    (11, 512, 20, "causal", "random"), (16, 513, 6, "none", "mixed"),
]


@pytest.mark.parametrize("n_q,n_kv,h,mask_kind,sink_kind", CASES)
def test_variant_against_oracle(torch, n_q, n_kv, h, mask_kind, sink_kind):
    say(f"variant n_q={n_q} n_kv={n_kv} heads={h} mask={mask_kind} sinks={sink_kind}")
    q, k, v, sinks = make(n_q * 131 + n_kv * 7 + h, n_q, n_kv, h, sink_kind)
    if mask_kind == "rows":
        mask = np.random.default_rng(n_kv).random((n_q, n_kv)) < 0.3
        mask[0] = False  # a row with no admitted key: the sink alone, O = 0
        got = run(torch, q, k, v, _lib.MASK_ROWS, mask=mask, sinks=sinks)
    else:
        mask = V.block_mask(n_q, n_kv, causal=mask_kind == "causal")
        mode = _lib.MASK_CAUSAL_BLOCK if mask_kind == "causal" else _lib.MASK_NONE
        got = run(torch, q, k, v, mode, sinks=sinks)
    ref = V.verify_attention_sinks(q, k, v, mask, sinks)
    check(got, ref, "o")
    if mask_kind == "rows":
        assert np.all(got[0] == 0)


def test_causal_block_mode_equals_its_mask_rows(torch):
    """The causal block computed in the kernel and the same mask passed as rows give
    bit-identical outputs (the arithmetic is the same; only the source of the bits differs)."""
    say("causal block mode vs explicit causal rows, 16 x 1000, 20 heads, sinks")
    q, k, v, sinks = make(77, 16, 1000, 20, "random")
    a = run(torch, q, k, v, _lib.MASK_CAUSAL_BLOCK, sinks=sinks)
    b = run(torch, q, k, v, _lib.MASK_ROWS, mask=V.block_mask(16, 1000, causal=True), sinks=sinks)
    assert np.array_equal(a, b)


def test_no_sink_is_plain_verification(torch):
    """Sinks of -inf, no sinks, and the 20-head entry point agree bit for bit."""
    say("sinks of -inf vs none vs edda_verify_attn, 16 x 700")
    q, k, v, _ = make(78, 16, 700, 20, None)
    a = run(torch, q, k, v, _lib.MASK_NONE)
    b = run(torch, q, k, v, _lib.MASK_NONE, sinks=np.full(20, -np.inf, dtype=np.float32))
    from whisper_asr_encoder_amd.encoder import VerifyAttention
    va = VerifyAttention(700)
    o = torch.empty(q.shape, dtype=torch.float16, device="cuda")
    va(dev(torch, q), dev(torch, k), dev(torch, v), None, o)
    torch.cuda.synchronize()
    assert np.array_equal(a, b) and np.array_equal(a, o.float().cpu().numpy())
