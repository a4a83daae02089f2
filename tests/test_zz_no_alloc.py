"""edda_verify_attn_noalloc (static scratch, no allocation) against edda_verify_attn (caller
workspace) through the C ABI: two calls in a row, the second with a smaller input, each
compared with the workspace entry point's output (same kernels, so bit for bit) and with the
fp64 oracle at the path's bar (max |delta| <= 3e-3, relative Frobenius <= 1e-3). The first
call needs the split path (its partials and arrival counters live in the static array), the
second reuses the array with fewer splits, a third takes one workgroup per head (no scratch);
the array's counters must be back at zero after every call for the next call to be right,
which the repeated calls check."""
import sys

import numpy as np
import pytest

import oracle
from whisper_asr_encoder_amd import _lib

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    _lib.load()
    return t


def case(seed, n_q, n_kv, kind):
    r = np.random.default_rng(seed)
    q = r.standard_normal((n_q, 20, 64)).astype(np.float16)
    k = r.standard_normal((n_kv, 20, 64)).astype(np.float16)
    v = r.standard_normal((n_kv, 20, 64)).astype(np.float16)
    mask = {"causal": oracle.causal_rows(n_q, n_kv), "none": None, "random": r.random((n_q, n_kv)) < 0.3}[kind]
    return q, k, v, mask


def test_noalloc_matches_workspace_entry(torch):
    from whisper_asr_encoder_amd.encoder import VerifyAttention
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    va = VerifyAttention(_lib.NOALLOC_MAX_KV)
    for n_q, n_kv, kind in ((16, 5000, "random"), (9, 1500, "none"), (16, 360, "causal"), (16, 8192, "causal"),
                            (3, 600, "random")):
        say(f"noalloc verify n_q={n_q} n_kv={n_kv} {kind}")
        q, k, v, mask = case(n_q * 131 + n_kv, n_q, n_kv, kind)
        qd, kd, vd, md = d(q), d(k), d(v), va.mask_rows(mask)
        o_ws = torch.full((n_q, 20, 64), float("nan"), dtype=torch.float16, device="cuda")
        o_na = torch.full((n_q, 20, 64), float("nan"), dtype=torch.float16, device="cuda")
        va(qd, kd, vd, md, o_ws)
        _lib.edda_verify_attn_noalloc(qd, kd, vd, md, o_na)
        torch.cuda.synchronize()
        got = o_na.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), "non-finite output"
        assert torch.equal(o_na, o_ws), "static-scratch result differs from the workspace entry point's"
        ref = oracle.verify_attention(q, k, v, mask)
        mx = float(np.abs(got - ref).max())
        fro = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        say(f"  max|d| {mx:.3e} rel_fro {fro:.3e}")
        assert mx <= 3e-3 and fro <= 1e-3
