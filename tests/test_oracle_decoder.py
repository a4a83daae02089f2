"""Pins for the decoder verification-layer oracle, independent of its own code: float64 torch
(MultiheadAttention, scaled_dot_product_attention, layer_norm, gelu, linear), brute force for
the cache append, closed forms, an invariance under relabelling cache slots, and planted
mistakes that must each fail one of these pins.
"""
import numpy as np
import pytest
import torch

import oracle.decoder_layer as D

F = torch.nn.functional
TOL = 1e-10


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


class _W:
    pass


def tiny(seed, d=16, ff=32, zero_out=False):
    r = np.random.default_rng(seed)
    w = _W()
    for n in ("ln1", "ln2", "ln3"):
        setattr(w, n + "_g", 1 + r.standard_normal(d) * 0.1)
        setattr(w, n + "_b", r.standard_normal(d) * 0.1)
    w.w_qkv, w.b_qkv = r.standard_normal((d, 3 * d)) * 0.4, r.standard_normal(3 * d) * 0.1
    w.b_qkv[d:2 * d] = 0
    w.w_o, w.b_o = r.standard_normal((d, d)) * 0.3, r.standard_normal(d) * 0.1
    w.w_qc, w.b_qc = r.standard_normal((d, d)) * 0.4, r.standard_normal(d) * 0.1
    w.w_oc, w.b_oc = r.standard_normal((d, d)) * 0.3, r.standard_normal(d) * 0.1
    w.w_fc1, w.b_fc1 = r.standard_normal((d, ff)) * 0.3, r.standard_normal(ff) * 0.1
    w.w_fc2, w.b_fc2 = r.standard_normal((ff, d)) * 0.2, r.standard_normal(d) * 0.1
    if zero_out:
        for n in ("w_o", "b_o", "w_oc", "b_oc", "w_fc2", "b_fc2"):
            setattr(w, n, np.zeros_like(getattr(w, n)))
    return w


def case(seed, n_q=4, n_kv=9, cap=12, frames=7, d=16, h=2):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n_q, d))
    kc, vc = r.standard_normal((cap, h, d // h)), r.standard_normal((cap, h, d // h))
    ck, cv = r.standard_normal((frames, h, d // h)), r.standard_normal((frames, h, d // h))
    slots = list(range(n_kv - n_q, n_kv))
    mask = np.zeros((n_q, n_kv), dtype=bool)
    for t in range(n_q):
        mask[t, :n_kv - n_q + t + 1] = True
    return x, kc, vc, ck, cv, slots, mask


def run(x, w, slots, kc, vc, n_kv, mask, ck, cv, h=2):
    return D.decoder_verify_layer(x, w, slots, kc, vc, n_kv, mask, ck, cv, n_heads=h)


def torch_layer(x, w, slots, kc, vc, n_kv, mask, ck, cv, h=2):
    """float64 torch reference: projections, SDPA on the appended cache, LayerNorm, GELU MLP."""
    d = x.shape[1]
    dh = d // h
    X = t64(x)
    ln = lambda a, g, b: F.layer_norm(a, (d,), t64(g), t64(b), eps=1e-5)
    sdpa = lambda q, k, v, m: F.scaled_dot_product_attention(
        q.reshape(-1, h, dh).transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
        attn_mask=None if m is None else t64(m).bool()).transpose(0, 1).reshape(-1, d)
    qkv = ln(X, w.ln1_g, w.ln1_b) @ t64(w.w_qkv) + t64(w.b_qkv)
    K, V = t64(kc).clone(), t64(vc).clone()
    K[slots] = qkv[:, d:2 * d].reshape(-1, h, dh)
    V[slots] = qkv[:, 2 * d:].reshape(-1, h, dh)
    x1 = X + sdpa(qkv[:, :d], K[:n_kv], V[:n_kv], mask) @ t64(w.w_o) + t64(w.b_o)
    qc = ln(x1, w.ln2_g, w.ln2_b) @ t64(w.w_qc) + t64(w.b_qc)
    x2 = x1 + sdpa(qc, t64(ck), t64(cv), None) @ t64(w.w_oc) + t64(w.b_oc)
    y = x2 + F.gelu(ln(x2, w.ln3_g, w.ln3_b) @ t64(w.w_fc1) + t64(w.b_fc1)) @ t64(w.w_fc2) + t64(w.b_fc2)
    return K.numpy(), V.numpy(), x1.numpy(), x2.numpy(), y.numpy()


@pytest.mark.parametrize("seed,n_q,n_kv", [(1, 4, 9), (2, 1, 5), (3, 5, 5)])
def test_layer_against_torch_sdpa(seed, n_q, n_kv):
    x, kc, vc, ck, cv, slots, mask = case(seed, n_q=n_q, n_kv=n_kv)
    w = tiny(seed)
    got = run(x, w, slots, kc, vc, n_kv, mask, ck, cv)
    K, V, x1, x2, y = torch_layer(x, w, slots, kc, vc, n_kv, mask, ck, cv)
    assert np.abs(got["k_cache"] - K).max() < TOL and np.abs(got["v_cache"] - V).max() < TOL
    for name, ref in (("x1", x1), ("x2", x2), ("y", y)):
        assert np.abs(got[name] - ref).max() < TOL, name


def test_self_attention_of_a_lone_block_is_causal_multihead_attention():
    """With the cache holding only the block (slots 0..n_q-1) and a causal mask, the
    self-attention sublayer is torch.nn.MultiheadAttention over LN1(x) with a causal mask."""
    n_q, d, h = 5, 16, 2
    x, kc, vc, ck, cv, _, _ = case(7, n_q=n_q, n_kv=n_q)
    w = tiny(7)
    mask = np.tril(np.ones((n_q, n_q), dtype=bool))
    got = run(x, w, list(range(n_q)), kc, vc, n_q, mask, ck, cv)
    mha = torch.nn.MultiheadAttention(d, h, bias=True, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        mha.in_proj_weight.copy_(t64(w.w_qkv).T)
        mha.in_proj_bias.copy_(t64(w.b_qkv))
        mha.out_proj.weight.copy_(t64(w.w_o).T)
        mha.out_proj.bias.copy_(t64(w.b_o))
        hh = F.layer_norm(t64(x)[None], (d,), t64(w.ln1_g), t64(w.ln1_b), eps=1e-5)
        a, _ = mha(hh, hh, hh, attn_mask=~t64(mask).bool(), need_weights=False)
    assert np.abs(got["x1"] - (t64(x) + a[0]).numpy()).max() < TOL


def test_append_writes_only_the_block_slots():
    x, kc, vc, ck, cv, _, _ = case(4, n_q=3, n_kv=8)
    slots = [6, 2, 7]
    kn, vn = np.ones((3, 2, 8)) * np.arange(3)[:, None, None], -np.ones((3, 2, 8))
    k, v = D.append_kv(kc, vc, slots, kn, vn)
    for s in range(kc.shape[0]):
        if s in slots:
            t = slots.index(s)
            assert (k[s] == kn[t]).all() and (v[s] == vn[t]).all()
        else:
            assert (k[s] == kc[s]).all() and (v[s] == vc[s]).all()
    assert k is not kc and not np.shares_memory(k, kc)


def test_cross_kv_against_torch_linear():
    r = np.random.default_rng(5)
    enc, wk, wv, bv = r.standard_normal((7, 16)), r.standard_normal((16, 16)), r.standard_normal((16, 16)), r.standard_normal(16)
    k, v = D.cross_kv(enc, wk, wv, bv, n_heads=2)
    assert np.abs(k.reshape(7, 16) - F.linear(t64(enc), t64(wk).T).numpy()).max() < 1e-12
    assert np.abs(v.reshape(7, 16) - F.linear(t64(enc), t64(wv).T, t64(bv)).numpy()).max() < 1e-12


def test_closed_form_zero_outputs_pass_the_residual_stream():
    x, kc, vc, ck, cv, slots, mask = case(6)
    got = run(x, tiny(6, zero_out=True), slots, kc, vc, 9, mask, ck, cv)
    assert np.abs(got["y"] - x).max() < 1e-15


def test_relabelling_slots_leaves_the_output_unchanged():
    """Moving the block into other free slots (with the mask moved along) changes nothing."""
    n_q, n_kv = 3, 9
    x, kc, vc, ck, cv, _, _ = case(8, n_q=n_q, n_kv=n_kv)
    w = tiny(8)
    a_slots = [6, 7, 8]
    b_slots = [1, 4, 8]
    perm = list(range(n_kv))
    # Slots 1, 4 (old history) swap with 6, 7 so the history stays at the same keys.
    perm[1], perm[6], perm[4], perm[7] = 6, 1, 7, 4
    mask_a = np.zeros((n_q, n_kv), dtype=bool)
    for t in range(n_q):
        mask_a[t, :6] = True
        mask_a[t, a_slots[:t + 1]] = True
    kb, vb = kc.copy(), vc.copy()
    kb[:n_kv], vb[:n_kv] = kc[perm], vc[perm]
    mask_b = mask_a[:, perm]
    ya = run(x, w, a_slots, kc, vc, n_kv, mask_a, ck, cv)["y"]
    yb = run(x, w, b_slots, kb, vb, n_kv, mask_b, ck, cv)["y"]
    assert np.abs(ya - yb).max() < 1e-12


# ---------------------------------------------------------------------------
# Planted mistakes.
# ---------------------------------------------------------------------------

ORIG = {n: getattr(D, n) for n in ("append_kv", "decoder_verify_layer", "cross_kv")}


def _append_in_order(k_cache, v_cache, slots, k_new, v_new):
    return ORIG["append_kv"](k_cache, v_cache, list(range(len(slots))), k_new, v_new)


def _cross_uses_self_cache(x, w, slots, kc, vc, n_kv, mask, ck, cv, n_heads=D.N_HEADS):
    return ORIG["decoder_verify_layer"](x, w, slots, kc, vc, n_kv, mask, np.asarray(kc)[:n_kv],
                                        np.asarray(vc)[:n_kv], n_heads)


def _no_x1_residual_in_x2(x, w, slots, kc, vc, n_kv, mask, ck, cv, n_heads=D.N_HEADS):
    out = ORIG["decoder_verify_layer"](x, w, slots, kc, vc, n_kv, mask, ck, cv, n_heads)
    out["y"] = out["y"] - out["x1"]
    return out


def _cross_k_with_bias(enc, w_k, w_v, b_v=None, n_heads=D.N_HEADS):
    k, v = ORIG["cross_kv"](enc, w_k, w_v, b_v, n_heads)
    return k + np.asarray(b_v).reshape(1, *k.shape[1:]), v


MUTANTS = {"append_in_order": ("append_kv", _append_in_order),
           "cross_uses_self_cache": ("decoder_verify_layer", _cross_uses_self_cache),
           "no_x1_residual": ("decoder_verify_layer", _no_x1_residual_in_x2),
           "cross_k_bias": ("cross_kv", _cross_k_with_bias)}


def run_pins():
    test_layer_against_torch_sdpa(1, 4, 9)
    test_append_writes_only_the_block_slots()
    test_cross_kv_against_torch_linear()
    test_relabelling_slots_leaves_the_output_unchanged()


def test_unmutated_pins_pass():
    run_pins()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    target, fn = MUTANTS[name]
    monkeypatch.setattr(D, target, fn)
    with pytest.raises(AssertionError):
        run_pins()
