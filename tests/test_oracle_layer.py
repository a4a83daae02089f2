"""Pins for the encoder-layer oracle (LayerNorm, GELU, MLP, convolutional stem, pre-norm
layer), each independent of the oracle's own code: float64 library routines (torch
layer_norm, gelu, conv1d, MultiheadAttention on the CPU), exact values of the normal CDF,
invariants, closed forms and scalar brute force on tiny shapes.
"""
import math

import numpy as np
import pytest
import torch

import oracle.encoder_layer as L

TOL = 1e-12
F = torch.nn.functional


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ---------------------------------------------------------------------------
# LayerNorm
# ---------------------------------------------------------------------------

def test_layer_norm_against_torch():
    r = np.random.default_rng(1)
    x = r.standard_normal((7, 40)) * 3 + 1.5
    g, b = 1 + r.standard_normal(40) * 0.1, r.standard_normal(40) * 0.1
    ref = F.layer_norm(t64(x), (40,), t64(g), t64(b), eps=1e-5).numpy()
    assert np.abs(L.layer_norm(x, g, b) - ref).max() < TOL


def test_layer_norm_brute_force():
    r = np.random.default_rng(2)
    x = r.standard_normal((3, 9))
    g, b = r.standard_normal(9), r.standard_normal(9)
    got = L.layer_norm(x, g, b)
    for i in range(3):
        row = [float(v) for v in x[i]]
        mu = math.fsum(row) / 9
        var = math.fsum((v - mu) ** 2 for v in row) / 9
        for j in range(9):
            assert abs(got[i, j] - ((row[j] - mu) / math.sqrt(var + 1e-5) * g[j] + b[j])) < 1e-12


def test_layer_norm_invariants():
    r = np.random.default_rng(3)
    x = r.standard_normal((5, 64)) * 2
    one, zero = np.ones(64), np.zeros(64)
    y = L.layer_norm(x, one, zero)
    assert np.abs(y.mean(1)).max() < 1e-12
    var = ((x - x.mean(1, keepdims=True)) ** 2).mean(1)
    assert np.abs(y.var(1) - var / (var + 1e-5)).max() < 1e-12  # biased variance inside
    assert np.abs(L.layer_norm(x + 7.25, one, zero) - y).max() < 1e-9  # shift invariance
    c = np.full((2, 16), 3.0)  # constant rows normalise to the shift
    assert np.abs(L.layer_norm(c, np.ones(16), np.arange(16.0)) - np.arange(16.0)).max() < 1e-12


# ---------------------------------------------------------------------------
# GELU
# ---------------------------------------------------------------------------

def test_gelu_exact_values():
    # Phi(1), Phi(2), Phi(-1): standard normal CDF values.
    assert abs(L.gelu([1.0])[0] - 0.8413447460685429) < 1e-15
    assert abs(L.gelu([2.0])[0] - 2 * 0.9772498680518208) < 1e-15
    assert abs(L.gelu([-1.0])[0] - (-0.15865525393145707)) < 1e-15
    assert L.gelu([0.0])[0] == 0.0


def test_gelu_against_torch_and_odd_identity():
    x = np.linspace(-6, 6, 241)
    ref = F.gelu(t64(x), approximate="none").numpy()
    assert np.abs(L.gelu(x) - ref).max() < 1e-14
    # gelu(x) - gelu(-x) = x (Phi(x) + Phi(-x) = 1); the tanh form misses this by ~1e-4.
    assert np.abs(L.gelu(x) - L.gelu(-x) - x).max() < 1e-14


# ---------------------------------------------------------------------------
# Linear, MLP
# ---------------------------------------------------------------------------

def test_linear_and_mlp_brute_force():
    r = np.random.default_rng(4)
    x, w1, b1 = r.standard_normal((2, 5)), r.standard_normal((5, 7)), r.standard_normal(7)
    w2, b2 = r.standard_normal((7, 3)), r.standard_normal(3)
    got = L.mlp(x, w1, b1, w2, b2)
    phi = lambda v: 0.5 * (1 + math.erf(v / math.sqrt(2)))
    for i in range(2):
        hid = [math.fsum(x[i, k] * w1[k, j] for k in range(5)) + b1[j] for j in range(7)]
        hid = [v * phi(v) for v in hid]
        for c in range(3):
            assert abs(got[i, c] - (math.fsum(hid[j] * w2[j, c] for j in range(7)) + b2[c])) < 1e-12


# ---------------------------------------------------------------------------
# Convolutional stem
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("stride", [1, 2])
@pytest.mark.parametrize("t_in", [1, 2, 5, 8])
def test_conv_against_torch(stride, t_in):
    r = np.random.default_rng(10 * stride + t_in)
    x, w, b = r.standard_normal((t_in, 6)), r.standard_normal((4, 6, 3)), r.standard_normal(4)
    ref = F.conv1d(t64(x.T[None]), t64(w), t64(b), stride=stride, padding=1)[0].T.numpy()
    got = L.conv1d_k3(x, w, b, stride)
    assert got.shape == ref.shape and np.abs(got - ref).max() < TOL


def test_conv_brute_force_taps():
    r = np.random.default_rng(11)
    x, w, b = r.standard_normal((6, 2)), r.standard_normal((3, 2, 3)), r.standard_normal(3)
    got = L.conv1d_k3(x, w, b, 2)
    for t in range(3):
        for o in range(3):
            acc = [b[o]]
            for tap in range(3):
                src = 2 * t + tap - 1
                if 0 <= src < 6:
                    acc += [x[src, c] * w[o, c, tap] for c in range(2)]
            assert abs(got[t, o] - math.fsum(acc)) < 1e-12


def test_stem_against_torch_and_shape():
    r = np.random.default_rng(12)
    mel = r.standard_normal((5, 10))  # [n_mels, frames]
    c1w, c1b = r.standard_normal((8, 5, 3)) * 0.3, r.standard_normal(8) * 0.1
    c2w, c2b = r.standard_normal((8, 8, 3)) * 0.3, r.standard_normal(8) * 0.1
    pos = r.standard_normal((5, 8))
    got = L.encoder_stem(mel, c1w, c1b, c2w, c2b, pos)
    h = F.gelu(F.conv1d(t64(mel[None]), t64(c1w), t64(c1b), padding=1))
    h = F.gelu(F.conv1d(h, t64(c2w), t64(c2b), stride=2, padding=1))[0].T + t64(pos)
    assert got.shape == (5, 8) and np.abs(got - h.numpy()).max() < TOL


# ---------------------------------------------------------------------------
# Pre-norm encoder layer
# ---------------------------------------------------------------------------

class _W:
    pass


def tiny_layer(seed, d=16, n_heads=2, ff=32, zero_mlp=False, zero_attn=False):
    r = np.random.default_rng(seed)
    w = _W()
    w.ln1_g, w.ln1_b = 1 + r.standard_normal(d) * 0.1, r.standard_normal(d) * 0.1
    w.w_qkv, w.b_qkv = r.standard_normal((d, 3 * d)) * 0.4, r.standard_normal(3 * d) * 0.1
    w.w_o, w.b_o = r.standard_normal((d, d)) * 0.3, r.standard_normal(d) * 0.1
    w.ln2_g, w.ln2_b = 1 + r.standard_normal(d) * 0.1, r.standard_normal(d) * 0.1
    w.w_fc1, w.b_fc1 = r.standard_normal((d, ff)) * 0.3, r.standard_normal(ff) * 0.1
    w.w_fc2, w.b_fc2 = r.standard_normal((ff, d)) * 0.2, r.standard_normal(d) * 0.1
    if zero_attn:
        w.w_o, w.b_o = np.zeros((d, d)), np.zeros(d)
    if zero_mlp:
        w.w_fc2, w.b_fc2 = np.zeros((ff, d)), np.zeros(d)
    return w


def torch_layer(x, w, n_heads, seq_len, chunk_len, valid_len):
    """float64 reference from torch.nn.MultiheadAttention and torch layers."""
    d = x.shape[1]
    mha = torch.nn.MultiheadAttention(d, n_heads, bias=True, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        mha.in_proj_weight.copy_(t64(w.w_qkv).T)
        mha.in_proj_bias.copy_(t64(w.b_qkv))
        mha.out_proj.weight.copy_(t64(w.w_o).T)
        mha.out_proj.bias.copy_(t64(w.b_o))
        xs = t64(x).reshape(-1, seq_len, d)
        i = torch.arange(seq_len)
        if chunk_len:
            lo = (i // chunk_len) * chunk_len
            hi = torch.clamp(lo + chunk_len, max=valid_len)
        else:
            lo, hi = torch.zeros_like(i), torch.full_like(i, valid_len)
        blocked = ~((i[None, :] >= lo[:, None]) & (i[None, :] < hi[:, None]))  # True = not admitted
        h = F.layer_norm(xs, (d,), t64(w.ln1_g), t64(w.ln1_b), eps=1e-5)
        a, _ = mha(h, h, h, attn_mask=blocked, need_weights=False)
        x1 = xs + a
        h2 = F.layer_norm(x1, (d,), t64(w.ln2_g), t64(w.ln2_b), eps=1e-5)
        y = x1 + F.gelu(h2 @ t64(w.w_fc1) + t64(w.b_fc1)) @ t64(w.w_fc2) + t64(w.b_fc2)
    return x1.reshape(-1, d).numpy(), y.reshape(-1, d).numpy()


@pytest.mark.parametrize("seq_len,chunk_len,valid_len,batch", [(6, 0, 6, 1), (8, 4, 7, 1), (5, 0, 5, 2)])
def test_layer_against_torch(seq_len, chunk_len, valid_len, batch):
    r = np.random.default_rng(seq_len * 31 + chunk_len)
    x = r.standard_normal((batch * seq_len, 16))
    w = tiny_layer(5 + batch)
    got = L.encoder_layer(x, w, batch, seq_len, chunk_len, valid_len, n_heads=2)
    x1, y = torch_layer(x, w, 2, seq_len, chunk_len, valid_len)
    assert np.abs(got["x1"] - x1).max() < 1e-10
    assert np.abs(got["y"] - y).max() < 1e-10


def test_layer_closed_forms():
    r = np.random.default_rng(6)
    x = r.standard_normal((6, 16))
    # No attention output and no MLP output: the residual stream passes through.
    w = tiny_layer(7, zero_attn=True, zero_mlp=True)
    got = L.encoder_layer(x, w, 1, 6, 0, 6, n_heads=2)
    assert np.abs(got["x1"] - x).max() < 1e-15 and np.abs(got["y"] - x).max() < 1e-15
    # MLP output = b_fc2 only: y = x1 + b_fc2.
    w = tiny_layer(8)
    w.w_fc2 = np.zeros_like(w.w_fc2)
    got = L.encoder_layer(x, w, 1, 6, 0, 6, n_heads=2)
    assert np.abs(got["y"] - got["x1"] - w.b_fc2).max() < 1e-15


def test_layer_row_subset_matches_full():
    r = np.random.default_rng(9)
    x = r.standard_normal((10, 16))
    w = tiny_layer(9)
    full = L.encoder_layer(x, w, 2, 5, 0, 5, n_heads=2)
    rows = np.array([1, 4, 7])
    sub = L.encoder_layer(x, w, 2, 5, 0, 5, n_heads=2, rows=rows)
    assert np.abs(sub["y"] - full["y"][rows]).max() < 1e-12
