"""Pins for the Q8_0 oracle (oracle/quant.py), independent of its own code: closed forms worked
out by hand (integer blocks, exact ties, one fp16 rounding of a scale), invariants (per-block
scales, power-of-two scaling, the error bound of rounding to the nearest code, the block
maximum on +-127), float64 torch linear on the dequantized weights, and planted mistakes that
must each fail one of these pins.
"""
import numpy as np
import pytest
import torch

import oracle.quant as Q

F = torch.nn.functional


def test_integer_block_is_exact():
    """A block of integers whose largest magnitude is 127 has d = 1 and q = x."""
    x = np.zeros((1, 32), dtype=np.float16)
    x[0] = np.arange(-16, 16) * 7
    x[0, 5] = -127
    q, d = Q.quantize_q8_0(x)
    assert d.dtype == np.float16 and d.shape == (1, 1) and float(d[0, 0]) == 1.0
    assert np.array_equal(q.astype(np.int64), x.astype(np.int64))


def test_ties_round_half_away_from_zero():
    """amax = 127/8 gives d = 1/8 exactly (1/d = 8); values (n + 1/2)/8 land on exact ties."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 127 / 8
    halves = np.array([0.5, 1.5, 2.5, 3.5, 10.5, 126.5], dtype=np.float32)
    x[0, 1:7] = halves / 8
    x[0, 7:13] = -halves / 8
    q, d = Q.quantize_q8_0(x.astype(np.float16))
    assert float(d[0, 0]) == 0.125
    assert list(q[0, 1:7]) == [1, 2, 3, 4, 11, 127]
    assert list(q[0, 7:13]) == [-1, -2, -3, -4, -11, -127]
    assert q[0, 0] == 127


def test_scale_is_rounded_to_fp16():
    """amax = 1: d = 1/127 in fp32 is stored as the nearest fp16, 2^-7 (1 + 8/1024)."""
    x = np.zeros((1, 32), dtype=np.float16)
    x[0, 3] = 1.0
    q, d = Q.quantize_q8_0(x)
    assert float(d[0, 0]) == 0.00787353515625
    assert q[0, 3] == 127 and not np.delete(q[0], 3).any()
    assert Q.dequantize_q8_0(q, d)[0, 3] == 127 * 0.00787353515625


def test_zero_block_and_independent_blocks():
    x = np.zeros((2, 96), dtype=np.float16)
    x[0, 32:64] = np.linspace(-3, 3, 32)       # block 1 of row 0
    x[0, 64:96] = np.linspace(-0.01, 0.02, 32)  # block 2 of row 0: its own small scale
    x[1, :32] = 1000.0
    q, d = Q.quantize_q8_0(x)
    assert d[0, 0] == 0 and not q[0, :32].any()
    assert np.isclose(float(d[0, 1]), 3 / 127, rtol=1e-3)
    assert np.isclose(float(d[0, 2]), 0.02 / 127, rtol=1e-3)
    assert (q[1, :32] == 127).all()


def test_power_of_two_scaling():
    r = np.random.default_rng(3)
    x = (r.standard_normal((4, 128)) * 0.5).astype(np.float16)
    q1, d1 = Q.quantize_q8_0(x)
    q2, d2 = Q.quantize_q8_0((x.astype(np.float32) * 8).astype(np.float16))
    assert np.array_equal(q1, q2)
    assert np.array_equal(d1.astype(np.float64) * 8, d2.astype(np.float64))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rounding_error_bound_and_block_maximum(seed):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((8, 256)) * 10.0 ** r.uniform(-3, 1, (8, 1))).astype(np.float16)
    q, d = Q.quantize_q8_0(x)
    assert np.abs(q.astype(np.int64)).max() <= 127
    xb = x.astype(np.float64).reshape(8, 8, 32)
    d32 = np.abs(xb).max(axis=2) / 127          # the fp32 scale before its fp16 rounding
    err = np.abs(xb - q.astype(np.float64).reshape(8, 8, 32) * d32[..., None])
    assert (err <= d32[..., None] * (0.5 + 1e-5)).all()
    idx = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(q.reshape(8, 8, 32).astype(np.int64), idx[..., None], axis=2)[..., 0]
    assert (np.abs(top) == 127).all()
    assert (np.sign(top) == np.sign(np.take_along_axis(xb, idx[..., None], axis=2)[..., 0])).all()


def test_linear_q8_against_torch():
    r = np.random.default_rng(5)
    x = r.standard_normal((5, 64)).astype(np.float16)
    w = (r.standard_normal((48, 64)) * 0.1).astype(np.float16)
    b = r.standard_normal(48)
    q, d = Q.quantize_q8_0(w)
    deq = torch.from_numpy(q.astype(np.float64)) * torch.from_numpy(d.astype(np.float64)).repeat_interleave(32, dim=1)
    ref = F.linear(torch.from_numpy(x.astype(np.float64)), deq, torch.from_numpy(b)).numpy()
    assert np.abs(Q.linear_q8(x, q, d, b) - ref).max() < 1e-12


# ---------------------------------------------------------------------------
# Planted mistakes.
# ---------------------------------------------------------------------------

ORIG = Q.quantize_q8_0


def _scale_128(w):
    q, d = ORIG(w)
    x = np.asarray(w, dtype=np.float32)
    amax = np.abs(x.reshape(x.shape[0], -1, 32)).max(axis=2)
    return q, (amax / np.float32(128)).astype(np.float16)


def _round_half_even(w):
    x = np.asarray(w, dtype=np.float32)
    n, k = x.shape
    b = x.reshape(n, k // 32, 32)
    d = (np.abs(b).max(axis=2) / np.float32(127)).astype(np.float32)
    inv = np.where(d != 0, np.float32(1) / np.where(d != 0, d, 1), 0).astype(np.float32)
    q = np.round((b * inv[..., None]).astype(np.float32))
    return q.reshape(n, k).astype(np.int8), d.astype(np.float16)


def _floor(w):
    x = np.asarray(w, dtype=np.float32)
    n, k = x.shape
    b = x.reshape(n, k // 32, 32)
    d = (np.abs(b).max(axis=2) / np.float32(127)).astype(np.float32)
    inv = np.where(d != 0, np.float32(1) / np.where(d != 0, d, 1), 0).astype(np.float32)
    q = np.floor((b * inv[..., None]).astype(np.float32))
    return q.reshape(n, k).astype(np.int8), d.astype(np.float16)


def _row_scale(w):
    x = np.asarray(w, dtype=np.float32)
    n, k = x.shape
    d = (np.abs(x).max(axis=1, keepdims=True) / np.float32(127)).astype(np.float32)
    inv = np.where(d != 0, np.float32(1) / np.where(d != 0, d, 1), 0).astype(np.float32)
    y = (x * inv).astype(np.float64)
    q = np.trunc(y + np.copysign(0.5, y))
    return q.astype(np.int8), np.repeat(d, k // 32, axis=1).astype(np.float16)


def _scale_not_fp16(w):
    q, _ = ORIG(w)
    x = np.asarray(w, dtype=np.float32)
    d = (np.abs(x.reshape(x.shape[0], -1, 32)).max(axis=2) / np.float32(127)).astype(np.float32)
    return q, d  # fp32 scale: dequantization then differs from fp16(d) q


MUTANTS = {"scale_128": _scale_128, "round_half_even": _round_half_even, "floor": _floor,
           "row_scale": _row_scale, "scale_not_fp16": _scale_not_fp16}


def run_pins():
    test_integer_block_is_exact()
    test_ties_round_half_away_from_zero()
    test_scale_is_rounded_to_fp16()
    test_zero_block_and_independent_blocks()
    test_rounding_error_bound_and_block_maximum(0)


def test_unmutated_pins_pass():
    run_pins()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(Q, "quantize_q8_0", MUTANTS[name])
    with pytest.raises(AssertionError):
        run_pins()


def test_dequantized_decoder_layer_wiring():
    """Weights that Q8_0 represents exactly (per block: integers times a power of two, one
    entry at +-127) give a dequantized decoder layer equal to the layer on the weights."""
    import oracle.decoder_layer as D
    from tests.test_oracle_decoder import case, tiny
    r = np.random.default_rng(11)
    w = tiny(11, d=32, ff=64)
    for name in Q.DequantizedDecoderWeights.MATRICES:
        m = np.asarray(getattr(w, name))              # [in, out]
        out_in = r.integers(-126, 127, size=m.T.shape).astype(np.float64)
        out_in.reshape(out_in.shape[0], -1, 32)[:, :, 0] = 127
        scale = 2.0 ** r.integers(-9, -5, size=(out_in.shape[0], out_in.shape[1] // 32))
        setattr(w, name, (out_in * np.repeat(scale, 32, axis=1)).T)
    codes = Q.quantize_decoder_weights(w)
    wq = Q.DequantizedDecoderWeights(w, codes)
    for name in Q.DequantizedDecoderWeights.MATRICES:
        assert np.array_equal(getattr(wq, name), getattr(w, name)), name
    x, kc, vc, ck, cv, slots, mask = case(12, d=32, h=2)
    got = D.decoder_verify_layer(x, wq, slots, kc, vc, 9, mask, ck, cv, n_heads=2)
    ref = D.decoder_verify_layer(x, w, slots, kc, vc, 9, mask, ck, cv, n_heads=2)
    assert np.array_equal(got["y"], ref["y"])
