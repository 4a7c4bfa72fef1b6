"""Pins of the oracle's rotary encoding and row quantisation (no GPU).

RoPE pins: the interleaved ("rotate every two") rotary implementation of a
third-party library (GPT-J in HuggingFace transformers) at small positions;
the rotation-group identity R(-delta) R(p) = R(p - delta) in fp32 to 1e-5 over
the positions a 42-step reset period reaches; p = 0 is the identity; pair norms
are kept; q.k depends on position differences only.

Quantisation pins: the absmax element of every non-zero row encodes to +-448;
the dequantisation error is within half an E4M3 ulp; zero rows give scale 0
and zero codes.
"""
import numpy as np
import pytest
import torch

import oracle

BASE = 10000.0


def test_rope_matches_gptj_interleaved_rotary():
    from transformers.models.gptj.modeling_gptj import (apply_rotary_pos_emb,
                                                         create_sinusoidal_positions)
    D, n = 64, 256
    rng = np.random.default_rng(1)
    x = rng.standard_normal((n, D)).astype(np.float32)
    pos = np.arange(n, dtype=np.int64)
    sc = create_sinusoidal_positions(n, D)                    # [n][D] = [sin | cos]
    sin, cos = sc[:, : D // 2], sc[:, D // 2:]
    xt = torch.from_numpy(x)[None, :, None, :]                # [batch, seq, heads, D]
    ref = apply_rotary_pos_emb(xt, sin[None], cos[None])[0, :, 0, :].numpy()
    got = oracle.rope_rows(x, pos, BASE)
    # the library forms angles in fp32: error <= n * 2^-24 rad per angle
    assert np.abs(got - ref).max() < 1e-4


def test_rope_group_identity_fp32():
    rng = np.random.default_rng(2)
    D, n = 128, 4000
    x = rng.standard_normal((n, D)).astype(np.float32)
    p = rng.integers(0, 37583, n)
    delta = rng.integers(1, 31795, n)
    a = oracle.rope_rows(oracle.rope_rows(x, p, BASE), -delta, BASE)
    b = oracle.rope_rows(x, p - delta, BASE)
    assert np.abs(a - b).max() <= 1e-5


def test_rope_position_zero_is_identity_and_norms_kept():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    assert np.array_equal(oracle.rope_rows(x, 0, BASE), x)
    p = rng.integers(-40000, 40000, 64)
    y = oracle.rope_rows(x, p, BASE)
    nx = np.hypot(x[:, 0::2], x[:, 1::2])
    ny = np.hypot(y[:, 0::2], y[:, 1::2])
    assert np.abs(ny - nx).max() <= 4e-7 * nx.max()


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(4)
    D, n = 128, 500
    q = rng.standard_normal((n, D)).astype(np.float32)
    k = rng.standard_normal((n, D)).astype(np.float32)
    pq = rng.integers(0, 6000, n)
    pk = rng.integers(0, 6000, n)
    c = rng.integers(-31794, 31794, n)
    d0 = (oracle.rope_rows(q, pq).astype(np.float64) * oracle.rope_rows(k, pk)).sum(-1)
    d1 = (oracle.rope_rows(q, pq + c).astype(np.float64) * oracle.rope_rows(k, pk + c)).sum(-1)
    assert np.abs(d0 - d1).max() <= 1e-5 * np.sqrt(D) * 4


def test_rope_is_not_a_half_split_rotation():
    # a rotation of (x[i], x[i + D/2]) pairs would move x[1] into x[D/2 + 1]
    D = 8
    x = np.zeros((1, D), np.float32)
    x[0, 0] = 1.0
    y = oracle.rope_rows(x, 1, BASE)[0]
    assert y[1] != 0.0 and np.all(y[2:] == 0.0)
    assert abs(y[0] - np.cos(1.0)) < 1e-7 and abs(y[1] - np.sin(1.0)) < 1e-7


# ---------------------------------------------------------------------------
def _half_ulp(t):
    a = np.abs(t).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))


def test_quant_rows_invariants():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((3000, 128)) * rng.uniform(1e-3, 50, (3000, 1))).astype(np.float32)
    y[7] = 0.0
    y[11, 5] = -0.0
    codes, scales = oracle.quant_rows(y)
    assert scales[7] == 0.0 and not codes[7].any()
    a = np.abs(y).max(axis=1)
    nz = a > 0
    am = np.abs(y).argmax(axis=1)
    top = codes[np.arange(len(y)), am]
    assert np.all((top[nz] & 0x7F) == 0x7E)
    assert np.all(np.abs(scales[nz] - a[nz] / 448.0) <= 1e-7 * a[nz] / 448.0)
    # error of each code against the scaled value is at most half an ulp
    t = y[nz].astype(np.float64) * (448.0 / a[nz, None])
    dec = oracle.e4m3_decode(codes[nz])
    assert np.all(np.abs(dec - t) <= _half_ulp(t) * (1 + 1e-6) + 1e-5)
    # dequantised rows reproduce the input within half an ulp of the scaled value
    x = oracle.dequant_rows(codes, scales)
    assert np.all(np.abs(x[nz] - y[nz]) <= (_half_ulp(t) + 1e-5) * scales[nz, None] * 1.0001)


def test_quant_sign_of_zero_and_tiny():
    y = np.zeros((1, 64), np.float32)
    y[0, 0] = 1.0
    y[0, 1] = -1e-9          # rounds to a negative zero code
    codes, s = oracle.quant_rows(y)
    assert codes[0, 0] == 0x7E and codes[0, 1] == 0x80 and codes[0, 2] == 0x00


def _tiny_rows(rng, D=64):
    """Rows whose absmax runs over every power of two from the smallest fp32
    denormal (2^-149) to 2^-40, each also one fp32 step above and below."""
    heads = []
    for j in range(-149, -39):
        b = np.float32(2.0 ** j)
        heads += [b, np.nextafter(b, np.float32(np.inf)), np.nextafter(b, np.float32(0))]
    heads = np.array([h for h in heads if h > 0], np.float32)
    n = heads.size
    y = (rng.uniform(-1, 1, (n, D)) * heads[:, None].astype(np.float64)).astype(np.float32)
    y[:, 0] = np.where(rng.random(n) < 0.5, heads, -heads)
    y = np.where(np.abs(y) <= np.abs(y[:, :1]), y, y[:, :1]).astype(np.float32)
    return y


def test_quant_tiny_rows_codes_finite_and_exact():
    """Down to the smallest fp32 denormal: no NaN codes, the absmax element
    encodes to +-448, and every code is within half an E4M3 ulp of the real
    value y * 448 / absmax (formed here in fp64)."""
    y = _tiny_rows(np.random.default_rng(6))
    codes, scales = oracle.quant_rows(y)
    assert not np.any((codes & 0x7F) == 0x7F), "NaN code"
    a = np.abs(y).max(axis=1).astype(np.float64)
    am = np.abs(y).argmax(axis=1)
    assert np.all((codes[np.arange(len(y)), am] & 0x7F) == 0x7E)
    t = y.astype(np.float64) * (448.0 / a[:, None])
    dec = oracle.e4m3_decode(codes)
    assert np.all(np.isfinite(dec))
    assert np.all(np.abs(dec - t) <= _half_ulp(t) * (1 + 1e-6) + 1e-5)
    # the scale is a / 448 in fp32 (tiny rows give denormal or zero scales)
    assert np.array_equal(scales, (y_abs := np.abs(y).max(axis=1)) / np.float32(448.0))
    assert np.all(np.isfinite(oracle.dequant_rows(codes, scales)))


def test_quant_codes_invariant_under_power_of_two_scaling():
    """y / absmax does not change when a row is multiplied by an exact power of
    two, so neither do its codes: tiny rows (where the fp32 inverse 448 / absmax
    would overflow) get the codes of the same row lifted into the normal range,
    and ordinary rows keep theirs under 2^-40 .. 2^40."""
    rng = np.random.default_rng(7)
    y = _tiny_rows(rng)
    lifted = (y.astype(np.float64) * 2.0 ** 100).astype(np.float32)
    assert np.array_equal(lifted.astype(np.float64) * 2.0 ** -100, y.astype(np.float64))   # exact
    c0, _ = oracle.quant_rows(y)
    c1, _ = oracle.quant_rows(lifted)
    assert np.array_equal(c0, c1)
    z = (rng.standard_normal((500, 128)) * rng.uniform(0.01, 100, (500, 1))).astype(np.float32)
    cz, _ = oracle.quant_rows(z)
    for k in (-40, -13, 5, 40):
        zk = (z.astype(np.float64) * 2.0 ** k).astype(np.float32)
        assert np.array_equal(oracle.quant_rows(zk)[0], cz), k
