"""Pins of the fp8 half of the oracle (CPU only).

The e4m3 codec is checked exhaustively against torch's float8_e4m3fn (a library
routine implementing the same OCP format); the Hadamard matrix against its
closed form H[i, j] = (-1)^popcount(i & j) / sqrt(d); the rotation against the
invariance of Q K^T; quantisation against its error bound.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F8.e4m3_value(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref[~nan])
    assert F8.e4m3_value(0x7E) == 448.0 and F8.e4m3_value(0x08) == 2.0 ** -6 and F8.e4m3_value(1) == 2.0 ** -9


def test_encode_matches_torch_rne_inside_range():
    vals = F8.e4m3_value(np.arange(0x7F))
    mids = (vals[1:] + vals[:-1]) / 2
    eps = np.nextafter(mids, np.inf) - mids
    pts = np.concatenate([vals, mids, mids + eps, mids - eps,
                          np.random.default_rng(0).uniform(0, 448, 20000),
                          np.random.default_rng(1).uniform(0, 0.02, 20000)])
    pts = np.concatenate([pts, -pts])
    pts = pts[np.abs(pts) <= 448]
    # torch rounds float32 -> e4m3; keep the points float32-exact so both see the same value
    pts32 = pts.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(pts32.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F8.e4m3_code(pts32)
    assert np.array_equal(ours, ref)


def test_encode_saturates_and_keeps_nan():
    assert F8.e4m3_code(1e9) == 0x7E and F8.e4m3_code(-1e9) == 0xFE
    assert F8.e4m3_code(460.0) == 0x7E          # 448 < x < 464: nearest is 448
    assert F8.e4m3_code(np.nan) == 0x7F
    assert F8.e4m3_round(1.0625) == 1.0         # tie -> even mantissa
    assert F8.e4m3_round(1.1875) == 1.25


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_hadamard_closed_form_and_orthogonality(d):
    H = F8.hadamard(d)
    i = np.arange(d)
    pop = np.vectorize(lambda x: bin(x).count("1"))(i[:, None] & i[None, :])
    np.testing.assert_array_equal(H, ((-1.0) ** pop) / np.sqrt(d))
    np.testing.assert_allclose(H @ H.T, np.eye(d), atol=1e-14)


def test_rotation_preserves_scores_and_attention():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 40, 128))
    k = rng.standard_normal((1, 2, 40, 128))
    v = rng.standard_normal((1, 2, 40, 128))
    signs = rng.integers(0, 2, 128) * 2 - 1
    qr, kr = F8.rotate(q, signs), F8.rotate(k, signs)
    np.testing.assert_allclose(qr @ kr.transpose(0, 1, 3, 2), q @ k.transpose(0, 1, 3, 2), atol=1e-11)
    O, L = A.attention(q, k, v, 0.1)
    O2, L2 = A.attention(qr, kr, v, 0.1)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L, atol=1e-12)
    # a wrong sign vector breaks the invariance (the signs must be applied to both sides)
    q_bad = F8.rotate(q, -signs)
    assert np.abs(q_bad @ kr.transpose(0, 1, 3, 2) - q @ k.transpose(0, 1, 3, 2)).max() > 1.0


def test_rotation_spreads_an_outlier_channel():
    x = np.zeros((1, 1, 1, 128)); x[..., 5] = 20.0
    signs = np.ones(128)
    r = F8.rotate(x, signs)
    np.testing.assert_allclose(np.abs(r), 20.0 / np.sqrt(128), atol=1e-12)


def test_quantize_error_bound_and_scale():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 300, 16)) * rng.uniform(0.01, 30, (2, 3, 1, 1))
    codes, scales = F8.quantize_rows(x, 128)
    assert scales.shape == (2, 3, 3) and scales.dtype == np.float32
    for t in range(3):
        blk = x[:, :, t * 128:(t + 1) * 128]
        np.testing.assert_array_equal(scales[:, :, t],
                                      (np.abs(blk).max(axis=(2, 3)) / 448.0).astype(np.float32))
    back = F8.dequantize_rows(codes, scales, 128)
    sc = np.repeat(scales.astype(np.float64), 128, axis=2)[:, :, :300, None]
    # relative half-step bound of e4m3 (3 mantissa bits) on normals, absolute on subnormals
    err = np.abs(back - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the tile maximum maps exactly onto +-448 * scale (up to the float32 rounding of the scale)
    assert np.all(np.isin(F8.e4m3_value(codes).max(axis=(2, 3)), [448.0]) |
                  np.isin(F8.e4m3_value(codes).min(axis=(2, 3)), [-448.0]))


def test_emulation_error_is_bounded_and_hadamard_helps():
    """The fp8 emulation's error against the exact oracle stays within the e4m3 bound
    (3 mantissa bits: about sqrt(2) * 2^-4 / sqrt(3) relative score error per unit-variance
    head, more where outliers inflate |q| |k|), and rotating Q, K lowers it on inputs with
    outlier entries (the page's claim, a ratio > 1 here)."""
    ratio = json.load(open(os.path.join(GOLDEN, "fp8_error_ratio.json")))
    rng = np.random.default_rng(9)
    B, H, N, d = 1, 2, 512, 128
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    for t in (q, k, v):
        idx = rng.choice(t.size, int(ratio["outlier_fraction"] * t.size), replace=False)
        t.reshape(-1)[idx] *= 20.0
    signs = rng.integers(0, 2, d) * 2 - 1
    scale = 1 / np.sqrt(d)
    O, _ = A.attention(q, k, v, scale)
    O = O.reshape(B * H, N, d)
    rel = lambda X: np.linalg.norm(X - O) / np.linalg.norm(O)
    # the page's setting: one e4m3 code per element of Q and K
    Oh, _ = F8.attention_emulated(q, k, v, signs, scale, rotate_qk=True, qk_codes=1)
    On, _ = F8.attention_emulated(q, k, v, signs, scale, rotate_qk=False, qk_codes=1)
    assert rel(Oh) < 0.1
    assert rel(On) / rel(Oh) > 1.2
    # value + residual codes remove most of the Q / K rounding error: what is left
    # is V's codes and P's rounding (each about 2^-4 / sqrt(3) * 0.7 relative)
    O2, _ = F8.attention_emulated(q, k, v, signs, scale, rotate_qk=True, qk_codes=2)
    assert rel(O2) < 0.05 and rel(O2) < 0.8 * rel(Oh)


def test_emulation_with_identity_codec_equals_exact():
    """With quantisation bypassed (all values already on the e4m3 grid and p_shift large
    enough that p lands on the grid only when exactly representable) the emulation's
    online-softmax walk reproduces the exact attention on grid-valued inputs."""
    rng = np.random.default_rng(11)
    grid = F8.e4m3_value(np.arange(0x30, 0x48))        # values in [0.125, 4)
    q = rng.choice(grid, (1, 1, 64, 128)) * rng.choice([-1, 1], (1, 1, 64, 128))
    k = np.zeros((1, 1, 64, 128))                        # all scores 0 -> p = 1 exactly
    v = rng.choice(grid, (1, 1, 64, 128)) * rng.choice([-1, 1], (1, 1, 64, 128))
    O, L = A.attention(q, k, v, 0.1)
    # per-tile scales keep the grid only if amax is a power of two times 448: normalise v
    Oe, Le = F8.attention_emulated(q, k, v, np.ones(128), 0.1, rotate_qk=False, block_n=16)
    np.testing.assert_allclose(Le, L.reshape(1, 64), atol=1e-12)
    np.testing.assert_allclose(Oe, O.reshape(1, 64, 128), atol=0.02 * np.abs(v).max())


def test_split_codes_residual_and_error():
    """value + residual codes on one tile scale: the residual is the rounding error
    of the value code rounded again, so the pair's error is the residual's own
    rounding error, at most half an e4m3 step of the residual (<= 2^-4 of it,
    or 2^-10 on the subnormal grid) -- about 2^-8 of the element instead of 2^-4."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 2, 260, 32)) * rng.uniform(0.1, 10, (2, 2, 1, 1))
    x[0, 1, 5, 3] *= 20.0
    c1, c2, sc = F8.quantize_rows_split(x)
    c1b, scb = F8.quantize_rows(x)
    np.testing.assert_array_equal(c1, c1b)
    np.testing.assert_array_equal(sc, scb)
    rep = np.repeat(sc.astype(np.float64), 128, axis=2)[:, :, :260, None]
    t = x / rep
    r = t - F8.e4m3_value(c1)
    err = np.abs(F8.e4m3_value(c1) + F8.e4m3_value(c2) - t)
    assert np.all(err <= np.maximum(np.abs(r) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-9))
    # the residual never needs more than the value code's half step: |c2| <= 16 < 448
    assert np.abs(F8.e4m3_value(c2)).max() <= 16.0
    big = np.abs(t) > 1.0
    assert np.median(err[big] / np.abs(t[big])) < 2.0 ** -8


@pytest.mark.parametrize("split,tau,rotate", [(True, None, True), (True, 4 * np.log(2), True),
                                              (False, 4 * np.log(2), True), (True, None, False)])
def test_emulation_matches_brute_force(split, tau, rotate):
    """The fp8 emulation (numpy) against an independent pure-Python brute force of
    the same scheme (tests/brute_fp8.py: e4m3 rounding by exponent and step, the
    closed-form Hadamard, per-element loops): rotation, tile scales, value and
    residual codes, the reference schedule and the rounding of P all agree."""
    from tests import brute_fp8 as BF
    rng = np.random.default_rng(23)
    N, d, tile, block = 22, 8, 8, 4
    q = rng.standard_normal((1, 1, N, d)) * 2
    k = rng.standard_normal((1, 1, N, d)) * 2
    v = rng.standard_normal((1, 1, N, d))
    q[..., 3] *= 20.0
    v[0, 0, 9] *= 20.0                      # an outlier V token: its tile has the largest scale
    signs = rng.integers(0, 2, d) * 2 - 1
    scale = 0.7
    Oe, Le = F8.attention_emulated(q, k, v, signs, scale, block_n=block, tile=tile, lazy_tau=tau,
                                   qk_codes=2 if split else 1, rotate_qk=rotate)
    Ob, Lb = BF.attend_fp8(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), [float(x) for x in signs],
                           scale, tile, block, tau=tau, split=split, rotate=rotate)
    np.testing.assert_allclose(Oe[0], np.array(Ob), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(Le[0], np.array(Lb), rtol=0, atol=1e-12)
    # and the scheme differs from the exact result by an fp8-sized amount, not 0
    O, _ = A.attention(q, k, v, scale)
    assert np.abs(Oe[0] - O[0, 0]).max() > 1e-4


def test_brute_force_e4m3_matches_codec():
    """The brute force's rounding equals the oracle codec on every code, every
    midpoint and points around them (so the brute-force pin is not vacuous)."""
    from tests import brute_fp8 as BF
    vals = F8.e4m3_value(np.arange(0x7F))
    mids = (vals[1:] + vals[:-1]) / 2
    pts = np.concatenate([vals, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                          np.random.default_rng(2).uniform(-500, 500, 2000)])
    ours = np.array([BF.e4m3(float(x)) for x in pts])
    np.testing.assert_array_equal(ours, F8.e4m3_round(pts))
