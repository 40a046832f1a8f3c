"""Pins of the float64 oracle against things other than itself (CPU only).

Brute force on tiny inputs, closed forms, invariants, and library routines
that reduce to a special case (torch's scaled_dot_product_attention on the CPU
in float64).  Each check is chosen so that a plausible slip in the oracle -- a
dropped term, a wrong sign or index, a transposed operand, an off-by-one in a
mask -- fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from tests import brute

C, W, D = A.MASK_CAUSAL, A.MASK_WINDOW, A.MASK_DOC


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _tolist(x):
    return np.asarray(x).tolist()


# ---------------------------------------------------------------- brute force
CASES = []
for (hq, hkv), mask, softcap, alibi in itertools.product(
        [(2, 2), (4, 2), (4, 1)], [0, C, C | W, D, D | C], [0.0, 2.5], [False, True]):
    CASES.append((hq, hkv, mask, softcap, alibi))


@pytest.mark.parametrize("hq,hkv,mask,softcap,alibi", CASES)
def test_brute_force_tiny(hq, hkv, mask, softcap, alibi):
    B, N, d = 2, 11, 5
    q = _rand((B, hq, N, d), 1)
    k = _rand((B, hkv, N, d), 2)
    v = _rand((B, hkv, N, d), 3)
    docs = np.array([[0, 0, 0, 1, 1, 2, 2, 2, 2, 3, 3], [0, 1, 1, 1, 1, 1, 2, 2, 3, 3, 3]])
    slopes = np.array([0.5, 0.25, 0.125, 0.0625])[:hq] if alibi else None
    window = 3 if mask & W else 0
    scale = 0.7
    O, L = A.attention(q, k, v, scale, mask, window, docs if mask & D else None, softcap, slopes,
                       threads=1)
    Ob, Lb = brute.attend(_tolist(q), _tolist(k), _tolist(v), scale, causal=bool(mask & C),
                          window=window, docs=_tolist(docs) if mask & D else None,
                          softcap=softcap, slopes=None if slopes is None else list(slopes))
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-13)


@pytest.mark.parametrize("Nq,Nk", [(3, 9), (9, 9), (9, 3)])
def test_brute_force_rectangular_causal(Nq, Nk):
    """Causal with Nq != Nk aligns bottom-right; with Nq > Nk the first rows see nothing."""
    q = _rand((1, 2, Nq, 4), 4)
    k = _rand((1, 2, Nk, 4), 5)
    v = _rand((1, 2, Nk, 4), 6)
    O, L = A.attention(q, k, v, 0.5, C, threads=1)
    Ob, Lb = brute.attend(_tolist(q), _tolist(k), _tolist(v), 0.5, causal=True)
    np.testing.assert_allclose(O, np.array(Ob), atol=1e-13)
    np.testing.assert_allclose(L, np.array(Lb), atol=1e-13)
    if Nq > Nk:
        assert np.all(np.isneginf(L[..., :Nq - Nk])) and np.all(O[..., :Nq - Nk, :] == 0)


# ---------------------------------------------------------------- closed forms (Q = 0)
def _zero_q(B, H, N, d, seed=7):
    return np.zeros((B, H, N, d)), _rand((B, H, N, d), seed), _rand((B, H, N, d), seed + 1)


def test_closed_form_dense():
    q, k, v = _zero_q(1, 2, 37, 8)
    O, L = A.attention(q, k, v, 0.3)
    np.testing.assert_allclose(L, np.log(37.0), atol=1e-14)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=1e-14)


def test_closed_form_causal_prefix_mean():
    q, k, v = _zero_q(1, 2, 37, 8)
    O, L = A.attention(q, k, v, 0.3, C)
    i = np.arange(37)
    np.testing.assert_allclose(L, np.broadcast_to(np.log(i + 1.0), L.shape), atol=1e-14)
    prefix = np.cumsum(v, axis=2) / (i + 1.0)[None, None, :, None]
    np.testing.assert_allclose(O, prefix, atol=1e-13)


@pytest.mark.parametrize("Wn", [1, 5, 16, 100])
def test_closed_form_window(Wn):
    """A window of W keys: row i sees min(i + 1, W) keys (the diagonal included)."""
    q, k, v = _zero_q(1, 1, 40, 4)
    O, L = A.attention(q, k, v, 1.0, C | W, window=Wn)
    i = np.arange(40)
    np.testing.assert_allclose(L[0, 0], np.log(np.minimum(i + 1, Wn)), atol=1e-14)
    lo = np.maximum(0, i - Wn + 1)
    ref = np.stack([v[0, 0, lo[r]:r + 1].mean(axis=0) for r in range(40)])
    np.testing.assert_allclose(O[0, 0], ref, atol=1e-13)


def test_closed_form_document_causal():
    docs = np.array([[0] * 5 + [1] * 9 + [2] * 3 + [3] * 13])
    q, k, v = _zero_q(1, 1, 30, 4)
    _, L = A.attention(q, k, v, 1.0, C | D, doc_ids=docs)
    start = np.array([0] * 5 + [5] * 9 + [14] * 3 + [17] * 13)
    np.testing.assert_allclose(L[0, 0], np.log(np.arange(30) - start + 1.0), atol=1e-14)
    _, L2 = A.attention(q, k, v, 1.0, D, doc_ids=docs)       # non-causal: whole document
    size = np.array([5] * 5 + [9] * 9 + [3] * 3 + [13] * 13)
    np.testing.assert_allclose(L2[0, 0], np.log(size), atol=1e-14)


def test_closed_form_causal_alibi_geometric():
    """Scores -s (i - j) on j <= i: lse_i = ln((1 - e^{-s(i+1)}) / (1 - e^{-s}))."""
    s = 2 ** -0.5
    q, k, v = _zero_q(1, 1, 30, 4)
    _, L = A.attention(q, k, v, 1.0, C, alibi_slopes=np.array([s]))
    i = np.arange(30)
    ref = np.log((1 - np.exp(-s * (i + 1))) / (1 - np.exp(-s)))
    np.testing.assert_allclose(L[0, 0], ref, atol=1e-13)
    # spot value checked by hand: i = 10
    assert abs(L[0, 0, 10] - math.log(sum(math.exp(-s * t) for t in range(11)))) < 1e-13


def test_softcap_fixes_zero_and_caps():
    q, k, v = _zero_q(1, 1, 20, 4)
    _, L = A.attention(q, k, v, 1.0, 0, softcap=50.0)
    np.testing.assert_allclose(L, np.log(20.0), atol=1e-14)
    # a huge raw score is capped to ~cap: one key with score 1e4 vs zeros
    q = np.zeros((1, 1, 1, 2)); q[..., 0] = 1.0
    k = np.zeros((1, 1, 3, 2)); k[0, 0, 0, 0] = 1e4
    v = np.zeros((1, 1, 3, 2))
    _, L = A.attention(q, k, v, 1.0, 0, softcap=3.0)
    ref = math.log(math.exp(3.0 * math.tanh(1e4 / 3.0)) + 2.0)
    assert abs(L[0, 0, 0] - ref) < 1e-13


# ---------------------------------------------------------------- invariants
def test_probability_rows_sum_to_one():
    q = _rand((1, 1, 50, 16), 11)
    k = _rand((1, 1, 50, 16), 12)
    s = A.scores(q[0, 0], k[0, 0], np.arange(50), 50, 50, 0.25, softcap=5.0, slope=0.1)
    for mask in (0, C, C | W):
        ok = A.allowed_mask(np.arange(50), np.arange(50), 50, 50, mask, 7)
        p, _, _ = A.probabilities(s, ok)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
        assert np.all(p[~ok] == 0)


def test_constant_v_gives_that_row():
    q = _rand((2, 2, 33, 8), 13)
    k = _rand((2, 2, 33, 8), 14)
    row = _rand((8,), 15)
    v = np.broadcast_to(row, (2, 2, 33, 8)).copy()
    for mask in (0, C, C | W):
        O, _ = A.attention(q, k, v, 0.4, mask, window=4, softcap=7.0, alibi_slopes=np.array([0.3, 0.1]))
        np.testing.assert_allclose(O, np.broadcast_to(row, O.shape), atol=1e-13)


def test_one_hot_dominant_score_selects_one_row():
    rng = np.random.default_rng(16)
    N, d, scale = 64, 32, 1 / math.sqrt(32)
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d)) * 0.05      # other scores of row i stay far below 10
    v = rng.standard_normal((1, 1, N, d))
    i, jstar = 40, 17
    qi = q[0, 0, i]
    k[0, 0, jstar] = (60.0 / scale) * qi / (qi @ qi)
    O, L = A.attention(q, k, v, scale)
    s = scale * (k[0, 0] @ qi)
    others = np.delete(s, jstar)
    assert abs(s[jstar] - 60.0) < 1e-9 and others.max() < 10.0
    assert np.abs(O[0, 0, i] - v[0, 0, jstar]).max() < N * math.exp(-50) * 10
    assert abs(L[0, 0, i] - 60.0) < 1e-12


@pytest.mark.parametrize("block", [1, 7, 64, 128, 200])
@pytest.mark.parametrize("mask,softcap,alibi", [(0, 0.0, False), (C, 0.0, False), (C | W, 4.0, True),
                                                  (C | D, 50.0, True)])
def test_tiled_equals_untiled(block, mask, softcap, alibi):
    B, H, N, d = 1, 2, 200, 16
    q = _rand((B, H, N, d), 20)
    k = _rand((B, H, N, d), 21)
    v = _rand((B, H, N, d), 22)
    docs = np.repeat(np.arange(5), [30, 70, 1, 60, 39])[None, :]
    slopes = np.array([0.25, 2 ** -5]) if alibi else None
    kw = dict(mask_kind=mask, window=37, doc_ids=docs if mask & D else None, softcap=softcap,
              alibi_slopes=slopes)
    O1, L1 = A.attention(q, k, v, 0.3, **kw)
    O2, L2 = A.attention_tiled(q, k, v, 0.3, block, **kw)
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    np.testing.assert_allclose(L2, L1, atol=1e-12)


def test_gqa_equals_repeated_heads():
    q = _rand((2, 8, 25, 8), 30)
    k = _rand((2, 2, 25, 8), 31)
    v = _rand((2, 2, 25, 8), 32)
    O, L = A.attention(q, k, v, 0.5, C)
    O2, L2 = A.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.5, C)
    np.testing.assert_allclose(O, O2, atol=1e-14)
    np.testing.assert_allclose(L, L2, atol=1e-14)
    # and a different grouping would differ: head 1 must read kv head 0, not kv head 1
    O3, _ = A.attention(q[:, :2], k, v, 0.5, C)
    assert np.abs(O3[:, 1] - O[:, 1]).max() > 1e-3


def test_joint_key_value_permutation_invariance():
    q = _rand((1, 2, 30, 8), 40)
    k = _rand((1, 2, 30, 8), 41)
    v = _rand((1, 2, 30, 8), 42)
    perm = np.random.default_rng(43).permutation(30)
    O, L = A.attention(q, k, v, 0.5, softcap=3.0)
    O2, L2 = A.attention(q, k[:, :, perm], v[:, :, perm], 0.5, softcap=3.0)
    np.testing.assert_allclose(O, O2, atol=1e-13)
    np.testing.assert_allclose(L, L2, atol=1e-13)


def test_row_shift_moves_lse_only():
    """Adding c_i to every score of row i shifts lse_i by c_i and leaves O unchanged."""
    q = _rand((1, 1, 30, 9), 50)
    k = _rand((1, 1, 30, 9), 51)
    v = _rand((1, 1, 30, 9), 52)
    q[..., -1] = 0.0
    k[..., -1] = 1.0
    O, L = A.attention(q, k, v, 0.5, C)
    c = _rand((30,), 53) * 3
    q2 = q.copy()
    q2[0, 0, :, -1] = c / 0.5
    O2, L2 = A.attention(q2, k, v, 0.5, C)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2[0, 0], L[0, 0] + c, atol=1e-13)


def test_huge_softcap_equals_no_cap():
    q = _rand((1, 2, 30, 8), 60)
    k = _rand((1, 2, 30, 8), 61)
    v = _rand((1, 2, 30, 8), 62)
    O, L = A.attention(q, k, v, 0.5, C)
    O2, L2 = A.attention(q, k, v, 0.5, C, softcap=1e6)
    np.testing.assert_allclose(O2, O, atol=1e-9)
    np.testing.assert_allclose(L2, L, atol=1e-9)


def test_alibi_sign_penalises_distance():
    """With a positive slope, far keys lose weight: lse drops below the no-bias value."""
    q, k, v = _zero_q(1, 1, 10, 2)
    _, L0 = A.attention(q, k, v, 1.0, C)
    _, L1 = A.attention(q, k, v, 1.0, C, alibi_slopes=np.array([0.5]))
    assert np.all(L1[0, 0, 1:] < L0[0, 0, 1:]) and abs(L1[0, 0, 0] - L0[0, 0, 0]) < 1e-15


# ---------------------------------------------------------------- library special case
def _sdpa_ref(q, k, v, scale, ok, bias=None):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    mask = torch.from_numpy(ok)
    if bias is not None:
        m = torch.where(mask, torch.from_numpy(bias), torch.tensor(-math.inf, dtype=torch.float64))
    else:
        m = mask
    return F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale,
                                          enable_gqa=True).numpy()


@pytest.mark.parametrize("mask", [0, C, C | W, C | D])
@pytest.mark.parametrize("alibi", [False, True])
def test_matches_torch_sdpa_float64(mask, alibi):
    B, Hq, Hkv, N, d = 1, 4, 2, 64, 16
    q = _rand((B, Hq, N, d), 70)
    k = _rand((B, Hkv, N, d), 71)
    v = _rand((B, Hkv, N, d), 72)
    docs = np.repeat(np.arange(3), [20, 30, 14])[None, :]
    slopes = np.array([0.5, 0.25, 0.1, 0.05]) if alibi else None
    O, L = A.attention(q, k, v, 0.25, mask, window=9, doc_ids=docs if mask & D else None,
                       alibi_slopes=slopes)
    i = np.arange(N)
    ok = np.ones((N, N), dtype=bool)
    if mask & C:
        ok &= i[None, :] <= i[:, None]
    if mask & W:
        ok &= i[:, None] - i[None, :] < 9
    if mask & D:
        ok &= docs[0][:, None] == docs[0][None, :]
    if alibi:
        bias = -(slopes[None, :, None, None] * (i[:, None] - i[None, :])[None, None]).repeat(B, 0)
        ref = _sdpa_ref(q, k, v, 0.25, np.broadcast_to(ok, (B, Hq, N, N)), bias)
    else:
        ref = _sdpa_ref(q, k, v, 0.25, ok)
    np.testing.assert_allclose(O, ref, atol=1e-12)
    # LSE via torch.logsumexp over explicitly built scores
    kr = np.repeat(k, 2, axis=1)
    s = 0.25 * np.einsum("bhid,bhjd->bhij", q, kr)
    if alibi:
        s = s + bias
    s = np.where(ok, s, -np.inf)
    np.testing.assert_allclose(L, torch.logsumexp(torch.from_numpy(s), dim=-1).numpy(), atol=1e-12)
