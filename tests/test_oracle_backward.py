"""Pins of the backward oracle (``oracle.attention.attention_backward``).

* central finite differences of the forward oracle's loss sum(dO * O) with
  respect to every entry of Q, K and V (tiny sizes, GQA, dense and causal);
* torch autograd in float64 through an explicit softmax formula (a library
  routine independent of the oracle's hand-derived gradient), GQA and causal;
* a masked key gets zero dK and dV from the rows that cannot see it.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("mask", [0, 1])
def test_finite_differences(mask):
    B, Hq, Hkv, N, d = 1, 2, 1, 5, 3
    q, k, v = _rand((B, Hq, N, d), 1), _rand((B, Hkv, N, d), 2), _rand((B, Hkv, N, d), 3)
    do = _rand((B, Hq, N, d), 4)
    scale = 0.7
    dQ, dK, dV = A.attention_backward(q, k, v, do, scale, mask)

    def loss(q_, k_, v_):
        O, _ = A.attention(q_, k_, v_, scale, mask, threads=1)
        return float((O * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                        loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7, err_msg=name)


def test_matches_torch_autograd_float64():
    B, Hq, Hkv, N, d = 2, 4, 2, 9, 6
    t = {n: torch.tensor(_rand(s, i), dtype=torch.float64, requires_grad=True)
         for i, (n, s) in enumerate((("q", (B, Hq, N, d)), ("k", (B, Hkv, N, d)), ("v", (B, Hkv, N, d))))}
    do = torch.tensor(_rand((B, Hq, N, d), 9), dtype=torch.float64)
    scale = 0.45
    kk = t["k"].repeat_interleave(Hq // Hkv, dim=1)
    vv = t["v"].repeat_interleave(Hq // Hkv, dim=1)
    s = scale * t["q"] @ kk.transpose(-1, -2)
    s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    O = torch.softmax(s, dim=-1) @ vv
    (O * do).sum().backward()
    dQ, dK, dV = A.attention_backward(t["q"].detach().numpy(), t["k"].detach().numpy(), t["v"].detach().numpy(),
                                      do.numpy(), scale, 1)
    np.testing.assert_allclose(dQ, t["q"].grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, t["k"].grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, t["v"].grad.numpy(), rtol=0, atol=1e-12)


def test_last_key_gets_gradient_only_from_the_last_row_under_causal():
    B, H, N, d = 1, 1, 6, 4
    q, k, v = _rand((B, H, N, d), 5), _rand((B, H, N, d), 6), _rand((B, H, N, d), 7)
    do = np.zeros((B, H, N, d))
    do[0, 0, :-1] = _rand((N - 1, d), 8)          # the last row's output gradient is zero
    _, dK, dV = A.attention_backward(q, k, v, do, 0.5, 1)
    np.testing.assert_array_equal(dK[0, 0, -1], np.zeros(d))
    np.testing.assert_array_equal(dV[0, 0, -1], np.zeros(d))
