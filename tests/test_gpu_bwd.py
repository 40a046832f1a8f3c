"""GPU parity of attn_bwd (dQ, dK, dV) against the float64 backward oracle.

Bar (derived from the arithmetic: P and dS enter the products rounded to bf16,
2^-9 relative, and the outputs are stored in bf16): per gradient, the largest
error at most 2e-2 of max(largest reference magnitude, 1) and the mean error at
most 1e-2 of max(mean reference magnitude, 0.1) -- unit-normal inputs give O(1)
gradients, and the floors keep the bar meaningful where a reference vanishes. The forward of the same call
provides O and the LSE.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from tiled_attention_05_amd import _lib
from tiled_attention_05_amd import inputs as I

pytestmark = pytest.mark.gpu


def _close(g, ref, label):
    # inputs are unit normal, so gradients are O(1); the floors make the bar
    # absolute where a reference vanishes (dQ of a single key is exactly 0)
    g = g.float().cpu().double().numpy()
    err = np.abs(g - ref)
    mx = err.max() / max(np.abs(ref).max(), 1.0)
    mn = err.mean() / max(np.abs(ref).mean(), 0.1)
    print(f"[parity-bwd] {label}: max-err/max-ref {mx:.3e}, mean-err/mean-ref {mn:.3e}", flush=True)
    assert mx <= 2e-2 and mn <= 1e-2, label


# the last two have 16 and 32 heads: their grids are dispatched in head groups per XCD
CASES = [(1, 2, 2, 64, 0), (1, 2, 2, 200, 1), (2, 4, 2, 300, 1), (1, 8, 1, 257, 0), (1, 2, 2, 1, 1),
         (1, 4, 4, 1000, 1), (2, 8, 8, 300, 1), (1, 32, 16, 200, 0)]


@pytest.mark.parametrize("B,Hq,Hkv,N,mask", CASES, ids=[f"{c[1]}x{c[2]}-N{c[3]}-m{c[4]}" for c in CASES])
def test_bwd_matches_oracle(B, Hq, Hkv, N, mask):
    print(f"[case] bwd B={B} Hq={Hq} Hkv={Hkv} N={N} mask={mask}", flush=True)
    g = torch.Generator("cpu").manual_seed(N + Hq)
    q = torch.randn(B, Hq, N, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, N, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, 128, generator=g).to(torch.bfloat16)
    do = torch.randn(B, Hq, N, 128, generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = _lib.fwd(qd, kd, vd, mask=mask)
    dq, dk, dv = _lib.bwd(qd, kd, vd, o, dod, lse, mask=mask)
    torch.cuda.synchronize()
    # the oracle's gradient of the exact forward (its O from the same exact inputs)
    dQ, dK, dV = A.attention_backward(q, k, v, do, 128 ** -0.5, mask)
    _close(dq, dQ, f"dQ N={N}")
    _close(dk, dK, f"dK N={N}")
    _close(dv, dV, f"dV N={N}")


def test_bwd_is_deterministic():
    g = torch.Generator("cpu").manual_seed(3)
    q, do = (torch.randn(1, 4, 500, 128, generator=g).to(torch.bfloat16).cuda() for _ in range(2))
    k, v = (torch.randn(1, 2, 500, 128, generator=g).to(torch.bfloat16).cuda() for _ in range(2))
    o, lse = _lib.fwd(q, k, v, mask=I.MASK_CAUSAL)
    a = _lib.bwd(q, k, v, o, do, lse, mask=I.MASK_CAUSAL)
    b = _lib.bwd(q, k, v, o, do, lse, mask=I.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_bwd_full_workload_sampled_heads():
    """The backward at the benchmarked shape and call (causal B=4 H=32 N=4096 d=128, the
    same inputs and output gradient as the benchmark, dispatched in XCD head groups),
    checked on sampled (batch, head) pairs. With as many key/value heads as query heads
    a head's gradients depend on that head alone, so the oracle runs one head at a time."""
    w = I.WORKLOADS[8]
    assert w.Hq == w.Hkv
    print(f"[case] bwd full workload B={w.B} H={w.Hq} N={w.N}", flush=True)
    x = I.inputs(w)
    g = torch.Generator("cpu").manual_seed(2000 + w.k)
    q, k, v = x["q"], x["k"], x["v"]
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = _lib.fwd(qd, kd, vd, scale=w.scale, mask=w.mask)
    dq, dk, dv = _lib.bwd(qd, kd, vd, o, dod, lse, scale=w.scale, mask=w.mask)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (1, 17), (w.B - 1, w.Hq - 1)]:
        s = (slice(b, b + 1), slice(h, h + 1))
        dQ, dK, dV = A.attention_backward(q[s], k[s], v[s], do[s], w.scale, w.mask)
        _close(dq[s], dQ, f"dQ b={b} h={h}")
        _close(dk[s], dK, f"dK b={b} h={h}")
        _close(dv[s], dV, f"dV b={b} h={h}")


def test_bwd_seeded_sweep():
    """24 seeded random shapes (batch, GQA ratio, ragged lengths, dense or
    causal) against the float64 backward oracle to the bar above."""
    import random
    rng = random.Random(8)
    for c in range(24):
        hkv = rng.choice([1, 2, 4])
        B, Hq, N, mask = rng.choice([1, 2]), hkv * rng.choice([1, 2, 4]), rng.choice([1, 31, 33, 128, 255, 400, 700]), \
            rng.choice([0, 1])
        print(f"[case] bwd sweep {c}: B={B} Hq={Hq} Hkv={hkv} N={N} mask={mask}", flush=True)
        g = torch.Generator("cpu").manual_seed(500 + c)
        q = torch.randn(B, Hq, N, 128, generator=g).to(torch.bfloat16)
        k = torch.randn(B, hkv, N, 128, generator=g).to(torch.bfloat16)
        v = torch.randn(B, hkv, N, 128, generator=g).to(torch.bfloat16)
        do = torch.randn(B, Hq, N, 128, generator=g).to(torch.bfloat16)
        qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
        o, lse = _lib.fwd(qd, kd, vd, mask=mask)
        dq, dk, dv = _lib.bwd(qd, kd, vd, o, dod, lse, mask=mask)
        torch.cuda.synchronize()
        dQ, dK, dV = A.attention_backward(q, k, v, do, 128 ** -0.5, mask)
        _close(dq, dQ, f"sweep {c} dQ")
        _close(dk, dK, f"sweep {c} dK")
        _close(dv, dV, f"sweep {c} dV")
