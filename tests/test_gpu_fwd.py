"""GPU parity of the fused forward against the float64 oracle (through the C ABI).

Small cases span several query / key tiles with ragged tails and run the whole
oracle; the full workloads (in the launch configuration the benchmark times)
are checked on every row of three heads per batch row. Bars: max-abs 2e-2, mean-abs
2e-3 on O, 1e-3 on LSE (the fp32 workload also meets 1e-4).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.gpu_util import assert_close, oracle, oracle_whole_heads, run_fwd, to_dev
from tiled_attention_05_amd import _lib
from tiled_attention_05_amd import inputs as I

pytestmark = pytest.mark.gpu

C, W, D = I.MASK_CAUSAL, I.MASK_WINDOW, I.MASK_DOC


def _case(w, seed=None, doc_range=None):
    x = I.inputs(w, seed)
    if doc_range is not None:
        g = torch.Generator("cpu").manual_seed(77 + w.N)
        rows = []
        for _ in range(w.B):
            lens = I.doc_lengths(w.N, g, *doc_range)
            rows.append(torch.repeat_interleave(torch.arange(len(lens), dtype=torch.int32), torch.tensor(lens)))
        x["doc_ids"] = torch.stack(rows)
    return x


def _check(w, x, label, **kw):
    print(f"[case] {label} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} mask={w.mask}", flush=True)
    o, lse = run_fwd(x, w.mask, w.window, w.softcap)
    O, L = oracle(x, w.scale, w.mask, w.window, w.softcap)
    return assert_close(o, lse, O, L, label=label, **kw)


def test_tiny_dense_fp32_workload():
    w = I.WORKLOADS[1]
    x = I.inputs(w)
    _check(w, x, "fp32 workload")
    o, lse = run_fwd(x, w.mask)
    O, L = oracle(x, w.scale, w.mask)
    assert_close(o, lse, O, L, max_abs=1e-4, mean_abs=1e-5, lse_tol=1e-5, label="fp32 workload tight")


SMALL = [
    ("causal d128", I.WORKLOADS[2].shrink(B=2, Hq=3, Hkv=3, N=1000), None),
    # 16 heads of 4 query tiles: the grid is dispatched two heads per XCD at a time
    ("causal 16 heads grouped", I.WORKLOADS[2].shrink(B=2, Hq=8, Hkv=8, N=1000), None),
    # grouped order with GQA: 8 key / value heads, their query heads placed 8 slots apart
    ("gqa 32 heads grouped", I.WORKLOADS[2].shrink(B=2, Hq=16, Hkv=4, N=900), None),
    ("dense d128", I.WORKLOADS[2].shrink(B=1, Hq=2, Hkv=2, N=777, mask=0), None),
    ("causal d64", I.WORKLOADS[2].shrink(B=1, Hq=2, Hkv=2, N=600, d=64), None),
    ("dense d64", I.WORKLOADS[2].shrink(B=1, Hq=2, Hkv=2, N=333, d=64, mask=0), None),
    ("gqa window", I.WORKLOADS[3].shrink(B=1, Hq=8, Hkv=2, N=1500, window=300), None),
    ("gqa window tiny W", I.WORKLOADS[3].shrink(B=1, Hq=4, Hkv=2, N=700, window=1), None),
    ("mqa causal", I.WORKLOADS[2].shrink(B=1, Hq=4, Hkv=1, N=520), None),
    ("docs softcap alibi", I.WORKLOADS[4].shrink(B=1, Hq=4, Hkv=4, N=2500), (64, 1024)),
    ("docs short", I.WORKLOADS[4].shrink(B=2, Hq=2, Hkv=2, N=900, softcap=0.0, alibi=False), (1, 40)),
    ("docs non-causal", I.WORKLOADS[4].shrink(B=2, Hq=2, Hkv=2, N=700, mask=D, softcap=0.0, alibi=False),
     (50, 300)),
    ("softcap dense", I.WORKLOADS[2].shrink(B=1, Hq=2, Hkv=2, N=400, mask=0, softcap=5.0), None),
    ("alibi causal", I.WORKLOADS[2].shrink(B=1, Hq=4, Hkv=4, N=400, alibi=True), None),
    ("window softcap d64", I.WORKLOADS[3].shrink(B=1, Hq=2, Hkv=1, N=500, d=64, window=77, softcap=3.0), None),
]


@pytest.mark.parametrize("label,w,docs", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(label, w, docs):
    _check(w, _case(w, doc_range=docs), label)


def test_softcap_polynomial_and_exact_tiles():
    """Soft-cap 50 with Q scaled by 6: 42 of the 980000 scores have
    |scale q.k| > 25, beyond the range of the kernel's polynomial form, so a
    few wave tiles take the exact form and the rest the polynomial in one
    launch."""
    w = I.WORKLOADS[2].shrink(B=1, Hq=2, Hkv=2, N=700, mask=0, softcap=50.0)
    x = I.inputs(w, seed=5)
    x["q"] = (x["q"].float() * 6).to(x["q"].dtype)
    s = (x["q"].float() @ x["k"].float().transpose(-1, -2)) * w.scale
    assert 0 < (s.abs() > 25).sum() < s.numel() // 1000
    _check(w, x, "softcap both forms")


def test_softcap_every_form():
    """Soft-cap 50 with the 32-row blocks of Q scaled by 1, 2.3, 4.5 and 8 in
    turn: the kernel picks its form per wave tile (32 rows x 64 keys) from the
    largest |scale q.k| of the tile -- degree-1 polynomial up to cap/8,
    degree-2 up to cap/4, degree-3 up to cap/2, the exact form beyond -- and
    every form is taken by some tile of this launch."""
    w = I.WORKLOADS[2].shrink(B=1, Hq=2, Hkv=2, N=512, mask=0, softcap=50.0)
    x = I.inputs(w, seed=9)
    f = torch.tensor([1.0, 2.3, 4.5, 8.0]).repeat(w.N // 128).repeat_interleave(32)
    x["q"] = (x["q"].float() * f[None, None, :, None]).to(x["q"].dtype)
    s = (x["q"].float() @ x["k"].float().transpose(-1, -2)) * w.scale
    tmax = s.abs().reshape(w.B, w.Hq, w.N // 32, 32, w.N // 64, 64).amax(dim=(3, 5))
    bands = [int(((tmax > lo) & (tmax <= hi)).sum()) for lo, hi in
             ((0, 6.25), (6.25, 12.5), (12.5, 25.0), (25.0, float("inf")))]
    print(f"[softcap forms] wave tiles per form (degree 1, 2, 3, exact): {bands}", flush=True)
    assert all(b > 0 for b in bands)
    _check(w, x, "softcap every form")


@pytest.mark.parametrize("N", [1, 5, 63, 64, 65, 255, 257])
@pytest.mark.parametrize("mask", [0, C])
def test_short_sequences(N, mask):
    w = I.WORKLOADS[2].shrink(B=1, Hq=2, Hkv=2, N=N, mask=mask)
    _check(w, I.inputs(w, seed=N), f"N={N} mask={mask}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Nq,Nk", [(300, 1000), (1000, 300), (64, 65)])
def test_rectangular_causal(dtype, Nq, Nk):
    g = torch.Generator("cpu").manual_seed(Nq * 7 + Nk)
    tq = torch.float32 if dtype == "f32" else torch.bfloat16
    x = {"q": torch.randn(1, 2, Nq, 64, generator=g).to(tq), "k": torch.randn(1, 2, Nk, 64, generator=g).to(tq),
         "v": torch.randn(1, 2, Nk, 64, generator=g).to(tq)}
    o, lse = run_fwd(x, C)
    O, L = oracle(x, 0.125, C)
    assert_close(o, lse, O, L, label=f"rect {dtype} {Nq}x{Nk}")
    if Nq > Nk:
        assert torch.all(o[:, :, :Nq - Nk].float() == 0)


@pytest.mark.parametrize("mask,docs", [(C | W, None), (C | D, (20, 200)), (0, None)])
def test_fp32_masks_and_mods(mask, docs):
    w = I.WORKLOADS[1].shrink(B=1, Hq=2, Hkv=1, N=300, d=64, mask=mask, window=50, softcap=4.0, alibi=True)
    x = _case(w, doc_range=docs)
    _check(w, x, f"fp32 mask={mask}", max_abs=1e-4, mean_abs=1e-5, lse_tol=1e-4)


def test_fp32_d128():
    w = I.WORKLOADS[1].shrink(B=1, Hq=2, Hkv=2, N=200, d=128, mask=C)
    _check(w, I.inputs(w), "fp32 d128", max_abs=1e-4, mean_abs=1e-5, lse_tol=1e-4)


# ------------------------------------------------------------------ full workloads, whole heads
@pytest.mark.parametrize("k", [2, 3, 4])
def test_full_workload_whole_heads(k):
    """The full workload in the benchmark's launch configuration; every row of
    heads {0, H/2, H-1} of every batch row against the oracle, and the whole
    output finite."""
    w = I.WORKLOADS[k]
    print(f"[case] full workload {k} {w.name}", flush=True)
    x = I.inputs(w)
    o, lse = run_fwd(x, w.mask, w.window, w.softcap)
    heads = [(b, h) for b in range(w.B) for h in sorted({0, w.Hq // 2, w.Hq - 1})]
    O, L = oracle_whole_heads(x, w, heads)
    og = torch.stack([o[b, h] for b, h in heads])
    lg = torch.stack([lse[b, h] for b, h in heads])
    assert_close(og, lg, O, L, label=f"workload {k}, {len(heads)} whole heads")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


# ------------------------------------------------------------------ determinism, capture, canaries
@pytest.mark.parametrize("growth", [5.0, 40.0])
@pytest.mark.parametrize("mask", [I.MASK_NONE, I.MASK_CAUSAL])
def test_scores_growing_along_keys(growth, mask):
    """Scores that grow along the keys (a ramp of `growth` log2 units over the
    sequence, through one channel), so that later key tiles exceed each row's
    exponent reference: by a few units (the exponents recomputed after the
    tile's row max, no reference moved) or by many (references moved and the
    output rescaled several times per row)."""
    w = I.WORKLOADS[2].shrink(B=1, Hq=4, Hkv=4, N=1500, mask=mask)
    x = I.inputs(w, seed=5)
    ramp = growth * torch.arange(w.N, dtype=torch.float64) / (w.N - 1) / (w.scale * math.log2(math.e))
    x["q"][..., 0] = 1.0
    x["k"][..., 0] = ramp.to(torch.bfloat16)
    _check(w, x, f"scores growing by {growth} log2 units along the keys, mask {mask}")


def test_bitwise_deterministic():
    w = I.WORKLOADS[2].shrink(B=2, Hq=4, Hkv=4, N=1100)
    x = I.inputs(w)
    outs = [run_fwd(x, w.mask) for _ in range(4)]
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_graph_capture_replays_match_eager():
    w = I.WORKLOADS[4].shrink(B=1, Hq=2, Hkv=2, N=1024)
    x = _case(w, doc_range=(100, 400))
    q, k, v, docs, sl = (to_dev(x[n]) for n in ("q", "k", "v", "doc_ids", "slopes"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device="cuda")
    kw = dict(scale=w.scale, mask=w.mask, doc_ids=docs, softcap=w.softcap, alibi_slopes=sl, out=o, lse=lse)
    o_ref, l_ref = _lib.fwd(q, k, v, **{**kw, "out": None, "lse": None})
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _lib.fwd(q, k, v, **kw)      # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _lib.fwd(q, k, v, **kw)
    for _ in range(3):
        o.fill_(7.0)
        lse.fill_(7.0)
        junk = torch.randn(1000, 1000, device="cuda") @ torch.randn(1000, 1000, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        del junk


def test_canaries_around_outputs_untouched():
    w = I.WORKLOADS[2].shrink(B=1, Hq=3, Hkv=3, N=333)
    x = I.inputs(w)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    n_o, n_l, pad = q.numel(), w.B * w.Hq * w.N, 4096
    ob = torch.full((n_o + 2 * pad,), 3.0, dtype=torch.bfloat16, device="cuda")
    lb = torch.full((n_l + 2 * pad,), 3.0, dtype=torch.float32, device="cuda")
    o = ob[pad:pad + n_o].view(q.shape)
    lse = lb[pad:pad + n_l].view(w.B, w.Hq, w.N)
    _lib.fwd(q, k, v, mask=w.mask, out=o, lse=lse)
    torch.cuda.synchronize()
    for buf, n in ((ob, n_o), (lb, n_l)):
        assert torch.all(buf[:pad].float() == 3.0) and torch.all(buf[pad + n:].float() == 3.0)
    O, L = oracle(x, w.scale, w.mask)
    assert_close(o, lse, O, L, label="canary case")


def test_lse_optional():
    w = I.WORKLOADS[2].shrink(B=1, Hq=2, Hkv=2, N=200)
    x = I.inputs(w)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o = _lib.fwd(q, k, v, mask=w.mask, with_lse=False)
    o2, _ = _lib.fwd(q, k, v, mask=w.mask)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


# ------------------------------------------------------------------ key-split (context-parallel) merge
def _merge(parts):
    """Exact merge of partial results over disjoint key sets: LSE = logsumexp of
    the partial LSEs, O = sum of exp(lse_s - LSE) O_s (rows without keys in a
    part carry LSE = -inf and weigh zero)."""
    lse = parts[0][1]
    for _, l in parts[1:]:
        lse = torch.logaddexp(lse, l)
    w = [torch.exp(l - lse).nan_to_num(0.0) for _, l in parts]
    o = sum(wi[..., None] * oi.float() for (oi, _), wi in zip(parts, w))
    return o, lse


@pytest.mark.parametrize("mask", [0, C])
def test_key_split_merge_matches_full(mask):
    """The key-sharded (context-parallel) form of the path on one GPU: K / V
    split in two key ranges, each processed by the kernel, partial (O, LSE)
    merged exactly; the result must meet the parity bar against the oracle on
    the unsplit inputs. Causal: the second range uses the kernel's
    bottom-right alignment (query i sees key j <= i); the first range is
    causal for queries before the split and dense after it."""
    w = I.WORKLOADS[2].shrink(B=1, Hq=4, Hkv=2, N=1000, mask=mask)
    split = 448
    print(f"[case] key split merge mask={mask} N={w.N} split={split}", flush=True)
    x = I.inputs(w)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    k1, v1 = k[:, :, :split].contiguous(), v[:, :, :split].contiguous()
    k2, v2 = k[:, :, split:].contiguous(), v[:, :, split:].contiguous()
    if mask == 0:
        first = _lib.fwd(q, k1, v1, scale=w.scale, mask=0)
    else:
        oa, la = _lib.fwd(q[:, :, :split].contiguous(), k1, v1, scale=w.scale, mask=C)
        ob, lb = _lib.fwd(q[:, :, split:].contiguous(), k1, v1, scale=w.scale, mask=0)
        first = (torch.cat([oa, ob], dim=2), torch.cat([la, lb], dim=2))
    second = _lib.fwd(q, k2, v2, scale=w.scale, mask=mask)
    torch.cuda.synchronize()
    o, lse = _merge([first, second])
    O, L = oracle(x, w.scale, mask)
    assert_close(o, lse, O, L, label=f"key split merge mask={mask}")


def test_binding_rejects_bad_shapes():
    """The binding checks every extent the kernels will touch before calling the
    library: a wrong doc_ids, slopes, out or lse shape raises ValueError."""
    w = I.WORKLOADS[2].shrink(B=2, Hq=4, Hkv=2, N=128)
    x = I.inputs(w)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    ids = torch.zeros(2, 128, dtype=torch.int32, device="cuda")
    bad = [dict(doc_ids=ids[:1], mask=C | D), dict(doc_ids=ids[:, :100].contiguous(), mask=C | D),
           dict(alibi_slopes=torch.ones(3, device="cuda")), dict(out=torch.empty_like(q)[:, :2]),
           dict(lse=torch.empty(2, 4, 100, device="cuda"))]
    for kw in bad:
        with pytest.raises(ValueError):
            _lib.fwd(q, k, v, **kw)
    o = torch.empty(2, 4, 128, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        _lib.fwd_fp8(torch.empty(100, dtype=torch.uint8, device="cuda"), q, q, 2, 4, 2, 128, 128, out=o)


_PERSIST_CHILD = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from tests.test_gpu_fwd import persistent_cases
outs = persistent_cases()
torch.save([(o.cpu(), l.cpu()) for o, l in outs], sys.argv[2])
"""


def persistent_cases():
    """Outputs of a few launches (causal, GQA + window, documents + mods, varlen).
    The last five have more work items than an MI355X has CUs (384 to 1024
    items, and over 300 list entries per head), so each persistent workgroup
    runs several items and reuses its LDS buffers (output staging included)
    from one item to the next (row counts not a multiple of the 256-row tile
    included)."""
    outs = []
    for w, docs in ((I.WORKLOADS[2].shrink(B=2, Hq=8, Hkv=8, N=1000), None),
                    (I.WORKLOADS[3].shrink(B=1, Hq=16, Hkv=4, N=1500, window=300), None),
                    (I.WORKLOADS[4].shrink(B=1, Hq=4, Hkv=4, N=2500), (64, 1024)),
                    (I.WORKLOADS[2].shrink(B=2, Hq=16, Hkv=16, N=4096), None),
                    (I.WORKLOADS[2].shrink(B=4, Hq=32, Hkv=32, N=2000), None),
                    (I.WORKLOADS[3].shrink(B=1, Hq=32, Hkv=8, N=3000, window=700), None),
                    (I.WORKLOADS[4].shrink(B=1, Hq=16, Hkv=16, N=8192), (64, 2048))):
        outs.append(run_fwd(_case(w, doc_range=docs), w.mask, w.window, w.softcap))
    lengths = [5000, 1, 777, 3000, 20000, 129, 9000, 2000, 300, 24590]   # 64 K tokens
    g = torch.Generator("cpu").manual_seed(11)
    total = sum(lengths)
    q = torch.randn(4, total, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(2, total, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(2, total, 128, generator=g).to(torch.bfloat16).cuda()
    cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0)), dtype=torch.int32).cuda()
    outs.append(_lib.fwd_varlen(q, k, v, cu, mask=I.MASK_CAUSAL))
    return outs


def test_persistent_launch_bitwise_equal():
    """ATTN_PERSISTENT=1 (a resident-sized grid walking the items in the same
    order) gives exactly the outputs of the one-workgroup-per-item launch."""
    import os
    import subprocess
    import sys
    import tempfile
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "persistent.pt")
        env = dict(os.environ, ATTN_PERSISTENT="1")
        r = subprocess.run([sys.executable, "-c", _PERSIST_CHILD, root, path], capture_output=True, text=True,
                           env=env, timeout=300)
        assert r.returncode == 0, r.stderr[-3000:]
        got = torch.load(path, weights_only=True)
    want = persistent_cases()
    for (o, l), (o2, l2) in zip(want, got):
        assert torch.equal(o.cpu(), o2) and torch.equal(l.cpu(), l2)
