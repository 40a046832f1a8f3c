"""GPU block-mask builder against a brute-force classification on the CPU, and
the forward kernel's own tile schedule against the builder."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from tiled_attention_05_amd import _lib
from tiled_attention_05_amd import inputs as I

pytestmark = pytest.mark.gpu

C, W, D = I.MASK_CAUSAL, I.MASK_WINDOW, I.MASK_DOC


def brute(B, Nq, Nk, mask, window, docs, bm, bn):
    nq, nk = -(-Nq // bm), -(-Nk // bn)
    kinds = np.zeros((B, nq, nk), dtype=np.int8)
    for b in range(B):
        ok = A.allowed_mask(np.arange(Nq), np.arange(Nk), Nq, Nk, mask, window,
                            None if docs is None else docs[b])
        for i in range(nq):
            for j in range(nk):
                blk = ok[i * bm:(i + 1) * bm, j * bn:(j + 1) * bn]
                kinds[b, i, j] = 0 if not blk.any() else (2 if blk.all() else 1)
    counts = np.stack([(kinds == c).sum(axis=2) for c in range(3)], axis=2)
    return kinds, counts


CASES = [
    (2, 300, 300, 1, 0, None, 128, 64),
    (1, 1000, 1000, 3, 200, None, 256, 64),
    (1, 1000, 1000, 3, 1, None, 64, 64),
    (2, 777, 777, 5, 0, (30, 300), 128, 64),
    (1, 600, 600, 4, 0, (1, 50), 100, 37),
    (1, 300, 900, 1, 0, None, 64, 128),
    (1, 900, 300, 1, 0, None, 128, 64),
    (1, 513, 513, 0, 0, None, 256, 128),
]


@pytest.mark.parametrize("B,Nq,Nk,mask,window,docr,bm,bn", CASES)
def test_builder_matches_brute_force(B, Nq, Nk, mask, window, docr, bm, bn):
    docs = None
    if docr is not None:
        rng = np.random.default_rng(Nq)
        rows = []
        for _ in range(B):
            lens, tot = [], 0
            while tot < Nk:
                n = min(int(rng.integers(docr[0], docr[1] + 1)), Nk - tot)
                lens.append(n)
                tot += n
            rows.append(np.repeat(np.arange(len(lens)), lens))
        docs = np.stack(rows).astype(np.int32)
    kinds, counts, flags = _lib.block_mask(B, Nq, Nk, mask, window,
                                           None if docs is None else torch.from_numpy(docs).cuda(), bm, bn)
    torch.cuda.synchronize()
    rk, rc = brute(B, Nq, Nk, mask, window, docs, bm, bn)
    assert np.array_equal(kinds.cpu().numpy(), rk)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert int(flags.item()) == 0


def test_builder_flags_decreasing_doc_ids():
    docs = torch.tensor([[0, 0, 1, 1, 0, 2, 2, 2]], dtype=torch.int32).cuda()
    _, _, flags = _lib.block_mask(1, 8, 8, _lib.MASK_DOC, 0, docs, 4, 4)
    torch.cuda.synchronize()
    assert int(flags.item()) & 1


# ------------------------------------------------------------------ the forward's own schedule
def _kinds_builder(B, Nq, Nk, mask, window, docs):
    kinds, _, _ = _lib.block_mask(B, Nq, Nk, mask, window, docs, block_m=32, block_n=64)
    return kinds


PLAN_CASES = [
    ("causal", 2, 1000, 1000, C, 0, None),
    ("dense ragged", 1, 300, 333, 0, 0, None),
    ("causal Nq<Nk", 1, 300, 1000, C, 0, None),
    ("causal Nq>Nk", 1, 1000, 300, C, 0, None),
    ("window", 2, 1500, 1500, C | W, 300, None),
    ("window 1", 1, 700, 700, C | W, 1, None),
    ("docs causal", 2, 2500, 2500, C | D, 0, (64, 1024)),
    ("docs short", 2, 900, 900, C | D, 0, (1, 40)),
    ("docs dense", 2, 700, 700, D, 0, (50, 300)),
]


@pytest.mark.parametrize("label,B,Nq,Nk,mask,window,docs", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_forward_schedule_equals_builder(label, B, Nq, Nk, mask, window, docs):
    """attn_fwd_tile_kinds (the forward kernel's own range and full-tile
    functions, per wave of 32 rows and 64-key tile) against the block-mask
    builder's exact table at the same tiling: identical, except that a ragged
    last key tile the builder finds full is partial in the forward."""
    print(f"[case] forward schedule {label}", flush=True)
    d = None
    if docs is not None:
        g = torch.Generator("cpu").manual_seed(Nq)
        rows = []
        for _ in range(B):
            lens = I.doc_lengths(Nk, g, *docs)
            rows.append(torch.repeat_interleave(torch.arange(len(lens), dtype=torch.int32), torch.tensor(lens)))
        d = torch.stack(rows).cuda()
    plan = _lib.fwd_tile_kinds(B, Nq, Nk, mask, window, d).cpu()
    ref = _kinds_builder(B, Nq, Nk, mask, window, d).cpu()
    torch.cuda.synchronize()
    assert plan.shape == ref.shape
    diff = plan != ref
    if Nk % 64:
        last = diff[:, :, -1]
        assert torch.all((plan[:, :, -1][last] == 1) & (ref[:, :, -1][last] == 2))
        diff[:, :, -1] = False
    assert not diff.any(), f"{int(diff.sum())} tiles differ"
    print(f"[schedule] {label}: empty {(plan == 0).float().mean():.4f} partial {(plan == 1).float().mean():.4f} "
          f"full {(plan == 2).float().mean():.4f}", flush=True)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_forward_schedule_workloads(k):
    """Same comparison on the full workloads' masks (document lengths of workload 4)."""
    w = I.WORKLOADS[k]
    print(f"[case] forward schedule workload {k}", flush=True)
    x = I.inputs(w)
    d = None if x["doc_ids"] is None else x["doc_ids"].cuda()
    plan = _lib.fwd_tile_kinds(w.B, w.N, w.N, w.mask, w.window, d).cpu()
    ref = _kinds_builder(w.B, w.N, w.N, w.mask, w.window, d).cpu()
    assert torch.equal(plan, ref)
    print(f"[schedule] workload {k}: skipped fraction {(plan == 0).float().mean():.4f}", flush=True)


_CHILD = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from tiled_attention_05_amd import _lib
q = torch.randn(1, 2, 640, 128, device="cuda").to(torch.bfloat16)
good = torch.repeat_interleave(torch.arange(4, dtype=torch.int32), torch.tensor([100, 200, 40, 300]))[None].cuda()
bad = good.clone()
bad[0, 350] = 0
for name, ids in (("good", good), ("bad", bad)):
    o = torch.empty_like(q)
    st = _lib.attn_fwd(q, q, q, o, None, 1, 2, 2, 640, 640, 128, 0.1, 5, 0, ids, 0.0, None, 1)
    torch.cuda.synchronize()
    print(name, st, flush=True)
# decode: a cached length beyond the table's capacity (3 blocks of 16) is
# rejected on the host before any launch
qd = torch.randn(1, 4, 128, device="cuda").to(torch.bfloat16)
cache = torch.randn(3, 2, 16, 128, device="cuda").to(torch.bfloat16)
table = torch.arange(3, dtype=torch.int32, device="cuda")[None]
od = torch.empty_like(qd)
for name, n in (("decode_fits", 48), ("decode_long", 60)):
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    st = _lib.attn_decode_paged(qd, cache, cache, table, lens, od, None, 1, 4, 2, 128, 16, 3, 0.1, 1, None, 1)
    torch.cuda.synchronize()
    print(name, st, flush=True)
"""


def test_attn_check_and_log_in_child_process():
    """ATTN_CHECK=1 rejects decreasing document ids (ATTN_ERR_INVALID_ARG, no
    launch) and accepts valid ones; ATTN_LOG=1 prints the grid and the tile
    counts, which match the forward's own schedule. The variables are read
    once per process, so this runs in one child process."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, ATTN_CHECK="1", ATTN_LOG="1")
    r = subprocess.run([sys.executable, "-c", _CHILD, root], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout, r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    lines = dict(l.split() for l in r.stdout.strip().splitlines())
    assert lines == {"good": "0", "bad": str(_lib.ERR_INVALID_ARG), "decode_fits": "0",
                     "decode_long": str(_lib.ERR_INVALID_ARG)}
    assert "grid=" in r.stderr and "doc_ids[0] decreases at 350" in r.stderr
    good = torch.repeat_interleave(torch.arange(4, dtype=torch.int32), torch.tensor([100, 200, 40, 300]))[None]
    plan = _lib.fwd_tile_kinds(1, 640, 640, C | D, 0, good.cuda()).cpu()
    want = (f"empty={int((plan == 0).sum())} partial={int((plan == 1).sum())} full={int((plan == 2).sum())}")
    assert want in r.stderr, want
