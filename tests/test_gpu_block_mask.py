"""GPU block-mask builder against a brute-force classification on the CPU."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from tiled_attention_05_amd import _lib

pytestmark = pytest.mark.gpu


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
