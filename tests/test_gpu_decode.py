"""GPU parity of attn_decode_paged against the paged-decode oracle, through the
C ABI. Bars as for attn_fwd: max-abs 2e-2, mean-abs 2e-3 on O, 1e-3 on LSE."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.gpu_util import assert_close
from tiled_attention_05_amd import _lib
from tiled_attention_05_amd import inputs as I

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, lens, splits
    (3, 4, 4, [1, 16, 17], 1),
    (2, 8, 2, [100, 1000], 1),
    (2, 8, 2, [100, 1000], 4),
    (4, 32, 1, [33, 300, 64, 5000], 8),
    (2, 16, 8, [0, 77], 3),
    (1, 6, 3, [4097], 16),
    (3, 4, 2, [31, 32, 65], 8),
    # equal and empty lengths: the sequences are launched longest first, ties by index
    (9, 4, 2, [50, 300, 50, 0, 300, 7, 1000, 50, 0], 4),
    (70, 4, 2, [(i * 37) % 50 * 7 for i in range(70)], 3),
    # lengths equal to the table's capacity with an odd number of blocks: the last
    # 32-key chunk's second page is past the row end and must not be read
    (2, 4, 2, [48, 16], 2),
    (1, 4, 1, [80], 1),
    (3, 8, 2, [112, 112, 3], 4),
]


@pytest.mark.parametrize("B,Hq,Hkv,lens,splits", CASES,
                         ids=[f"B{c[0]}-{c[1]}x{c[2]}-{c[3][:4]}-s{c[4]}" for c in CASES])
def test_decode_matches_oracle(B, Hq, Hkv, lens, splits):
    print(f"[case] decode B={B} Hq={Hq} Hkv={Hkv} lens={lens} splits={splits}", flush=True)
    q, kc, vc, bt, sl = I.decode_inputs(B, Hq, Hkv, 128, lens, seed=sum(lens) + splits)
    scale = 128 ** -0.5
    o, lse = _lib.decode_paged(q.cuda(), kc.cuda(), vc.cuda(), bt.cuda(), sl.cuda(), scale=scale,
                               num_splits=splits)
    torch.cuda.synchronize()
    O, L = A.decode_paged(q, kc, vc, bt, sl, scale)
    assert_close(o, lse, O, L, label=f"decode {lens} s{splits}")


def test_decode_splits_agree():
    """More splits change only the rounding of the merge: outputs within the bf16 bar of one split."""
    q, kc, vc, bt, sl = I.decode_inputs(2, 8, 2, 128, [3000, 2500], seed=9)
    args = [t.cuda() for t in (q, kc, vc, bt, sl)]
    o1, l1 = _lib.decode_paged(*args, num_splits=1)
    o8, l8 = _lib.decode_paged(*args, num_splits=8)
    torch.cuda.synchronize()
    assert (o1.float() - o8.float()).abs().max().item() <= 2e-2
    assert (l1 - l8).abs().max().item() <= 1e-3


def test_decode_workload_sampled_sequences():
    """The decode workload (64 sequences of 1024-8192 cached tokens, GQA 32/8) in
    the configuration the benchmark times, checked on 6 sampled sequences."""
    w = I.WORKLOADS[7]
    lens = I.decode_lengths(w)
    q, kc, vc, bt, sl = I.decode_inputs(w.B, w.Hq, w.Hkv, w.d, lens, seed=w.k)
    print(f"[case] decode workload lens {min(lens)}..{max(lens)}", flush=True)
    o, lse = _lib.decode_paged(q.cuda(), kc.cuda(), vc.cuda(), bt.cuda(), sl.cuda(), scale=w.scale,
                               num_splits=w.extra.get("splits", 4))
    torch.cuda.synchronize()
    pick = [0, 5, 17, 33, 50, 63]
    O, L = A.decode_paged(q[pick], kc, vc, bt[pick], sl[pick], w.scale)
    assert_close(o[pick], lse[pick], O, L, label="decode workload sampled")
