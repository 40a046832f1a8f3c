"""Seeded sweep of the bf16 forward over random combinations of the features
(shape, GQA ratio, head dim, mask kind, window, document ids, soft-cap, ALiBi)
at sizes the oracle finishes in milliseconds: every case against the float64
oracle to the bf16 bars, and bit for bit against the single-stage build (a
tile read before its copy landed, or a buffer refilled while another wave
still reads it, would show up as a difference there)."""
import os
import random

import pytest
import torch

from tests.gpu_util import assert_close, oracle, run_fwd
from tiled_attention_05_amd import _lib
from tiled_attention_05_amd import inputs as I

pytestmark = pytest.mark.gpu

MASKS = [I.MASK_NONE, I.MASK_CAUSAL, I.MASK_CAUSAL | I.MASK_WINDOW, I.MASK_CAUSAL | I.MASK_DOC, I.MASK_DOC]
SIZES = [1, 7, 31, 64, 65, 200, 255, 256, 257, 511, 700, 1023, 1300]


def _cases(n, seed):
    rng = random.Random(seed)
    out = []
    for c in range(n):
        hkv = rng.choice([1, 2, 4])
        mask = rng.choice(MASKS)
        w = I.WORKLOADS[rng.choice([2, 3, 4])].shrink(
            B=rng.choice([1, 2]), Hq=hkv * rng.choice([1, 2, 4]), Hkv=hkv, N=rng.choice(SIZES),
            d=rng.choice([64, 128, 128]), mask=mask,
            window=rng.choice([1, 17, 100, 300]) if mask & I.MASK_WINDOW else 0,
            softcap=rng.choice([0.0, 0.0, 20.0, 50.0]), alibi=rng.random() < 0.4, extra={})
        out.append((c, w, rng.randrange(1 << 30)))
    return out


@pytest.mark.parametrize("group", range(4))
def test_forward_feature_sweep(group):
    assert os.path.exists(_lib.PATH_SINGLE_STAGE), "libattn_single_stage.so is built with libattn.so"
    for c, w, seed in _cases(50, 1000 + group):
        label = (f"sweep {group}.{c} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} mask={w.mask} "
                 f"window={w.window} softcap={w.softcap} alibi={w.alibi} seed={seed}")
        print(f"[case] {label}", flush=True)
        x = I.inputs(w, seed)
        o, lse = run_fwd(x, w.mask, w.window, w.softcap)
        with _lib.library(_lib.PATH_SINGLE_STAGE):
            o1, lse1 = run_fwd(x, w.mask, w.window, w.softcap)
        assert torch.equal(o, o1) and torch.equal(lse, lse1), f"single-stage build differs: {label}"
        O, L = oracle(x, w.scale, w.mask, w.window, w.softcap)
        assert_close(o, lse, O, L, label=label)
