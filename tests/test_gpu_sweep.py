"""Seeded sweeps over random combinations of each entry point's features, at
sizes the oracle finishes in milliseconds.

The bf16 forward (shape, GQA ratio, head dim, mask kind, window, document ids,
soft-cap, ALiBi): every case against the float64 oracle to the bf16 bars, and
bit for bit against the single-stage build (a tile read before its copy
landed, or a buffer refilled while another wave still reads it, would show up
as a difference there). Packed variable-length batches, paged decode and the
fp8 forward: against their oracles to the same bars as their own tests."""
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


def test_varlen_sweep():
    """Seeded random packed batches (empty, one-token and long sequences mixed,
    GQA, masks, soft-cap, ALiBi) through attn_fwd_varlen: against the oracle,
    and the workspace tile list bit-exact against its host-side definition."""
    from oracle import attention as A
    from tests.test_gpu_varlen import _pack, _tile_list
    rng = random.Random(21)
    for c in range(24):
        lengths = [rng.choice([0, 1, 2, 31, 64, 255, 256, 257, 700, 1500]) for _ in range(rng.randint(1, 9))]
        if sum(lengths) == 0:
            lengths.append(5)
        hkv = rng.choice([1, 2])
        hq = hkv * rng.choice([1, 2, 4])
        mask = rng.choice([0, I.MASK_CAUSAL, I.MASK_CAUSAL | I.MASK_WINDOW])
        window = rng.choice([1, 50, 300]) if mask & I.MASK_WINDOW else 0
        softcap = rng.choice([0.0, 30.0])
        alibi = rng.random() < 0.3
        label = f"varlen sweep {c} lengths={lengths} Hq={hq} Hkv={hkv} mask={mask} W={window} cap={softcap} alibi={alibi}"
        print(f"[case] {label}", flush=True)
        q, k, v, cu = _pack(lengths, hq, hkv, 128, torch.bfloat16, seed=300 + c)
        slopes = I.alibi_slopes(hq) if alibi else None
        ws = torch.empty(q.shape[1], dtype=torch.int32, device="cuda")
        o, lse = _lib.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), scale=128 ** -0.5, mask=mask,
                                 window=window, softcap=softcap,
                                 alibi_slopes=None if slopes is None else slopes.cuda(), workspace=ws)
        torch.cuda.synchronize()
        tiles = _tile_list(lengths)
        if tiles is not None:
            assert ws[:len(tiles)].cpu().tolist() == tiles, label
        O, L = A.attention_varlen(q, k, v, cu, 128 ** -0.5, mask, window, softcap, slopes)
        assert_close(o[None], lse[None], O[None], L[None], label=label)


def test_decode_sweep():
    """Seeded random paged-decode batches (empty to 3000-token caches, GQA
    ratios, 1 to 12 key splits) against the paged-decode oracle."""
    from oracle import attention as A
    rng = random.Random(31)
    for c in range(24):
        B = rng.randint(1, 12)
        hkv = rng.choice([1, 2, 4, 8])
        hq = hkv * rng.choice([1, 2, 4])
        lens = [rng.choice([0, 1, 15, 16, 17, 31, 32, 33, 500, 1024, 3000]) for _ in range(B)]
        splits = rng.randint(1, 12)
        label = f"decode sweep {c} B={B} Hq={hq} Hkv={hkv} lens={lens} splits={splits}"
        print(f"[case] {label}", flush=True)
        q, kc, vc, bt, sl = I.decode_inputs(B, hq, hkv, 128, lens, seed=700 + c)
        o, lse = _lib.decode_paged(q.cuda(), kc.cuda(), vc.cuda(), bt.cuda(), sl.cuda(), scale=128 ** -0.5,
                                   num_splits=splits)
        torch.cuda.synchronize()
        O, L = A.decode_paged(q, kc, vc, bt, sl, 128 ** -0.5)
        assert_close(o, lse, O, L, label=label)


def test_fp8_sweep():
    """Seeded random fp8 shapes (batch, GQA ratio, ragged lengths) on the
    oracle's own e4m3 codes: against the exact float64 attention to the 5e-2
    relative-RMS bar and against the emulation of the scheme."""
    import numpy as np
    from oracle import attention as A
    from oracle import fp8 as F8
    from tests.test_gpu_fp8 import FP8_RELRMS, _pack_oracle, _relrms
    rng = random.Random(41)
    for c in range(10):
        hkv = rng.choice([1, 2])
        hq = hkv * rng.choice([1, 2])
        N = rng.choice([1, 100, 128, 129, 300, 511, 700])
        w = I.WORKLOADS[5].shrink(B=1, Hq=hq, Hkv=hkv, N=N)
        seed = 900 + c
        label = f"fp8 sweep {c} Hq={hq} Hkv={hkv} N={N} seed={seed}"
        print(f"[case] {label}", flush=True)
        x = I.inputs(w, seed, "channels")
        q8, k8, v8 = _pack_oracle(w, x)
        o, lse = _lib.fwd_fp8(q8, k8, v8, w.B, hq, hkv, N, 128, scale=w.scale)
        torch.cuda.synchronize()
        q64, k64, v64 = (x[n].double().numpy() for n in ("q", "k", "v"))
        og = o.float().cpu().double().numpy().reshape(hq, N, 128)
        lg = lse.cpu().double().numpy().reshape(hq, N)
        Oe, Le = F8.attention_emulated(q64, k64, v64, x["signs"].numpy(), w.scale, lazy_tau=4 * np.log(2))
        O, L = A.attention(q64, k64, v64, w.scale)
        r_emu, r_exact = _relrms(og, Oe), _relrms(og, O.reshape(hq, N, 128))
        print(f"[fp8] {label}: relRMS vs emulation {r_emu:.3e}, vs exact {r_exact:.3e}", flush=True)
        assert r_emu <= 1e-2 and np.abs(lg - Le).max() <= 1e-3 and r_exact <= FP8_RELRMS, label
