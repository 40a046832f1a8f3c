"""The single-stage debug build of the forward kernels gives exactly the outputs
of the pipelined library.

libattn_single_stage.so is the same library with the bf16 and fp8 forward
kernels compiled with -DATTN_SINGLE_STAGE: one key/value tile in flight, every
copy waited for as soon as it is issued, LDS fragments read just before their
product. Both builds do the same arithmetic in the same order, so a difference
can only come from a tile read before its copy landed or a buffer refilled
while another wave still reads it.
"""
import os

import pytest
import torch

from tests.gpu_util import run_fwd
from tests.test_gpu_fwd import _case
from tiled_attention_05_amd import _lib
from tiled_attention_05_amd import inputs as I

pytestmark = pytest.mark.gpu


def _both(fn):
    assert os.path.exists(_lib.PATH_SINGLE_STAGE), "libattn_single_stage.so is built with libattn.so"
    want = fn()
    torch.cuda.synchronize()
    with _lib.library(_lib.PATH_SINGLE_STAGE):
        got = fn()
        torch.cuda.synchronize()
    return want, got


def _equal(want, got, label):
    for a, b in zip(want, got):
        same = torch.equal(a, b)
        if not same:
            d = (a.float() - b.float()).abs()
            print(f"[single-stage] {label}: {int((d > 0).sum())} elements differ, max {float(d.max()):.3e}",
                  flush=True)
        assert same, label


BF16_CASES = [
    ("causal ragged", I.WORKLOADS[2].shrink(B=2, Hq=8, Hkv=8, N=1000), None),
    ("dense d=64", I.WORKLOADS[2].shrink(B=1, Hq=4, Hkv=4, N=700, d=64, mask=I.MASK_NONE), None),
    ("gqa window", I.WORKLOADS[3].shrink(B=1, Hq=16, Hkv=4, N=1500, window=300), None),
    ("docs softcap alibi", I.WORKLOADS[4].shrink(B=1, Hq=4, Hkv=4, N=2500), (64, 1024)),
    ("softcap dense", I.WORKLOADS[4].shrink(B=1, Hq=4, Hkv=4, N=900, mask=I.MASK_NONE, alibi=False), None),
    ("alibi causal", I.WORKLOADS[4].shrink(B=1, Hq=4, Hkv=4, N=1100, mask=I.MASK_CAUSAL, softcap=0.0), None),
]


@pytest.mark.parametrize("label,w,docs", BF16_CASES, ids=[c[0] for c in BF16_CASES])
def test_bf16_forward_single_stage_bitwise(label, w, docs):
    print(f"[case] single-stage {label} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} mask={w.mask}", flush=True)
    x = _case(w, doc_range=docs)
    want, got = _both(lambda: run_fwd(x, w.mask, w.window, w.softcap))
    _equal(want, got, label)


def test_bf16_causal_prefill_workload_single_stage_bitwise():
    """The full causal prefill (2048 workgroups, every CU busy); also prints
    both builds' launch times, the single-stage one being the slower."""
    w = I.WORKLOADS[2]
    print(f"[case] single-stage causal prefill B={w.B} H={w.Hq} N={w.N}", flush=True)
    x = I.inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))

    def run():
        o, lse = _lib.fwd(q, k, v, scale=w.scale, mask=w.mask)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(5):
            _lib.fwd(q, k, v, scale=w.scale, mask=w.mask, out=o, lse=lse)
        ev[1].record()
        torch.cuda.synchronize()
        run.ms.append(ev[0].elapsed_time(ev[1]) / 5)
        return o, lse

    run.ms = []
    want, got = _both(run)
    print(f"[single-stage] causal prefill: pipelined {run.ms[0]:.3f} ms, single-stage {run.ms[1]:.3f} ms", flush=True)
    _equal(want, got, "causal prefill workload")


def test_varlen_single_stage_bitwise():
    lengths = [300, 1, 777, 64, 1500, 129]
    g = torch.Generator("cpu").manual_seed(5)
    total = sum(lengths)
    q = torch.randn(8, total, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(2, total, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(2, total, 128, generator=g).to(torch.bfloat16).cuda()
    cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0)), dtype=torch.int32).cuda()
    print(f"[case] single-stage varlen lengths={lengths}", flush=True)
    want, got = _both(lambda: _lib.fwd_varlen(q, k, v, cu, mask=I.MASK_CAUSAL))
    _equal(want, got, "varlen")


@pytest.mark.parametrize("N", [1000, 2048])
def test_fp8_forward_single_stage_bitwise(N):
    w = I.WORKLOADS[5].shrink(B=2, Hq=4, Hkv=4, N=N)
    print(f"[case] single-stage fp8 B={w.B} H={w.Hq} N={w.N}", flush=True)
    x = I.inputs(w)
    q8, k8, v8 = _lib.fp8_prepare(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["signs"].cuda())
    want, got = _both(lambda: _lib.fwd_fp8(q8, k8, v8, w.B, w.Hq, w.Hkv, w.N, 128, scale=w.scale))
    _equal(want, got, f"fp8 N={N}")
