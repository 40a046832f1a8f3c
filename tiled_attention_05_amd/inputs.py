"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds input generation only, none of the attention arithmetic:
Q/K/V draws, document lengths, outlier channels, ALiBi slopes and the random
Hadamard signs are all *inputs* of the method, drawn here and handed to both the
HIP path and the CPU oracle.

Recipe (fixed so every run sees the same data):

* Q, K, V: ``torch.Generator('cpu')`` seeded ``1000 + k`` (k = workload number),
  drawn in the order Q, K, V with ``torch.randn(..., dtype=float32)``, then cast
  to bfloat16 (round to nearest even) for the bf16 workloads.  Layout BHSD.
* Auxiliary draws use a second generator seeded ``k``, in this order: outlier
  channels of Q then K (fp8 workload), document lengths (document workload),
  Hadamard signs (fp8 workload).
* Document lengths: scalar ``randint(512, 8193)`` draws (uniform on [512, 8192])
  until the total reaches N; the last document is cut to fit.  ``doc_ids`` is
  the non-decreasing document index of every token.
* fp8 outliers: 0.1 % of the Hq*d (head, feature) channels, rounded to the
  nearest integer (at least one), picked independently for Q and for K; those
  columns are multiplied by 20 for every batch and token before the cast.  The
  alternative construction scales 0.1 % of individual entries of Q, K and V.
* ALiBi slopes: slope_h = 2^(-8 (h + 1) / H), h = 0 .. H-1.
* Hadamard signs: ``randint(0, 2, (d,)) * 2 - 1`` as int8.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

# mask flags; the same values as the C header (checked by a CPU test)
MASK_NONE = 0
MASK_CAUSAL = 1
MASK_WINDOW = 2
MASK_DOC = 4


@dataclass(frozen=True)
class Workload:
    k: int                    # workload number: seeds are k and 1000 + k
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str                # "f32" | "bf16" | "fp8"
    mask: int = MASK_NONE
    window: int = 0
    softcap: float = 0.0
    alibi: bool = False
    outlier_frac: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def shrink(self, **kw) -> "Workload":
        """Same structure at other sizes (used for parity at sizes the oracle finishes fast)."""
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny_dense_fp32", B=1, Hq=2, Hkv=2, N=128, d=64, dtype="f32"),
    2: Workload(2, "causal_prefill_bf16", B=4, Hq=32, Hkv=32, N=4096, d=128, dtype="bf16",
                mask=MASK_CAUSAL),
    3: Workload(3, "gqa_sliding_window_bf16", B=2, Hq=32, Hkv=8, N=16384, d=128, dtype="bf16",
                mask=MASK_CAUSAL | MASK_WINDOW, window=4096),
    4: Workload(4, "docs_softcap_alibi_bf16", B=1, Hq=16, Hkv=16, N=32768, d=128, dtype="bf16",
                mask=MASK_CAUSAL | MASK_DOC, softcap=50.0, alibi=True),
    5: Workload(5, "fp8_hadamard", B=4, Hq=16, Hkv=16, N=8192, d=128, dtype="fp8",
                outlier_frac=0.001),
    # backward of the causal prefill (same shapes as workload 2)
    8: Workload(8, "causal_prefill_bf16_backward", B=4, Hq=32, Hkv=32, N=4096, d=128, dtype="bf16",
                mask=MASK_CAUSAL, extra={"backward": True}),
    # one-token decode over a paged cache: 64 sequences of [1024, 8192] cached tokens, 16-token blocks
    7: Workload(7, "decode_paged_bf16", B=64, Hq=32, Hkv=8, N=8192, d=128, dtype="bf16",
                extra={"decode": True, "len_range": (1024, 8192), "block": 16, "splits": 8}),
    # packed variable-length batch: sequences of [128, 4096] tokens, causal within each
    6: Workload(6, "varlen_causal_bf16", B=1, Hq=32, Hkv=8, N=32768, d=128, dtype="bf16",
                mask=MASK_CAUSAL | MASK_DOC, extra={"varlen": True, "len_range": (128, 4096)}),
}


def qkv(w: Workload, seed: int | None = None, outliers: str = "channels", aux=None):
    """Q [B,Hq,N,d], K and V [B,Hkv,N,d] on the CPU (fp32 or bf16; fp8 workloads give bf16).

    Outliers (fp8 workloads) are drawn from ``aux``, the auxiliary generator.
    """
    g = torch.Generator("cpu").manual_seed(1000 + w.k if seed is None else 1000 + seed)
    q = torch.randn(w.B, w.Hq, w.N, w.d, generator=g, dtype=torch.float32)
    k = torch.randn(w.B, w.Hkv, w.N, w.d, generator=g, dtype=torch.float32)
    v = torch.randn(w.B, w.Hkv, w.N, w.d, generator=g, dtype=torch.float32)
    if w.outlier_frac > 0 and outliers != "none":
        if aux is None:
            aux = aux_generator(w, seed)
        if outliers == "channels":
            for t, H in ((q, w.Hq), (k, w.Hkv)):
                n = max(1, round(w.outlier_frac * H * w.d))
                ch = torch.randperm(H * w.d, generator=aux)[:n]
                for c in ch.tolist():
                    t[:, c // w.d, :, c % w.d] *= 20.0
        elif outliers == "entries":
            for t in (q, k, v):
                n = max(1, round(w.outlier_frac * t.numel()))
                idx = torch.randperm(t.numel(), generator=aux)[:n]
                t.view(-1)[idx] *= 20.0
        else:
            raise ValueError(outliers)
    if w.dtype in ("bf16", "fp8"):
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    return q, k, v


def aux_generator(w: Workload, seed: int | None = None):
    """The auxiliary generator of a workload, seeded with its number k (or ``seed``)."""
    return torch.Generator("cpu").manual_seed(w.k if seed is None else seed)


def doc_lengths(N: int, g: torch.Generator, lo: int = 512, hi: int = 8192):
    """Document lengths drawn from ``g``, uniform on [lo, hi], last one cut so they sum to N."""
    out, tot = [], 0
    while tot < N:
        n = int(torch.randint(lo, hi + 1, (1,), generator=g).item())
        n = min(n, N - tot)
        out.append(n)
        tot += n
    return out


def doc_ids(w: Workload, seed: int | None = None, aux=None):
    """int32 [B, N] non-decreasing document index per token (batch rows drawn in turn)."""
    rows = []
    g = aux_generator(w, seed) if aux is None else aux
    lo, hi = w.extra.get("len_range", (512, 8192))
    for b in range(w.B):
        lens = doc_lengths(w.N, g, lo, hi)
        rows.append(torch.repeat_interleave(torch.arange(len(lens), dtype=torch.int32),
                                            torch.tensor(lens)))
    return torch.stack(rows)


def decode_inputs(B, Hq, Hkv, d, lens, block=16, seed=0, dtype=torch.bfloat16):
    """Paged decode inputs: q [B, Hq, d]; k_cache / v_cache [num_blocks, Hkv, block, d]
    holding every sequence's keys in blocks placed by a seeded permutation;
    block_table int32 [B, max_blocks] (unused entries 0); seq_lens int32 [B]."""
    g = torch.Generator("cpu").manual_seed(1000 + seed)
    lens = [int(x) for x in lens]
    nbs = [-(-n // block) for n in lens]
    total = max(1, sum(nbs))
    maxb = max(1, max(nbs))
    q = torch.randn(B, Hq, d, generator=g).to(dtype)
    kc = torch.randn(total, Hkv, block, d, generator=g).to(dtype)
    vc = torch.randn(total, Hkv, block, d, generator=g).to(dtype)
    perm = torch.randperm(total, generator=g)
    table = torch.zeros(B, maxb, dtype=torch.int32)
    at = 0
    for b, nb in enumerate(nbs):
        table[b, :nb] = perm[at:at + nb].to(torch.int32)
        at += nb
    return q, kc, vc, table, torch.tensor(lens, dtype=torch.int32)


def decode_lengths(w: Workload, seed: int | None = None):
    """Cached lengths of a decode workload: uniform on its len_range, from the auxiliary generator."""
    lo, hi = w.extra["len_range"]
    g = aux_generator(w, seed)
    return torch.randint(lo, hi + 1, (w.B,), generator=g).tolist()


def cu_seqlens(ids_row):
    """int32 [n + 1] start offsets of the runs of a non-decreasing id row
    (the packed-sequence offsets of a variable-length batch), last = len."""
    ids = torch.as_tensor(ids_row).to(torch.int64)
    starts = torch.nonzero(torch.diff(ids, prepend=ids[:1] - 1)).flatten()
    return torch.cat([starts, torch.tensor([ids.numel()])]).to(torch.int32)


def rope_tables(N: int, d: int, base: float = 10000.0):
    """float32 [N, d/2] cos and sin of the rotary angles t * base^(-2i/d) (computed in float64)."""
    t = torch.arange(N, dtype=torch.float64)[:, None]
    theta = base ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    return torch.cos(t * theta).to(torch.float32), torch.sin(t * theta).to(torch.float32)


def alibi_slopes(H: int):
    """float32 [H]: 2^(-8 (h + 1) / H)."""
    h = torch.arange(H, dtype=torch.float64)
    return torch.pow(2.0, -8.0 * (h + 1) / H).to(torch.float32)


def hadamard_signs(d: int, g: torch.Generator):
    """int8 [d] of +-1 drawn from ``g``."""
    return (torch.randint(0, 2, (d,), generator=g) * 2 - 1).to(torch.int8)


def inputs(w: Workload, seed: int | None = None, outliers: str = "channels"):
    """Every input of one workload as CPU tensors: q, k, v, doc_ids, slopes, signs."""
    aux = aux_generator(w, seed)
    q, k, v = qkv(w, seed, outliers, aux)               # outlier channels first ...
    docs = doc_ids(w, aux=aux) if w.mask & MASK_DOC else None
    signs = hadamard_signs(w.d, aux) if w.dtype == "fp8" else None   # ... then the signs
    return {
        "q": q, "k": k, "v": v, "doc_ids": docs,
        "slopes": alibi_slopes(w.Hq) if w.alibi else None, "signs": signs,
    }
