"""Helpers of the GPU parity tests: upload, run, compare against the oracle."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import attention as A
from tiled_attention_05_amd import _lib

# bars: bf16 (and the fp32 workload) max-abs 2e-2, mean-abs 2e-3 over all of O; LSE 1e-3
MAX_ABS, MEAN_ABS, LSE_TOL = 2e-2, 2e-3, 1e-3


def to_dev(x):
    return None if x is None else x.to("cuda").contiguous()


def run_fwd(x, w_mask, window=0, softcap=0.0, scale=None):
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = _lib.fwd(q, k, v, scale=scale, mask=w_mask, window=window, doc_ids=to_dev(x.get("doc_ids")),
                      softcap=softcap, alibi_slopes=to_dev(x.get("slopes")))
    torch.cuda.synchronize()
    return o, lse


def errors(o_gpu, lse_gpu, O_ref, L_ref):
    o = o_gpu.detach().float().cpu().double().numpy().reshape(O_ref.shape)
    lse = lse_gpu.detach().cpu().double().numpy().reshape(L_ref.shape)
    err = np.abs(o - O_ref)
    fin = np.isfinite(L_ref)
    assert np.array_equal(fin, np.isfinite(lse)), "rows without keys must give LSE = -inf exactly"
    assert np.all(np.isneginf(lse[~fin]))
    lerr = np.abs(lse[fin] - L_ref[fin]).max() if fin.any() else 0.0
    return float(err.max()), float(err.mean()), float(lerr)


def assert_close(o_gpu, lse_gpu, O_ref, L_ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS, lse_tol=LSE_TOL,
                 label=""):
    mx, mn, le = errors(o_gpu, lse_gpu, O_ref, L_ref)
    print(f"[parity] {label} max_abs={mx:.3e} mean_abs={mn:.3e} lse_max={le:.3e}", flush=True)
    assert mx <= max_abs, f"{label}: max-abs {mx} > {max_abs}"
    assert mn <= mean_abs, f"{label}: mean-abs {mn} > {mean_abs}"
    assert le <= lse_tol, f"{label}: lse error {le} > {lse_tol}"
    return mx, mn, le


def oracle(x, scale, mask, window=0, softcap=0.0, heads=None, rows=None):
    return A.attention(x["q"], x["k"], x["v"], scale, mask, window, x.get("doc_ids"), softcap,
                       x.get("slopes"), heads=heads, rows=rows)


def oracle_whole_heads(x, w, heads, threads=None, chunk=1024):
    """Every row of the given (b, h) heads, the oracle run on row chunks of
    each head in parallel (rows are independent, so the result is the
    untiled one). Returns (O [n, N, d], LSE [n, N])."""
    from threadpoolctl import threadpool_limits
    N = w.N
    jobs = [(i, bh, np.arange(r0, min(r0 + chunk, N))) for i, bh in enumerate(heads) for r0 in range(0, N, chunk)]
    O = np.empty((len(heads), N, w.d))
    L = np.empty((len(heads), N))

    def run(job):
        i, bh, rows = job
        o, l = A.attention(x["q"], x["k"], x["v"], w.scale, w.mask, w.window, x.get("doc_ids"), w.softcap,
                           x.get("slopes"), heads=[bh], rows=rows, threads=1)
        O[i, rows] = o[0]
        L[i, rows] = l[0]

    n = threads or min(16, len(os.sched_getaffinity(0)))
    with threadpool_limits(limits=1), ThreadPoolExecutor(n) as ex:
        list(ex.map(run, jobs))
    return O, L
