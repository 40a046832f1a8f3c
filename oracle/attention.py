"""Plain float64 attention: the definition the fused kernel must reproduce.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the product.

What is computed, and where it comes from
-----------------------------------------
The method only reorders the computation of softmax(Q K^T) V; its result is the
exact one ("FlashAttention-2 (FR)", opening section: exact attention without
precision loss; "FlashAttention-3 : une attention plus rapide ...", section
"Rappel du fonctionnement de FlashAttention": tiling plus softmax rescaling
gives the correct output without approximation). So this oracle is the plain
definition, materialising every score row, as the standard attention described
in "Les kernels d'attention rapide et la fusion d'operateurs ...", section
"Attention de type FlashAttention et attention paginee" (a T x T score matrix
per head).

For query head h of batch b (all arithmetic in float64):

1. GQA: query head h reads key/value head g = floor(h / (Hq/Hkv)).
2. s_ij = scale * sum_c q[b,h,i,c] k[b,g,j,c].
3. Soft-cap (if softcap > 0): s <- softcap * tanh(s / softcap).
4. ALiBi (if slopes given): s_ij <- s_ij - slope_h * (i - j).
5. Mask: allowed(i, j) per ``allowed_mask``; disallowed scores do not count.
6. m_i = max over allowed j of s_ij;  e_ij = exp(s_ij - m_i) on allowed pairs,
   0 elsewhere;  l_i = sum_j e_ij;  o_i = sum_j e_ij v[b,g,j,:] / l_i;
   lse_i = m_i + ln l_i.  A row with no allowed key gets o_i = 0, lse_i = -inf.

Score and mask modifiers (soft-capping, ALiBi, sliding window, document
masking) are the ones "FlexAttention de PyTorch avec FlashAttention-4 change la
donne" (opening section) lists as user patterns; the sliding window is a mask
change ("FlashAttention-3 : ...", section "Avis de Hacker News"). The pages
fix neither their constants nor their order; the readings taken here are:
scale first, then the cap, then the signed ALiBi bias; a window of W keys
(i - j < W, diagonal included); causal aligned bottom-right when Nq != Nk.

``attention_tiled`` walks the keys block by block with the running max / running
sum recurrences (the plainest reading of "update the softmax statistics per
block and accumulate the output on chip", "Les kernels d'attention rapide ...",
same section). It exists only so tests can check tiled == untiled.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Mask flags (bit set). Same numeric values as the library's public header;
# a CPU test asserts the two agree, nothing here is imported from there.
MASK_NONE = 0
MASK_CAUSAL = 1
MASK_WINDOW = 2   # sliding window, only together with CAUSAL
MASK_DOC = 4      # packed documents, with or without CAUSAL


def _f64(x):
    """Exact upcast of the stored values (fp32 / bf16 torch tensors or numpy)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def allowed_mask(rows, cols, Nq, Nk, mask_kind, window=0, doc_row=None):
    """Boolean [len(rows), len(cols)]: may query ``rows[a]`` attend to key ``cols[b]``.

    causal   : j <= i + (Nk - Nq)                (bottom-right alignment)
    window   : additionally (i + Nk - Nq) - j < window
    document : doc[i] == doc[j]  (and causal if CAUSAL is set); Nq == Nk
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    off = Nk - Nq
    if mask_kind & MASK_CAUSAL:
        ok &= j <= i + off
    if mask_kind & MASK_WINDOW:
        ok &= (i + off) - j < window
    if mask_kind & MASK_DOC:
        doc = np.asarray(doc_row, dtype=np.int64)
        ok &= doc[i] == doc[j]
    return ok


def scores(q_rows, k_all, rows, Nq, Nk, scale, softcap=0.0, slope=None):
    """Raw modified scores s_ij (steps 2-4) for the given query rows, float64."""
    s = scale * (q_rows @ k_all.T)
    if softcap > 0.0:
        s = softcap * np.tanh(s / softcap)
    if slope is not None:
        i = np.asarray(rows, dtype=np.float64)[:, None]
        j = np.arange(Nk, dtype=np.float64)[None, :]
        s = s - slope * (i - j)
    return s


def probabilities(s, ok):
    """Row softmax over allowed entries (step 6), returning (P, m, l)."""
    s_m = np.where(ok, s, -np.inf)
    m = s_m.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.where(ok, np.exp(s_m - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
    return p, m, l


def _head(qh, kh, vh, rows, Nq, Nk, scale, mask_kind, window, doc_row, softcap, slope, chunk):
    out_o = np.empty((len(rows), qh.shape[1]), dtype=np.float64)
    out_l = np.empty(len(rows), dtype=np.float64)
    cols = np.arange(Nk)
    for a in range(0, len(rows), chunk):
        r = rows[a:a + chunk]
        s = scores(qh[r], kh, r, Nq, Nk, scale, softcap, slope)
        ok = allowed_mask(r, cols, Nq, Nk, mask_kind, window, doc_row)
        p, m, l = probabilities(s, ok)
        out_o[a:a + len(r)] = p @ vh
        with np.errstate(divide="ignore"):
            out_l[a:a + len(r)] = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out_o, out_l


def attention(q, k, v, scale, mask_kind=MASK_NONE, window=0, doc_ids=None, softcap=0.0,
              alibi_slopes=None, heads=None, rows=None, threads=None, chunk=512):
    """Exact attention forward. q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] (BHSD).

    heads : optional list of (b, h) pairs to evaluate (default: all).
    rows  : optional array of query rows to evaluate for every selected head.
    Returns (O, LSE) float64 with shapes [n_heads_sel, n_rows, d] and
    [n_heads_sel, n_rows] when ``heads``/``rows`` are given, else
    [B,Hq,Nq,d] and [B,Hq,Nq].
    """
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    slopes = None if alibi_slopes is None else _f64(alibi_slopes)
    docs = None if doc_ids is None else np.asarray(_f64(doc_ids), dtype=np.int64)
    if mask_kind & MASK_DOC and docs is None:
        raise ValueError("document mask needs doc_ids")
    full = heads is None and rows is None
    sel = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    rr = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)

    def job(bh):
        b, h = bh
        g = h // G
        # upcast one head at a time (exact), so sampled checks stay small
        return _head(_f64(q[b, h]), _f64(k[b, g]), _f64(v[b, g]), rr, Nq, Nk, float(scale), mask_kind,
                     window, None if docs is None else docs[b], float(softcap),
                     None if slopes is None else float(slopes[h]), chunk)

    nthreads = threads or min(len(sel), os.cpu_count() or 1)
    if nthreads > 1:
        # one BLAS thread per worker: parallelism comes from the (b, h) pool
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1), ThreadPoolExecutor(nthreads) as ex:
            res = list(ex.map(job, sel))
    else:
        res = [job(x) for x in sel]
    O = np.stack([r[0] for r in res])
    L = np.stack([r[1] for r in res])
    if full:
        return O.reshape(B, Hq, Nq, d), L.reshape(B, Hq, Nq)
    return O, L


def attention_tiled(q, k, v, scale, block, mask_kind=MASK_NONE, window=0, doc_ids=None,
                    softcap=0.0, alibi_slopes=None):
    """Same result via per-key-block online softmax (running max m, running sum l).

    Per row: m = -inf, l = 0, acc = 0; for each key block:
      m' = max(m, blockmax);  alpha = exp(m - m') (1 when m' = -inf);
      e = exp(s_blk - m') on allowed entries;  l = alpha l + sum e;
      acc = alpha acc + e V_blk.   Finally O = acc / l, lse = m + ln l.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    G = Hq // Hkv
    slopes = None if alibi_slopes is None else _f64(alibi_slopes)
    docs = None if doc_ids is None else np.asarray(_f64(doc_ids), dtype=np.int64)
    O = np.zeros((B, Hq, Nq, d))
    L = np.full((B, Hq, Nq), -np.inf)
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            m = np.full(Nq, -np.inf)
            l = np.zeros(Nq)
            acc = np.zeros((Nq, d))
            for j0 in range(0, Nk, block):
                cols = np.arange(j0, min(j0 + block, Nk))
                s = scale * (q[b, h] @ k[b, g, cols].T)
                if softcap > 0.0:
                    s = softcap * np.tanh(s / softcap)
                if slopes is not None:
                    s = s - slopes[h] * (rows[:, None] - cols[None, :]).astype(np.float64)
                ok = allowed_mask(rows, cols, Nq, Nk, mask_kind, window,
                                  None if docs is None else docs[b])
                s = np.where(ok, s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                ref = np.where(np.isfinite(m_new), m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - ref), 1.0)
                e = np.where(ok, np.exp(s - ref[:, None]), 0.0)
                l = alpha * l + e.sum(axis=1)
                acc = alpha[:, None] * acc + e @ v[b, g, cols]
                m = m_new
            has = l > 0
            O[b, h] = np.where(has[:, None], acc / np.where(has, l, 1.0)[:, None], 0.0)
            with np.errstate(divide="ignore"):
                L[b, h] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, L


def allowed_pairs(Nq, Nk, mask_kind, window=0, doc_row=None, chunk=1024):
    """Number of allowed (i, j) pairs of one head, by direct enumeration."""
    cols = np.arange(Nk)
    n = 0
    for a in range(0, Nq, chunk):
        r = np.arange(a, min(a + chunk, Nq))
        n += int(allowed_mask(r, cols, Nq, Nk, mask_kind, window, doc_row).sum())
    return n


def attention_varlen(q, k, v, cu_seqlens, scale, mask_kind=MASK_NONE, window=0, softcap=0.0,
                     alibi_slopes=None, threads=None):
    """Exact forward over a packed batch of sequences, one sequence at a time.

    q [Hq, total, d], k / v [Hkv, total, d]; sequence s is tokens
    cu_seqlens[s] .. cu_seqlens[s+1]-1 and attends only within itself
    ("FlashAttention-3 : ...", section "Optimisations restantes et integration
    future": variable-length sequences). Each sequence is cut out and passed to
    ``attention`` as a batch of one, with its own positions (mask_kind: NONE or
    CAUSAL, optionally | WINDOW). Returns (O [Hq, total, d], LSE [Hq, total]).
    """
    Hq, total, d = q.shape
    cu = [int(x) for x in np.asarray(_f64(cu_seqlens)).astype(np.int64)]
    O = np.zeros((Hq, total, d))
    L = np.full((Hq, total), -np.inf)
    for a, b in zip(cu[:-1], cu[1:]):
        if b <= a:
            continue
        o, l = attention(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], scale, mask_kind, window,
                         None, softcap, alibi_slopes, threads=threads)
        O[:, a:b] = o[0]
        L[:, a:b] = l[0]
    return O, L


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale, block_size=16):
    """Exact one-token decode over a paged key/value cache.

    q [B, Hq, d] (the newest token of each sequence); k_cache / v_cache
    [num_blocks, Hkv, block_size, d]; block_table [B, max_blocks] (logical block
    i of sequence b lives in physical block block_table[b, i]); seq_lens [B].
    The keys of sequence b are gathered in logical order and the query attends
    to all of them ("Les kernels d'attention rapide ...", section "Attention de
    type FlashAttention et attention paginee": the cache is kept in fixed-size
    blocks addressed through a table). Returns (O [B, Hq, d], LSE [B, Hq]).
    """
    qn = np.asarray(_f64(q))
    kc = _f64(k_cache)
    vc = _f64(v_cache)
    bt = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    B, Hq, d = qn.shape
    O = np.zeros((B, Hq, d))
    L = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(lens[b])
        if n <= 0:
            continue
        nb = -(-n // block_size)
        blocks = bt[b, :nb]
        k = np.concatenate([kc[p] for p in blocks], axis=1)[:, :n]   # [Hkv, n, d]
        v = np.concatenate([vc[p] for p in blocks], axis=1)[:, :n]
        o, l = attention(qn[b][None, :, None, :], k[None], v[None], scale, threads=1)
        O[b] = o[0, :, 0]
        L[b] = l[0, :, 0]
    return O, L


def attention_backward(q, k, v, do, scale, mask_kind=MASK_NONE):
    """Exact gradients of the forward (float64) for an output gradient ``do``.

    With P the row softmax of the masked scores s = scale q.k, O = P V and
    D_i = sum_c dO_ic O_ic (= sum_j P_ij dP_ij):
        dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
    summed over the query heads of each key/value head. This is the chain rule
    through the softmax; the method recomputes P from the saved LSE instead of
    storing it, and its result stays exact and deterministic ("FlashAttention-2
    (FR)", section "Performance et efficacite"). q [B,Hq,N,d], k/v [B,Hkv,Nk,d],
    do like q. Returns (dQ, dK, dV) float64.
    """
    q, k, v, do = (np.asarray(_f64(x)) for x in (q, k, v, do))
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    G = Hq // Hkv
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    ok = allowed_mask(np.arange(Nq), np.arange(Nk), Nq, Nk, mask_kind)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = scale * q[b, h] @ k[b, g].T
            s = np.where(ok, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(ok, np.exp(s - m), 0.0)
            l = e.sum(axis=1, keepdims=True)
            P = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
            O = P @ v[b, g]
            dP = do[b, h] @ v[b, g].T
            D = (do[b, h] * O).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dQ[b, h] = scale * dS @ k[b, g]
            dK[b, g] += scale * dS.T @ q[b, h]
            dV[b, g] += P.T @ do[b, h]
    return dQ, dK, dV
