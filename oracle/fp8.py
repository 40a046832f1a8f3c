"""fp8 (OCP e4m3) pieces of the oracle: codec, Hadamard rotation, quantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
-------
"FlashAttention-3 : une attention plus rapide ...", section "Fonctionnalites
des GPU Hopper : WGMMA, TMA, FP8": fp8 doubles matrix throughput at a cost in
precision.  Same page, section "Basse precision FP8 et incoherent processing":
Q and K are multiplied by a random orthogonal matrix, a Hadamard transform with
random signs applied per head in O(d log d), to spread outliers before
quantisation.  Readings taken where the page is silent: the normalised
Sylvester matrix H_d / sqrt(d); one seeded +-1 sign vector D shared by all
heads; Q' = Q D H, K' = K D H, V not rotated; one fp32 scale per tile of 128
tokens of one head (scale = amax / 448, 1 when the tile is all zero); codes are
OCP e4m3 (no infinities, max finite 448) rounded to nearest-even with
saturation at +-448.

Everything here is float64 except the stored scale, which is rounded to
float32 because that is what the quantised format carries.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
SCALE_TILE = 128


def e4m3_value(code):
    """Decode e4m3 codes (uint8 array-like) from the format definition.

    bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.
    exponent 0: subnormal, value 2^-6 * m/8.  S.1111.111 is NaN; no infinities.
    """
    c = np.asarray(code, dtype=np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


_POS_CODES = np.arange(0x7F, dtype=np.int64)          # 0x00..0x7E: all non-negative finite codes
_POS_VALS = e4m3_value(_POS_CODES)                     # strictly increasing with the code


def e4m3_code(x):
    """Round float64 values to e4m3 codes: nearest, ties to even mantissa, saturating.

    NaN -> 0x7F.  |x| >= 448 -> 0x7E (448) with the sign of x.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALS) - 1)
    d_hi = _POS_VALS[hi] - a
    d_lo = a - _POS_VALS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    code = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi])
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def e4m3_round(x):
    """Value of x after an e4m3 round trip (float64)."""
    return e4m3_value(e4m3_code(x))


def hadamard(d):
    """Normalised Sylvester-Hadamard matrix: H_1 = [1], H_2n = [[H, H], [H, -H]], / sqrt(d)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def rotate(x, signs):
    """x D H over the last axis (D = diag(signs)), float64."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    return (x * s) @ hadamard(x.shape[-1])


def quantize_rows(x, tile=SCALE_TILE):
    """Per-tile quantisation of x [B, H, N, d] along the token axis N.

    Returns (codes uint8 [B,H,N,d], scales float32 [B,H,ceil(N/tile)]).
    scale = float32(amax / 448) (1 for an all-zero tile); code = e4m3(x / scale).
    """
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    nt = -(-N // tile)
    scales = np.empty((B, H, nt), dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    for t in range(nt):
        blk = x[:, :, t * tile:(t + 1) * tile, :]
        amax = np.abs(blk).max(axis=(2, 3))
        sc = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
        scales[:, :, t] = sc
        codes[:, :, t * tile:(t + 1) * tile, :] = e4m3_code(blk / sc.astype(np.float64)[:, :, None, None])
    return codes, scales


def quantize_rows_split(x, tile=SCALE_TILE):
    """Two e4m3 codes per element sharing the tile scale of ``quantize_rows``.

    code1 = e4m3(x / scale) and code2 = e4m3(x / scale - value(code1)): the
    residual of the first rounding, rounded again on the same scale, so that
    value(code1) + value(code2) carries about 2 x 3 mantissa bits. Returns
    (code1, code2, scales). Not on the page: an e4m3 expansion of the rotated
    Q and K, taken because a single code misses the fp8 accuracy bar on
    inputs with outlier channels.
    """
    c1, sc = quantize_rows(x, tile)
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[2]
    rep = np.repeat(sc.astype(np.float64), tile, axis=2)[:, :, :N, None]
    t = np.clip(x / rep, -E4M3_MAX, E4M3_MAX)
    c2 = e4m3_code(t - e4m3_value(c1))
    return c1, c2, sc


def dequantize_rows(codes, scales, tile=SCALE_TILE):
    """Inverse of ``quantize_rows``: value(code) * scale, float64."""
    v = e4m3_value(codes)
    N = v.shape[2]
    rep = np.repeat(np.asarray(scales, dtype=np.float64), tile, axis=2)[:, :, :N]
    return v * rep[..., None]


def rope_tables(N, d, base=10000.0):
    """cos / sin of the rotary angles t * base^(-2i/d), t < N, i < d/2, float64 [N, d/2]."""
    t = np.arange(N, dtype=np.float64)[:, None]
    theta = base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    return np.cos(t * theta), np.sin(t * theta)


def rope(x, cos, sin):
    """Rotary position embedding of x [..., N, d] with the given tables [N, d/2].

    Dimension i (< d/2) is paired with i + d/2 and the pair is turned by the
    token's angle: (a, b) -> (a cos - b sin, a sin + b cos). Applied to Q and K
    before the Hadamard rotation: both are memory-bound passes over the same
    rows, so one kernel can do both ("FlashAttention-3 : ...", section "Basse
    precision FP8 et incoherent processing"). The pairing and the caller-given
    tables are readings; the page names the rotary embedding only.
    """
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def prepare(q, k, v, signs, tile=SCALE_TILE, rope_cos=None, rope_sin=None):
    """The fp8 prepare step: (optionally RoPE, then) rotate Q and K, then
    quantise Q, K, V per tile.

    Returns a dict with the rotated float64 inputs, (codes, scales) pairs for
    Q, K and V, and (value codes, residual codes, scales) for Q and K under
    "q_split" / "k_split".
    """
    if rope_cos is not None:
        q = rope(q, rope_cos, rope_sin)
        k = rope(k, rope_cos, rope_sin)
    qr = rotate(q, signs)
    kr = rotate(k, signs)
    vv = np.asarray(v, dtype=np.float64)
    return {
        "q_rot": qr, "k_rot": kr,
        "q": quantize_rows(qr, tile), "k": quantize_rows(kr, tile), "v": quantize_rows(vv, tile),
        "q_split": quantize_rows_split(qr, tile), "k_split": quantize_rows_split(kr, tile),
    }


def attention_emulated(q, k, v, signs, scale, block_n=64, p_shift=4, rotate_qk=True,
                       tile=SCALE_TILE, heads=None, lazy_tau=None, qk_codes=2):
    """fp8 emulation of the whole path, float64 arithmetic (no mask).

    Q, K (rotated when ``rotate_qk``) and V are quantised per tile of ``tile``
    tokens. With ``qk_codes`` = 2, Q and K carry a value code and a residual
    code on one scale (``quantize_rows_split``) and a score is the sum of the
    three products value.value + value.residual + residual.value (the
    residual.residual term, below 2^-8 of the score, is left out); with 1,
    value codes only. The online softmax walks key blocks of ``block_n``:
    running max m; each block's probabilities p = exp(s - m) are stored as
    e4m3(p * 2^p_shift * s_v / s_vmax) (s_v: the V scale of the block's tile,
    s_vmax: the largest V scale of the head) and multiply the V codes; the
    running sum uses the unrounded p; the output is rescaled by
    s_vmax / 2^p_shift at the end.

    ``lazy_tau`` (natural-log units) selects the other valid reference schedule:
    the exponent reference is moved to the running max only when that max has
    grown by more than lazy_tau (p then stays below e^lazy_tau); in exact
    arithmetic both schedules give the same O and LSE, in fp8 they round P on
    different grids.
    Returns (O, LSE) of the selected heads, [n, N, d] and [n, N].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if rotate_qk:
        q, k = rotate(q, signs), rotate(k, signs)
    if qk_codes == 2:
        q1, q2, qs = quantize_rows_split(q, tile)
        k1, k2, ks = quantize_rows_split(k, tile)
        qa, qb = dequantize_rows(q1, qs, tile), dequantize_rows(q2, qs, tile)
        ka, kb = dequantize_rows(k1, ks, tile), dequantize_rows(k2, ks, tile)
    elif qk_codes == 1:
        qa, ka = dequantize_rows(*quantize_rows(q, tile), tile), dequantize_rows(*quantize_rows(k, tile), tile)
        qb, kb = np.zeros_like(qa), np.zeros_like(ka)
    else:
        raise ValueError("qk_codes must be 1 or 2")
    vc, vs = quantize_rows(v, tile)
    v8 = e4m3_value(vc)
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    sel = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    Nk = k.shape[2]
    outs, lses = [], []
    two = float(2 ** p_shift)
    for b, h in sel:
        g = h // G
        svmax = float(vs[b, g].max())
        m = np.full(N, -np.inf)
        l = np.zeros(N)
        acc = np.zeros((N, d))
        for j0 in range(0, Nk, block_n):
            cols = slice(j0, min(j0 + block_n, Nk))
            s = scale * (qa[b, h] @ ka[b, g, cols].T + qa[b, h] @ kb[b, g, cols].T + qb[b, h] @ ka[b, g, cols].T)
            m_new = np.maximum(m, s.max(axis=1))
            if lazy_tau is not None:
                m_new = np.where(np.isfinite(m) & (m_new <= m + lazy_tau), m, m_new)
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
            p = np.exp(s - m_new[:, None])
            l = alpha * l + p.sum(axis=1)
            r = float(vs[b, g, j0 // tile]) / svmax
            p8 = e4m3_round(p * two * r)
            acc = alpha[:, None] * acc + p8 @ v8[b, g, cols]
            m = m_new
        outs.append(acc * (svmax / two) / l[:, None])
        lses.append(m + np.log(l))
    return np.stack(outs), np.stack(lses)
