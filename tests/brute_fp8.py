"""Pure-Python brute force of the fp8 scheme on tiny inputs (a pin of the
oracle's fp8 emulation, written without numpy and without oracle/).

Each step is taken from its definition:
  * e4m3 (OCP): 3 mantissa bits, exponent bias 7, normals down to 2^-6,
    subnormals spaced 2^-9, largest finite 448; rounding to the nearest
    representable value, ties to the even mantissa, saturating at +-448;
  * the normalised Sylvester-Hadamard matrix, entry (i, j) equal to
    (-1)^popcount(i & j) / sqrt(d), applied after the +-1 sign flip;
  * one float32 scale per tile of tokens of one head: amax / 448 (1 when the
    tile is all zero);
  * Q and K as value + residual codes on one scale (the residual is the first
    rounding's error, rounded again), a score summing value.value,
    value.residual and residual.value;
  * online softmax over key blocks with a running exponent reference that
    moves only when the block max exceeds it by more than ``tau`` (natural
    log units; None = always), P stored as e4m3(p * 2^shift * s_v / s_vmax),
    the running sum on the unrounded p, O rescaled by s_vmax / 2^shift.
"""
import math
import struct


def f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def e4m3(x):
    """Nearest e4m3 value of x (ties to even mantissa), saturating at +-448."""
    if x == 0.0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = min(abs(x), 448.0)
    e = math.frexp(a)[1] - 1            # a in [2^e, 2^(e+1))
    step = 2.0 ** (max(e, -6) - 3)     # spacing in this binade (subnormals: 2^-9)
    n = a / step                        # exact: step is a power of two
    fl = math.floor(n)
    r = n - fl
    if r > 0.5 or (r == 0.5 and fl % 2 == 1):
        fl += 1
    return sign * min(fl * step, 448.0)


def hadamard_row_times(x, signs):
    d = len(x)
    y = [x[c] * signs[c] for c in range(d)]
    return [math.fsum(y[i] * (-1.0) ** bin(i & j).count("1") for i in range(d)) / math.sqrt(d)
            for j in range(d)]


def quantise(rows, tile, split):
    """rows: list over tokens of lists over d. Returns (values, residuals, scales per tile)."""
    N = len(rows)
    vals, res, scales = [], [], []
    for t0 in range(0, N, tile):
        blk = rows[t0:t0 + tile]
        amax = max(abs(x) for r in blk for x in r)
        s = f32(amax / 448.0) if amax > 0 else 1.0
        scales.append(s)
        for r in blk:
            t = [max(-448.0, min(448.0, x / s)) for x in r]
            c1 = [e4m3(x) for x in t]
            vals.append([c * s for c in c1])
            res.append([e4m3(x - c) * s if split else 0.0 for x, c in zip(t, c1)])
    return vals, res, scales


def attend_fp8(q, k, v, signs, scale, tile, block, shift=4, tau=None, split=True, rotate=True):
    """q, k, v: [N][d] lists of one head. Returns (O [N][d], LSE [N])."""
    if rotate:
        q = [hadamard_row_times(r, signs) for r in q]
        k = [hadamard_row_times(r, signs) for r in k]
    qa, qb, _ = quantise(q, tile, split)
    ka, kb, _ = quantise(k, tile, split)
    v8, _, vs = quantise(v, tile, False)
    vcode = [[x / vs[j // tile] for x in r] for j, r in enumerate(v8)]   # the e4m3 values themselves
    svmax = max(vs)
    N, Nk, d = len(q), len(k), len(v[0])
    O, L = [], []
    for i in range(N):
        m, l = -math.inf, 0.0
        acc = [0.0] * d
        for j0 in range(0, Nk, block):
            js = range(j0, min(j0 + block, Nk))
            s = {j: scale * math.fsum(qa[i][c] * ka[j][c] + qa[i][c] * kb[j][c] + qb[i][c] * ka[j][c]
                                      for c in range(d)) for j in js}
            mb = max(s.values())
            m_new = max(m, mb)
            if tau is not None and m != -math.inf and m_new <= m + tau:
                m_new = m
            alpha = math.exp(m - m_new) if m != -math.inf else 0.0
            p = {j: math.exp(s[j] - m_new) for j in js}
            l = alpha * l + math.fsum(p.values())
            r = vs[j0 // tile] / svmax
            p8 = {j: e4m3(p[j] * 2.0 ** shift * r) for j in js}
            acc = [alpha * acc[c] + math.fsum(p8[j] * vcode[j][c] for j in js) for c in range(d)]
            m = m_new
        O.append([a * svmax / 2.0 ** shift / l for a in acc])
        L.append(m + math.log(l))
    return O, L
