"""Pure-Python brute-force attention for tiny inputs (an oracle pin, not the oracle).

Written independently of ``oracle/``: nested loops, ``math.exp``, ``math.tanh``
and ``math.fsum`` over Python floats.  Used only on inputs of a few tokens.
"""
import math


def attend(q, k, v, scale, causal=False, window=0, docs=None, softcap=0.0, slopes=None):
    """q: [B][Hq][Nq][d] nested lists; k, v: [B][Hkv][Nk][d]. Returns (O, LSE) nested lists."""
    B, Hq, Nq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Nk = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    O, L = [], []
    for b in range(B):
        Ob, Lb = [], []
        for h in range(Hq):
            g = h // group
            Oh, Lh = [], []
            for i in range(Nq):
                ii = i + (Nk - Nq)              # query position on the key axis
                s = {}
                for j in range(Nk):
                    if causal and j > ii:
                        continue
                    if window and ii - j >= window:
                        continue
                    if docs is not None and docs[b][i] != docs[b][j]:
                        continue
                    x = scale * math.fsum(q[b][h][i][c] * k[b][g][j][c] for c in range(d))
                    if softcap > 0:
                        x = softcap * math.tanh(x / softcap)
                    if slopes is not None:
                        x -= slopes[h] * (i - j)
                    s[j] = x
                if not s:
                    Oh.append([0.0] * d)
                    Lh.append(-math.inf)
                    continue
                m = max(s.values())
                w = {j: math.exp(x - m) for j, x in s.items()}
                tot = math.fsum(w.values())
                Oh.append([math.fsum(w[j] * v[b][g][j][c] for j in w) / tot for c in range(d)])
                Lh.append(m + math.log(tot))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return O, L
