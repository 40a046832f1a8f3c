"""Pins of the paged-decode oracle (``oracle.attention.decode_paged``).

* identity block table: equals the plain attention of the last query over the
  contiguous sequence (and the brute-force loops on a tiny case);
* permuting physical blocks (and the table with them) changes nothing;
* the split-and-merge identity the GPU path uses: attention over two halves of
  the keys, merged by LSE = logaddexp(LSE_1, LSE_2), O = sum exp(LSE_s - LSE) O_s,
  equals attention over all keys.
"""
import numpy as np

from oracle import attention as A
from tests import brute


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _paged(kv, bs, perm=None):
    """kv [Hkv, n, d] contiguous -> cache [nb, Hkv, bs, d] and its table (optionally permuted)."""
    Hkv, n, d = kv.shape
    nb = -(-n // bs)
    pad = np.zeros((Hkv, nb * bs, d))
    pad[:, :n] = kv
    blocks = pad.reshape(Hkv, nb, bs, d).transpose(1, 0, 2, 3)
    order = np.arange(nb) if perm is None else perm
    cache = np.empty_like(blocks)
    cache[order] = blocks          # logical block i stored at physical order[i]
    return cache, order


def test_identity_table_equals_contiguous_attention_and_brute_force():
    Hq, Hkv, d, n = 4, 2, 8, 37
    q = _rand((1, Hq, d), 1)
    k, v = _rand((Hkv, n, d), 2), _rand((Hkv, n, d), 3)
    kc, bt = _paged(k, 16)
    vc, _ = _paged(v, 16)
    O, L = A.decode_paged(q, kc, vc, bt[None], [n], 0.3)
    Oc, Lc = A.attention(q[:, :, None, :], k[None], v[None], 0.3, threads=1)
    np.testing.assert_allclose(O, Oc[:, :, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L, Lc[:, :, 0], rtol=0, atol=1e-14)
    Ob, Lb = brute.attend([q[0][:, None, :].tolist()], [k.tolist()], [v.tolist()], 0.3)
    np.testing.assert_allclose(O[0], np.array(Ob[0])[:, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(L[0], np.array(Lb[0])[:, 0], rtol=0, atol=1e-13)


def test_block_permutation_changes_nothing():
    Hq, Hkv, d = 2, 1, 4
    lens = [33, 5]
    q = _rand((2, Hq, d), 4)
    outs = []
    for perm_seed in (None, 7):
        kcs, vcs, tables, base = [], [], [], 0
        for b, n in enumerate(lens):
            k, v = _rand((Hkv, n, d), 10 + b), _rand((Hkv, n, d), 20 + b)
            nb = -(-n // 16)
            perm = None if perm_seed is None else np.random.default_rng(perm_seed + b).permutation(nb)
            kc, order = _paged(k, 16, perm)
            vc, _ = _paged(v, 16, perm)
            kcs.append(kc)
            vcs.append(vc)
            row = np.zeros(3, dtype=np.int64)
            row[:nb] = order + base
            tables.append(row)
            base += nb
        outs.append(A.decode_paged(q, np.concatenate(kcs), np.concatenate(vcs), np.stack(tables), lens, 0.5))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_split_merge_identity():
    Hq, Hkv, d, n = 2, 2, 8, 50
    q = _rand((1, Hq, 1, d), 5)
    k, v = _rand((1, Hkv, n, d), 6), _rand((1, Hkv, n, d), 7)
    O, L = A.attention(q, k, v, 0.4, threads=1)
    parts = [A.attention(q, k[:, :, a:b], v[:, :, a:b], 0.4, threads=1) for a, b in ((0, 21), (21, 50))]
    Lm = np.logaddexp(parts[0][1], parts[1][1])
    Om = sum(np.exp(l - Lm)[..., None] * o for o, l in parts)
    np.testing.assert_allclose(Om, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lm, L, rtol=0, atol=1e-13)
