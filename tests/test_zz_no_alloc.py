"""attn_decode_paged_noalloc (fixed device scratch, no allocation) against
attn_decode_paged with a caller workspace, through the C ABI: two calls in a
row, the second with a smaller input, each bit-identical to the allocating
entry point (same kernels), and the reference itself within the decode bars
of the oracle; sizes beyond the scratch are rejected before any launch."""
import pytest
import torch

from oracle import attention as A
from tests.gpu_util import assert_close
from tiled_attention_05_amd import _lib
from tiled_attention_05_amd import inputs as I

pytestmark = pytest.mark.gpu


def _noalloc(q, kc, vc, bt, sl, splits):
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq), 7.0, device="cuda")
    st = _lib.attn_decode_paged_noalloc(q, kc, vc, bt, sl, o, lse, B, Hq, Hkv, d, 16, bt.shape[1], d ** -0.5,
                                        splits, _lib.BF16)
    return st, o, lse


@pytest.mark.parametrize("first,second", [
    ((8, 32, 8, [300, 4096, 17, 1000, 5000, 64, 2048, 1], 8), (3, 8, 2, [77, 1500, 16], 4)),
    ((64, 32, 8, None, 8), (5, 4, 1, [0, 33, 700, 16, 48], 3)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for i, (B, Hq, Hkv, lens, splits) in enumerate((first, second)):
        if lens is None:
            lens = I.decode_lengths(I.WORKLOADS[7])[:B]
        print(f"[case] noalloc call {i + 1}: B={B} Hq={Hq} Hkv={Hkv} splits={splits} lens={lens[:6]}", flush=True)
        q, kc, vc, bt, sl = (t.cuda() for t in I.decode_inputs(B, Hq, Hkv, 128, lens, seed=11 + i))
        st, o, lse = _noalloc(q, kc, vc, bt, sl, splits)
        assert st == _lib.OK, _lib.attn_status_string(st)
        o_ref, l_ref = _lib.decode_paged(q, kc, vc, bt, sl, scale=128 ** -0.5, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"call {i + 1}: O differs"
        assert torch.equal(lse, l_ref), f"call {i + 1}: LSE differs"
        O, L = A.decode_paged(q.cpu(), kc.cpu(), vc.cpu(), bt.cpu(), sl.cpu(), 128 ** -0.5)
        assert_close(o, lse, O, L, label=f"noalloc call {i + 1}")


def test_noalloc_rejects_sizes_beyond_the_scratch():
    q, kc, vc, bt, sl = (t.cuda() for t in I.decode_inputs(2, 4, 2, 128, [16, 16], seed=3))
    # 256 sequences x 64 heads x 16 splits x 129 floats > 4 * 2^20: rejected before any launch
    big_q = torch.zeros(256, 64, 128, dtype=torch.bfloat16, device="cuda")
    big_sl = torch.zeros(256, dtype=torch.int32, device="cuda")
    big_bt = torch.zeros(256, 1, dtype=torch.int32, device="cuda")
    o = torch.empty_like(big_q)
    st = _lib.attn_decode_paged_noalloc(big_q, kc, vc, big_bt, big_sl, o, None, 256, 64, 2, 128, 16, 1, 0.1, 16,
                                        _lib.BF16)
    assert st == _lib.ERR_INVALID_ARG
    # one split needs no scratch at all
    st, o1, _ = _noalloc(q, kc, vc, bt, sl, 1)
    torch.cuda.synchronize()
    assert st == _lib.OK
