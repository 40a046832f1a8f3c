"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects invalid or unsupported arguments before any HIP call (no compute call
is made here: every call below fails validation and returns immediately)."""
import ctypes
import math
import os
import re

import pytest

from tiled_attention_05_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 0x1000   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding():
    text = open(HEADER).read()
    vals = dict(re.findall(r"\b(ATTN_\w+)\s*=\s*(-?\d+)", text))
    assert int(vals["ATTN_OK"]) == _lib.OK
    assert int(vals["ATTN_ERR_INVALID_ARG"]) == _lib.ERR_INVALID_ARG
    assert int(vals["ATTN_ERR_UNSUPPORTED"]) == _lib.ERR_UNSUPPORTED
    assert int(vals["ATTN_ERR_HIP"]) == _lib.ERR_HIP
    assert (int(vals["ATTN_F32"]), int(vals["ATTN_BF16"]), int(vals["ATTN_FP8_E4M3"])) == (0, 1, 2)
    assert (int(vals["ATTN_MASK_CAUSAL"]), int(vals["ATTN_MASK_WINDOW"]), int(vals["ATTN_MASK_DOC"])) == \
        (_lib.MASK_CAUSAL, _lib.MASK_WINDOW, _lib.MASK_DOC)


def test_status_strings(lib):
    for s in (0, -1, -2, -3):
        txt = _lib.attn_status_string(s)
        assert txt and txt != "unknown status"
    assert _lib.attn_status_string(12345) == "unknown status"


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, Nq=16, Nk=16, d=128, scale=0.1,
             mask=0, window=0, doc=None, softcap=0.0, slopes=None, dtype=1)
    a.update(kw)
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                        a["Nk"], a["d"], a["scale"], a["mask"], a["window"], a["doc"], a["softcap"],
                        a["slopes"], a["dtype"], None)


INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None),
    dict(B=0), dict(Hq=0), dict(Hkv=0), dict(Nq=0), dict(Nk=-3), dict(d=0),
    dict(Hq=3, Hkv=2),
    dict(scale=math.nan), dict(scale=math.inf),
    dict(softcap=-1.0), dict(softcap=math.nan),
    dict(mask=8), dict(mask=3, window=0), dict(mask=4, doc=None), dict(dtype=7),
]
UNSUPPORTED = [
    dict(d=96), dict(d=256), dict(mask=2, window=4), dict(mask=4, doc=FAKE, Nq=8, Nk=16),
    dict(dtype=2, mask=1), dict(dtype=2, d=64), dict(dtype=2, Nq=8, Nk=16), dict(dtype=2, softcap=5.0),
    dict(dtype=2, slopes=FAKE),
]


@pytest.mark.parametrize("kw", INVALID)
def test_fwd_rejects_invalid(lib, kw):
    assert _fwd(lib, **kw) == _lib.ERR_INVALID_ARG


@pytest.mark.parametrize("kw", UNSUPPORTED)
def test_fwd_rejects_unsupported(lib, kw):
    assert _fwd(lib, **kw) == _lib.ERR_UNSUPPORTED


def _varlen(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, cu=FAKE, ns=3, total=100, Hq=2, Hkv=2, d=128, scale=0.1,
             mask=1, window=0, softcap=0.0, slopes=None, ws=FAKE, dtype=1)
    a.update(kw)
    return lib.attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["ns"], a["total"], a["Hq"],
                               a["Hkv"], a["d"], a["scale"], a["mask"], a["window"], a["softcap"], a["slopes"],
                               a["ws"], a["dtype"], None)


VARLEN_INVALID = [
    dict(cu=None), dict(ws=None), dict(q=None), dict(o=None), dict(ns=0), dict(total=0),
    dict(mask=4), dict(mask=5), dict(mask=8), dict(mask=3, window=0), dict(Hq=3, Hkv=2),
    dict(scale=math.nan), dict(softcap=-2.0), dict(dtype=9),
]
VARLEN_UNSUPPORTED = [dict(dtype=2), dict(d=96), dict(mask=2, window=8)]


@pytest.mark.parametrize("kw", VARLEN_INVALID)
def test_fwd_varlen_rejects_invalid(lib, kw):
    assert _varlen(lib, **kw) == _lib.ERR_INVALID_ARG


@pytest.mark.parametrize("kw", VARLEN_UNSUPPORTED)
def test_fwd_varlen_rejects_unsupported(lib, kw):
    assert _varlen(lib, **kw) == _lib.ERR_UNSUPPORTED


def test_fp8_buffer_bytes(lib):
    # 300 tokens -> 384 padded rows of 128 bytes in two code planes (value,
    # residual), 3 float32 scales per head
    assert _lib.attn_fp8_buffer_bytes(2, 3, 300, 128) == 2 * (2 * 3 * 384 * 128) + 2 * 3 * 3 * 4
    assert _lib.attn_fp8_buffer_bytes(0, 3, 300, 128) == 0


def test_fp8_prepare_validation(lib):
    f = lib.attn_fp8_prepare
    assert f(None, FAKE, FAKE, 1, 1, 1, 8, 128, FAKE, FAKE, FAKE, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, 1, 3, 2, 8, 128, FAKE, FAKE, FAKE, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, 1, 2, 2, 8, 128, FAKE, None, FAKE, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, 1, 2, 2, 8, 64, FAKE, FAKE, FAKE, FAKE, None) == _lib.ERR_UNSUPPORTED


def test_fp8_prepare_rope_validation(lib):
    f = lib.attn_fp8_prepare_rope
    ok = (FAKE, FAKE, FAKE, 1, 2, 2, 8, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    for i, want in ((9, _lib.ERR_INVALID_ARG), (10, _lib.ERR_INVALID_ARG), (0, _lib.ERR_INVALID_ARG),
                    (11, _lib.ERR_INVALID_ARG)):
        a = list(ok)
        a[i] = None
        assert f(*a) == want
    a = list(ok)
    a[7] = 64
    assert f(*a) == _lib.ERR_UNSUPPORTED


def test_block_mask_validation(lib):
    assert _lib.attn_block_mask_bytes(1, 100, 100, 0, 64) == 0
    assert _lib.attn_block_mask_bytes(1, 100, 100, 8192, 64) == 0
    n = _lib.attn_block_mask_bytes(2, 100, 130, 32, 64)
    assert n == ((2 * 4 * 3 + 15) // 16) * 16 + 2 * 4 * 3 * 4 + 4
    f = lib.attn_block_mask_build
    assert f(1, 100, 100, 1, 0, None, 32, 64, None, None) == _lib.ERR_INVALID_ARG
    assert f(1, 100, 100, 1, 0, None, 0, 64, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(1, 100, 100, 16, 0, None, 32, 64, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(1, 100, 100, 4, 0, None, 32, 64, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(1, 100, 100, 2, 5, None, 32, 64, FAKE, None) == _lib.ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_no_device_calls_return_hip_error(lib):
    """With no GPU present, a call that passes validation reaches the HIP launch
    and returns ATTN_ERR_HIP; nothing crashes. Skipped wherever a GPU is
    visible: the pointers here are fake and must never reach a real launch."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")
    F = FAKE
    calls = {
        "fwd": lambda: lib.attn_fwd(F, F, F, F, None, 1, 2, 2, 16, 16, 128, 0.1, 0, 0, None, 0.0, None, 1, None),
        "fwd_fp8": lambda: lib.attn_fwd(F, F, F, F, None, 1, 2, 2, 16, 16, 128, 0.1, 0, 0, None, 0.0, None, 2,
                                        None),
        "varlen": lambda: lib.attn_fwd_varlen(F, F, F, F, None, F, 2, 16, 2, 2, 128, 0.1, 1, 0, 0.0, None, F, 1,
                                              None),
        "prepare": lambda: lib.attn_fp8_prepare(F, F, F, 1, 2, 2, 16, 128, None, F, F, F, None),
        "block_mask": lambda: lib.attn_block_mask_build(1, 16, 16, 1, 0, None, 32, 64, F, None),
        "tile_kinds": lambda: lib.attn_fwd_tile_kinds(1, 16, 16, 1, 0, None, F, None),
        "decode": lambda: lib.attn_decode_paged(F, F, F, F, F, F, None, 1, 2, 2, 128, 16, 4, 0.1, 1, None, 1, None),
        "decode_noalloc": lambda: lib.attn_decode_paged_noalloc(F, F, F, F, F, F, None, 1, 2, 2, 128, 16, 4, 0.1, 2,
                                                                1, None),
        "bwd": lambda: lib.attn_bwd(F, F, F, F, F, F, F, F, F, F, 1, 2, 2, 16, 128, 0.1, 1, 1, None),
    }
    for name, call in calls.items():
        assert call() == _lib.ERR_HIP, name
