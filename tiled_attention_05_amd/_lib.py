"""ctypes binding of libattn.so (the C ABI declared in include/attn.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels. PyTorch provides device memory and the current stream. The
low-level functions keep the C names and return the C status; the helpers
``fwd``, ``fp8_prepare`` and ``block_mask`` allocate outputs with torch and
raise ``AttnError`` on a non-zero status. There is no fallback: without the
built library every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

import torch

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
# the same library with the forward kernels built -DATTN_SINGLE_STAGE (tests only)
PATH_SINGLE_STAGE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_single_stage.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP = 0, -1, -2, -3
F32, BF16, FP8_E4M3 = 0, 1, 2
MASK_NONE, MASK_CAUSAL, MASK_WINDOW, MASK_DOC = 0, 1, 2, 4
FP8_TILE = 128

EXPORTS = ("attn_fwd", "attn_fwd_varlen", "attn_fp8_buffer_bytes", "attn_fp8_prepare", "attn_fp8_prepare_rope",
           "attn_block_mask_bytes", "attn_block_mask_build", "attn_fwd_tile_kinds_bytes", "attn_fwd_tile_kinds",
           "attn_decode_workspace_floats", "attn_decode_paged", "attn_decode_paged_noalloc", "attn_bwd",
           "attn_status_string")

_lib = None
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


def load():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(PATH)
    return _lib


@contextlib.contextmanager
def library(path):
    """Route every call made inside the block through the library at path
    (another build of the same C ABI, e.g. PATH_SINGLE_STAGE)."""
    global _lib
    saved = _lib
    _lib = _open(path)
    try:
        yield _lib
    finally:
        _lib = saved


def _open(path):
    """Load the library at path and declare the C signatures of include/attn.h."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with `python -m tiled_attention_05_amd.build`")
    lib = ctypes.CDLL(path)
    lib.attn_fwd.restype = _i
    lib.attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _f, _vp,
                             _i, _vp]
    lib.attn_fwd_varlen.restype = _i
    lib.attn_fwd_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _f, _vp,
                                    _vp, _i, _vp]
    lib.attn_fp8_buffer_bytes.restype = _sz
    lib.attn_fp8_buffer_bytes.argtypes = [_i, _i, _i, _i]
    lib.attn_fp8_prepare.restype = _i
    lib.attn_fp8_prepare.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]
    lib.attn_fp8_prepare_rope.restype = _i
    lib.attn_fp8_prepare_rope.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp]
    lib.attn_decode_workspace_floats.restype = _sz
    lib.attn_decode_workspace_floats.argtypes = [_i, _i, _i, _i]
    lib.attn_decode_paged.restype = _i
    lib.attn_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp,
                                      _i, _vp]
    lib.attn_decode_paged_noalloc.restype = _i
    lib.attn_decode_paged_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                              _i, _i, _vp]
    lib.attn_bwd.restype = _i
    lib.attn_bwd.argtypes = [_vp] * 10 + [_i, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.attn_block_mask_bytes.restype = _sz
    lib.attn_block_mask_bytes.argtypes = [_i, _i, _i, _i, _i]
    lib.attn_block_mask_build.restype = _i
    lib.attn_block_mask_build.argtypes = [_i, _i, _i, _i, _i, _vp, _i, _i, _vp, _vp]
    lib.attn_fwd_tile_kinds_bytes.restype = _sz
    lib.attn_fwd_tile_kinds_bytes.argtypes = [_i, _i, _i]
    lib.attn_fwd_tile_kinds.restype = _i
    lib.attn_fwd_tile_kinds.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, _vp]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [_i]
    return lib


def _ptr(t):
    return None if t is None else (t if isinstance(t, int) else t.data_ptr())


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ------------------------------------------------------------------ C names
def attn_status_string(status: int) -> str:
    return load().attn_status_string(status).decode()


status_string = attn_status_string


def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, mask_kind, window, doc_ids, softcap,
             alibi_slopes, dtype, stream=None) -> int:
    return load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, scale,
                           mask_kind, window, _ptr(doc_ids), softcap, _ptr(alibi_slopes), dtype,
                           _stream(stream))


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, num_seqs, total, Hq, Hkv, d, scale, mask_kind, window,
                    softcap, alibi_slopes, workspace, dtype, stream=None) -> int:
    return load().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), num_seqs,
                                  total, Hq, Hkv, d, scale, mask_kind, window, softcap, _ptr(alibi_slopes),
                                  _ptr(workspace), dtype, _stream(stream))


def attn_fp8_buffer_bytes(B, H, N, d) -> int:
    return load().attn_fp8_buffer_bytes(B, H, N, d)


def attn_fp8_prepare(q, k, v, B, Hq, Hkv, N, d, signs, q8, k8, v8, stream=None) -> int:
    return load().attn_fp8_prepare(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N, d, _ptr(signs), _ptr(q8),
                                   _ptr(k8), _ptr(v8), _stream(stream))


def attn_fp8_prepare_rope(q, k, v, B, Hq, Hkv, N, d, signs, rope_cos, rope_sin, q8, k8, v8, stream=None) -> int:
    return load().attn_fp8_prepare_rope(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N, d, _ptr(signs), _ptr(rope_cos),
                                        _ptr(rope_sin), _ptr(q8), _ptr(k8), _ptr(v8), _stream(stream))


def attn_decode_workspace_floats(B, Hq, d, num_splits) -> int:
    return load().attn_decode_workspace_floats(B, Hq, d, num_splits)


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv, d, block_size, max_blocks,
                      scale, num_splits, workspace, dtype, stream=None) -> int:
    return load().attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                    _ptr(o), _ptr(lse), B, Hq, Hkv, d, block_size, max_blocks, scale, num_splits,
                                    _ptr(workspace), dtype, _stream(stream))


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv, d, block_size,
                              max_blocks, scale, num_splits, dtype, stream=None) -> int:
    return load().attn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                            _ptr(seq_lens), _ptr(o), _ptr(lse), B, Hq, Hkv, d, block_size,
                                            max_blocks, scale, num_splits, dtype, _stream(stream))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, Hq, Hkv, N, d, scale, mask_kind, dtype,
             stream=None) -> int:
    return load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                           _ptr(workspace), B, Hq, Hkv, N, d, scale, mask_kind, dtype, _stream(stream))


def attn_block_mask_bytes(B, Nq, Nk, block_m, block_n) -> int:
    return load().attn_block_mask_bytes(B, Nq, Nk, block_m, block_n)


def attn_block_mask_build(B, Nq, Nk, mask_kind, window, doc_ids, block_m, block_n, out, stream=None) -> int:
    return load().attn_block_mask_build(B, Nq, Nk, mask_kind, window, _ptr(doc_ids), block_m, block_n,
                                        _ptr(out), _stream(stream))


def attn_fwd_tile_kinds_bytes(B, Nq, Nk) -> int:
    return load().attn_fwd_tile_kinds_bytes(B, Nq, Nk)


def attn_fwd_tile_kinds(B, Nq, Nk, mask_kind, window, doc_ids, out, stream=None) -> int:
    return load().attn_fwd_tile_kinds(B, Nq, Nk, mask_kind, window, _ptr(doc_ids), _ptr(out), _stream(stream))


# ------------------------------------------------------------------ helpers
def _need(t, name, dtype=None, ndim=None, shape=None, numel=None):
    """Check a device tensor argument; ``shape`` (exact) or ``numel`` (a lower
    bound) guard the extent the kernels will read or write."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA/HIP tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} must hold at least {numel} elements, got {t.numel()}")


def fwd(q, k, v, scale=None, mask=MASK_NONE, window=0, doc_ids=None, softcap=0.0, alibi_slopes=None,
        with_lse=True, out=None, lse=None, stream=None):
    """O (and LSE) of the fused forward for fp32 / bf16 BHSD tensors."""
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(q.dtype)
    if dt is None:
        raise ValueError("q must be float32 or bfloat16 (fp8: use fwd_fp8)")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, 4)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if v.shape != k.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    if doc_ids is not None:
        _need(doc_ids, "doc_ids", torch.int32, shape=(B, Nk))
    if alibi_slopes is not None:
        _need(alibi_slopes, "alibi_slopes", torch.float32, 1, numel=Hq)
    if out is not None:
        _need(out, "out", q.dtype, shape=q.shape)
    if with_lse and lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq, Nq))
    o = torch.empty_like(q) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty(B, Hq, Nq, device=q.device, dtype=torch.float32)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = attn_fwd(q, k, v, o, lse if with_lse else None, B, Hq, Hkv, Nq, Nk, d, sc, mask, window, doc_ids,
                  softcap, alibi_slopes, dt, stream)
    if st:
        raise AttnError(st, "attn_fwd")
    return (o, lse) if with_lse else o


def fwd_varlen(q, k, v, cu_seqlens, scale=None, mask=MASK_NONE, window=0, softcap=0.0, alibi_slopes=None,
               with_lse=True, out=None, lse=None, workspace=None, stream=None):
    """Forward over packed sequences: q [Hq, total, d], k / v [Hkv, total, d],
    cu_seqlens int32 [num_seqs + 1] on the device (sequence s owns tokens
    cu_seqlens[s] .. cu_seqlens[s + 1] - 1)."""
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(q.dtype)
    if dt is None:
        raise ValueError("q must be float32 or bfloat16")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, 3)
    Hq, total, d = q.shape
    Hkv = k.shape[0]
    if v.shape != k.shape or k.shape[1] != total or k.shape[2] != d:
        raise ValueError("k and v must be [Hkv, total, d] matching q")
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, numel=2)
    if alibi_slopes is not None:
        _need(alibi_slopes, "alibi_slopes", torch.float32, 1, numel=Hq)
    if out is not None:
        _need(out, "out", q.dtype, shape=q.shape)
    if with_lse and lse is not None:
        _need(lse, "lse", torch.float32, shape=(Hq, total))
    if workspace is not None:
        _need(workspace, "workspace", torch.int32, numel=total)
    o = torch.empty_like(q) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty(Hq, total, device=q.device, dtype=torch.float32)
    ws = torch.empty(total, device=q.device, dtype=torch.int32) if workspace is None else workspace
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = attn_fwd_varlen(q, k, v, o, lse if with_lse else None, cu_seqlens, cu_seqlens.numel() - 1, total, Hq,
                         Hkv, d, sc, mask, window, softcap, alibi_slopes, ws, dt, stream)
    if st:
        raise AttnError(st, "attn_fwd_varlen")
    return (o, lse) if with_lse else o


def bwd(q, k, v, o, dout, lse, scale=None, mask=MASK_NONE, workspace=None, stream=None):
    """(dQ, dK, dV) of the forward for output gradient dout (bf16 BHSD, d = 128)."""
    _need(q, "q", torch.bfloat16, 4)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1] if isinstance(k, torch.Tensor) and k.dim() == 4 else 0
    for t, n, shp in ((k, "k", (B, Hkv, N, d)), (v, "v", (B, Hkv, N, d)), (o, "o", q.shape),
                      (dout, "dout", q.shape)):
        _need(t, n, torch.bfloat16, shape=shp)
    _need(lse, "lse", torch.float32, shape=(B, Hq, N))
    if workspace is not None:
        _need(workspace, "workspace", torch.float32, numel=B * Hq * N)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(B * Hq * N, device=q.device, dtype=torch.float32) if workspace is None else workspace
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, B, Hq, Hkv, N, d, sc, mask, BF16, stream)
    if st:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale=None, num_splits=1, with_lse=True, out=None,
                 lse=None, workspace=None, stream=None):
    """One-token decode over a paged cache: q [B, Hq, d]; caches [num_blocks, Hkv, block_size, d];
    block_table int32 [B, max_blocks]; seq_lens int32 [B] (device tensors)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, d = q.shape
    _need(block_table, "block_table", torch.int32, 2)
    if block_table.shape[0] != B:
        raise ValueError(f"block_table must have {B} rows")
    _need(seq_lens, "seq_lens", torch.int32, shape=(B,))
    _, Hkv, bs, _ = k_cache.shape
    if v_cache.shape != k_cache.shape or k_cache.shape[3] != d:
        raise ValueError("caches must be [num_blocks, Hkv, block_size, d] matching q")
    if out is not None:
        _need(out, "out", torch.bfloat16, shape=q.shape)
    if with_lse and lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq))
    o = torch.empty_like(q) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    n = attn_decode_workspace_floats(B, Hq, d, num_splits)
    if workspace is not None and n > 0:
        _need(workspace, "workspace", torch.float32, numel=n)
    ws = workspace
    if ws is None and n > 0:
        ws = torch.empty(n, device=q.device, dtype=torch.float32)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse if with_lse else None, B, Hq, Hkv,
                           d, bs, block_table.shape[1], sc, num_splits, ws, BF16, stream)
    if st:
        raise AttnError(st, "attn_decode_paged")
    return (o, lse) if with_lse else o


def fp8_prepare(q, k, v, signs, stream=None, rope_cos=None, rope_sin=None):
    """Rotate Q, K (random-sign Hadamard; none if signs is None) and quantise Q, K, V
    to packed e4m3 buffers. With rope_cos / rope_sin (float32 [N, d/2]) the
    rotary embedding of Q and K runs first, in the same kernel."""
    _need(q, "q", torch.bfloat16, 4)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1] if isinstance(k, torch.Tensor) and k.dim() == 4 else 0
    _need(k, "k", torch.bfloat16, shape=(B, Hkv, N, d))
    _need(v, "v", torch.bfloat16, shape=(B, Hkv, N, d))
    if signs is not None:
        _need(signs, "signs", torch.int8, shape=(d,))
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("rope_cos and rope_sin go together")
    if rope_cos is not None:
        _need(rope_cos, "rope_cos", torch.float32, 2)
        _need(rope_sin, "rope_sin", torch.float32, 2)
        if rope_cos.shape != (q.shape[2], q.shape[3] // 2) or rope_sin.shape != rope_cos.shape:
            raise ValueError("rope tables must be [N, d/2]")
    nq = attn_fp8_buffer_bytes(B, Hq, N, d)
    nk = attn_fp8_buffer_bytes(B, Hkv, N, d)
    q8 = torch.empty(nq, dtype=torch.uint8, device=q.device)
    k8 = torch.empty(nk, dtype=torch.uint8, device=q.device)
    v8 = torch.empty(nk, dtype=torch.uint8, device=q.device)
    if rope_cos is None:
        st = attn_fp8_prepare(q, k, v, B, Hq, Hkv, N, d, signs, q8, k8, v8, stream)
    else:
        st = attn_fp8_prepare_rope(q, k, v, B, Hq, Hkv, N, d, signs, rope_cos, rope_sin, q8, k8, v8, stream)
    if st:
        raise AttnError(st, "attn_fp8_prepare")
    return q8, k8, v8


def fwd_fp8(q8, k8, v8, B, Hq, Hkv, N, d, scale=None, with_lse=True, stream=None, out=None, lse=None):
    """O (bf16) and LSE of the fp8 forward on buffers written by fp8_prepare."""
    for t, n, H in ((q8, "q8", Hq), (k8, "k8", Hkv), (v8, "v8", Hkv)):
        _need(t, n, torch.uint8, 1, numel=attn_fp8_buffer_bytes(B, H, N, d))
    if out is not None:
        _need(out, "out", torch.bfloat16, shape=(B, Hq, N, d))
    if with_lse and lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq, N))
    o = torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device=q8.device) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty(B, Hq, N, device=q8.device, dtype=torch.float32)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = attn_fwd(q8, k8, v8, o, lse if with_lse else None, B, Hq, Hkv, N, N, d, sc, MASK_NONE, 0, None,
                  0.0, None, FP8_E4M3, stream)
    if st:
        raise AttnError(st, "attn_fwd(fp8)")
    return (o, lse) if with_lse else o


def fp8_unpack(buf, B, H, N, d, transposed=False):
    """Views of a packed fp8 buffer: (value codes uint8, scales float32)."""
    npad = (N + FP8_TILE - 1) // FP8_TILE * FP8_TILE
    n = B * H * npad * d
    codes = buf[:n].view(B, H, d, npad) if transposed else buf[:n].view(B, H, npad, d)
    scales = buf[2 * n:2 * n + B * H * (npad // FP8_TILE) * 4].view(torch.float32).view(B, H, npad // FP8_TILE)
    return codes, scales


def fp8_unpack_residual(buf, B, H, N, d):
    """View of the residual codes (uint8 [B, H, Np, d]) of a packed Q or K buffer."""
    npad = (N + FP8_TILE - 1) // FP8_TILE * FP8_TILE
    n = B * H * npad * d
    return buf[n:2 * n].view(B, H, npad, d)


def block_mask(B, Nq, Nk, mask, window=0, doc_ids=None, block_m=128, block_n=64, device="cuda",
               stream=None):
    """(kinds int8 [B, nQt, nKt], counts int32 [B, nQt, 3], flags int) of the block classification."""
    nbytes = attn_block_mask_bytes(B, Nq, Nk, block_m, block_n)
    if nbytes == 0:
        raise AttnError(ERR_INVALID_ARG, "attn_block_mask_bytes")
    out = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    st = attn_block_mask_build(B, Nq, Nk, mask, window, doc_ids, block_m, block_n, out, stream)
    if st:
        raise AttnError(st, "attn_block_mask_build")
    nq, nk = -(-Nq // block_m), -(-Nk // block_n)
    kb = (B * nq * nk + 15) // 16 * 16
    kinds = out[:B * nq * nk].view(torch.int8).view(B, nq, nk)
    counts = out[kb:kb + B * nq * 3 * 4].view(torch.int32).view(B, nq, 3)
    flags = out[kb + B * nq * 12:kb + B * nq * 12 + 4].view(torch.int32)
    return kinds, counts, flags


def fwd_tile_kinds(B, Nq, Nk, mask, window=0, doc_ids=None, device="cuda", stream=None):
    """int8 [B, ceil(Nq/32), ceil(Nk/64)]: the forward's own tile schedule
    (0 empty, 1 partial, 2 full) for blocks of 32 query rows by 64-key tiles."""
    n = attn_fwd_tile_kinds_bytes(B, Nq, Nk)
    if n == 0:
        raise AttnError(ERR_INVALID_ARG, "attn_fwd_tile_kinds_bytes")
    if doc_ids is not None:
        _need(doc_ids, "doc_ids", torch.int32, 2)
        if tuple(doc_ids.shape) != (B, Nk):
            raise ValueError(f"doc_ids must be [B, Nk] = [{B}, {Nk}]")
    out = torch.empty(n, dtype=torch.int8, device=device)
    st = attn_fwd_tile_kinds(B, Nq, Nk, mask, window, doc_ids, out, stream)
    if st:
        raise AttnError(st, "attn_fwd_tile_kinds")
    return out.view(B, -(-Nq // 32), -(-Nk // 64))
