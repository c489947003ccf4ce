"""Thin ctypes binding of libfa.so (declared in include/fa.h).

Only argument marshalling happens here: shapes and dtypes are read off the torch
tensors, device pointers and the current HIP stream are passed to the C ABI,
and status codes become exceptions.  Every step of the attention itself runs
in the library's kernels.  Missing library -> RuntimeError; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_LIBRARY selects another build of the same library, such as the build of
# the C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.
LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa.so")

FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once.  torch is imported first so that the library binds to
    the HIP runtime torch already loaded (one runtime per process)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads libamdhip64 before libfa.so resolves it)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m tiled_online_softmax_04_amd.build`")
    lib = ctypes.CDLL(path)
    lib.fa_fwd.restype = _c_int
    lib.fa_fwd.argtypes = [_c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                           ctypes.c_float, _c_int, _c_void_p, _c_void_p]
    lib.fa_fwd_partial.restype = _c_int
    lib.fa_fwd_partial.argtypes = [_c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   ctypes.c_float, _c_int, _c_void_p, _c_int, _c_int, _c_void_p]
    lib.fa_fwd_fp8.restype = _c_int
    lib.fa_fwd_fp8.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                               _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                               ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                               _c_int, _c_void_p, _c_void_p]
    lib.fa_paged_prefill.restype = _c_int
    lib.fa_paged_prefill.argtypes = [_c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                     _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_int, _c_int, _c_int, ctypes.c_float, _c_int, _c_void_p,
                                     _c_void_p]
    lib.fa_merge.restype = _c_int
    lib.fa_merge.argtypes = [_c_int, _c_void_p, _c_void_p, _c_int, ctypes.c_longlong, _c_int,
                             _c_void_p, _c_void_p, _c_void_p]
    lib.fa_paged_decode_workspace_size.restype = ctypes.c_size_t
    lib.fa_paged_decode_workspace_size.argtypes = [_c_int] * 6
    lib.fa_paged_decode.restype = _c_int
    lib.fa_paged_decode.argtypes = [_c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    ctypes.c_float, _c_void_p, _c_void_p, ctypes.c_size_t,
                                    _c_void_p]
    lib.fa_paged_decode_noalloc.restype = _c_int
    lib.fa_paged_decode_noalloc.argtypes = [_c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                            _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_int, _c_int, ctypes.c_float, _c_void_p,
                                            _c_void_p]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [_c_int]
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    _lib = lib
    return lib


class FAError(RuntimeError):
    pass


def check(status: int) -> None:
    if status == FA_OK:
        return
    lib = load_library()
    msg = f"{lib.fa_status_string(status).decode()}: {lib.fa_last_error().decode()}"
    if status in (FA_ERR_INVALID, FA_ERR_WORKSPACE):
        raise ValueError(msg)
    if status == FA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise FAError(msg)


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if t.dtype not in codes:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, name, ndim, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def fwd(q, k, v, scale: float | None = None, causal: bool = False, seq_lens=None, out=None,
        stream=None):
    """O = softmax(scale * Q K^T [masked]) V.  q [B, Hq, n, d], k [B, Hkv, m, d],
    v [B, Hkv, m, dv] on one device, one dtype; seq_lens: None or int32 [B]
    left-padded lengths.  scale defaults to 1/sqrt(d)."""
    import torch
    lib = load_library()
    _require(q, "q", 4, q.device)
    _require(k, "k", 4, q.device)
    _require(v, "v", 4, q.device)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, Hq, n, d = q.shape
    Bk, Hkv, m, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape[:3]) != (B, Hkv, m):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    dv = v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if seq_lens is not None:
        _require(seq_lens, "seq_lens", 1, q.device)
        if seq_lens.dtype != torch.int32 or seq_lens.shape[0] != B:
            raise ValueError("seq_lens must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, n, dv), dtype=q.dtype, device=q.device)
    else:
        _require(out, "out", 4, q.device)
        if out.dtype != q.dtype or tuple(out.shape) != (B, Hq, n, dv):
            raise ValueError("out has the wrong shape or dtype")
    check(lib.fa_fwd(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, n, m, d, dv,
                     float(scale), 1 if causal else 0, _ptr(seq_lens), _stream(stream)))
    return out


def _check_qkv(q, k, v, seq_lens):
    import torch
    _require(q, "q", 4, q.device)
    _require(k, "k", 4, q.device)
    _require(v, "v", 4, q.device)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, Hq, n, d = q.shape
    Bk, Hkv, m, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape[:3]) != (B, Hkv, m):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if seq_lens is not None:
        _require(seq_lens, "seq_lens", 1, q.device)
        if seq_lens.dtype != torch.int32 or seq_lens.shape[0] != B:
            raise ValueError("seq_lens must be int32 [B]")
    return B, Hq, Hkv, n, m, d, v.shape[3]


def fwd_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float,
            scale: float | None = None, causal: bool = False, seq_lens=None,
            out_dtype=None, out=None, stream=None):
    """Attention on FP8 inputs: q, k, v hold E4M3 codes (torch.uint8 or
    torch.float8_e4m3fn, shapes as ``fwd``); the real inputs are descale *
    E4M3(code) per tensor.  O is out_dtype (default bfloat16).  scale defaults
    to 1/sqrt(d)."""
    import torch
    lib = load_library()
    fp8 = getattr(torch, "float8_e4m3fn", None)
    for name, t_ in (("q", q), ("k", k), ("v", v)):
        if t_.dtype not in (torch.uint8, fp8):
            raise ValueError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn), "
                             f"got {t_.dtype}")
    qb, kb, vb = (t_ if t_.dtype == torch.uint8 else t_.view(torch.uint8) for t_ in (q, k, v))
    B, Hq, Hkv, n, m, d, dv = _check_qkv(qb, kb, vb, seq_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, n, dv), dtype=out_dtype or torch.bfloat16, device=q.device)
    else:
        _require(out, "out", 4, q.device)
        if tuple(out.shape) != (B, Hq, n, dv) or (out_dtype is not None and out.dtype != out_dtype):
            raise ValueError("out has the wrong shape or dtype")
    check(lib.fa_fwd_fp8(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(out), _dtype_code(out), B, Hq, Hkv,
                         n, m, d, dv, float(scale), float(q_descale), float(k_descale),
                         float(v_descale), 1 if causal else 0, _ptr(seq_lens), _stream(stream)))
    return out


def fwd_partial(q, k, v, key_begin: int, key_end: int, scale: float | None = None,
                causal: bool = False, seq_lens=None, out=None, lse=None, stream=None):
    """Attention over the keys in [key_begin, key_end) only.  Returns
    (o float32 [B, Hq, n, dv], lse float32 [B, Hq, n]): o is normalised over
    the row's allowed keys in the range, lse = ln(sum exp(scale * q.k)) over
    them (-inf, with o = 0, where there are none).  Pieces of disjoint ranges
    combine with ``merge``."""
    import torch
    lib = load_library()
    B, Hq, Hkv, n, m, d, dv = _check_qkv(q, k, v, seq_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, n, dv), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
    _require(out, "out", 4, q.device)
    _require(lse, "lse", 3, q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, n, dv):
        raise ValueError("out must be float32 [B, Hq, n, dv]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, n):
        raise ValueError("lse must be float32 [B, Hq, n]")
    check(lib.fa_fwd_partial(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                             B, Hq, Hkv, n, m, d, dv, float(scale), 1 if causal else 0,
                             _ptr(seq_lens), int(key_begin), int(key_end), _stream(stream)))
    return out, lse


def merge(o_parts, lse_parts, out_dtype=None, out=None, lse_out=None, want_lse: bool = False,
          stream=None):
    """Combine pieces over disjoint key ranges: o_parts float32 [P, ..., dv]
    and lse_parts float32 [P, ...] (stacked ``fwd_partial`` results) give
    O [..., dv] in out_dtype (default bfloat16) and, with want_lse or lse_out,
    the merged lse [...]."""
    import torch
    lib = load_library()
    dev = o_parts.device
    if not o_parts.is_cuda or not lse_parts.is_cuda:
        raise ValueError("o_parts and lse_parts must be device tensors")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts and lse_parts must be float32")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    if tuple(o_parts.shape[:-1]) != tuple(lse_parts.shape) or o_parts.dim() < 2:
        raise ValueError("o_parts must be lse_parts' shape plus a trailing dv")
    P, dv = o_parts.shape[0], o_parts.shape[-1]
    row_shape = tuple(o_parts.shape[1:-1])
    rows = int(math.prod(row_shape))
    if out is None:
        out = torch.empty((*row_shape, dv), dtype=out_dtype or torch.bfloat16, device=dev)
    if (want_lse or lse_out is not None) and lse_out is None:
        lse_out = torch.empty(row_shape, dtype=torch.float32, device=dev)
    if tuple(out.shape) != (*row_shape, dv) or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out has the wrong shape or layout")
    if lse_out is not None and (tuple(lse_out.shape) != row_shape or lse_out.dtype != torch.float32
                                or not lse_out.is_contiguous() or not lse_out.is_cuda):
        raise ValueError("lse_out must be float32 with the rows' shape")
    check(lib.fa_merge(_dtype_code(out), _ptr(o_parts), _ptr(lse_parts), P, rows, dv, _ptr(out),
                       _ptr(lse_out), _stream(stream)))
    return (out, lse_out) if lse_out is not None else out


def paged_prefill(q, k_cache, v_cache, block_table, seq_lens, block_size: int | None = None,
                  scale: float | None = None, causal: bool = True, out=None, stream=None):
    """A chunk of n query tokens per sequence over a paged cache that holds the
    chunk's keys too: q [S, Hq, n, d] (row i is token seq_lens[s] - n + i);
    k_cache [NB, bs, Hkv, d]; v_cache [NB, bs, Hkv, dv]; block_table int32
    [S, max_blocks]; seq_lens int32 [S] total lengths.  Returns [S, Hq, n, dv]."""
    import torch
    lib = load_library()
    dev = q.device
    _require(q, "q", 4, dev)
    _require(k_cache, "k_cache", 4, dev)
    _require(v_cache, "v_cache", 4, dev)
    _require(block_table, "block_table", 2, dev)
    _require(seq_lens, "seq_lens", 1, dev)
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_cache, v_cache must share a dtype")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    S, Hq, n, d = q.shape
    NB, bs, Hkv, dk = k_cache.shape
    dv = v_cache.shape[3]
    if block_size is None:
        block_size = bs
    if bs != block_size or dk != d or tuple(v_cache.shape[:3]) != (NB, bs, Hkv):
        raise ValueError("cache shapes do not match q / block_size")
    if block_table.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("block_table / seq_lens batch mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((S, Hq, n, dv), dtype=q.dtype, device=dev)
    else:
        _require(out, "out", 4, dev)
        if out.dtype != q.dtype or tuple(out.shape) != (S, Hq, n, dv):
            raise ValueError(f"out must be {q.dtype} {(S, Hq, n, dv)}, got {out.dtype} "
                             f"{tuple(out.shape)}")
    check(lib.fa_paged_prefill(_dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_table), _ptr(seq_lens), block_size, S, Hq, Hkv, n, d,
                               dv, NB, block_table.shape[1], float(scale), 1 if causal else 0,
                               _ptr(out), _stream(stream)))
    return out


def paged_decode_workspace_size(num_seqs, heads_q, heads_kv, dv, max_blocks_per_seq,
                                block_size) -> int:
    return int(load_library().fa_paged_decode_workspace_size(num_seqs, heads_q, heads_kv, dv,
                                                            max_blocks_per_seq, block_size))


def _decode_shapes(q, k_cache, v_cache, block_table, seq_lens, block_size, out):
    """Checks shared by the two decode entry points; returns the sizes and the
    output tensor (allocated when `out` is None)."""
    import torch
    dev = q.device
    _require(q, "q", 3, dev)
    _require(k_cache, "k_cache", 4, dev)
    _require(v_cache, "v_cache", 4, dev)
    _require(block_table, "block_table", 2, dev)
    _require(seq_lens, "seq_lens", 1, dev)
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_cache, v_cache must share a dtype")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    S, Hq, d = q.shape
    NB, bs, Hkv, dk = k_cache.shape
    dv = v_cache.shape[3]
    if block_size is None:
        block_size = bs
    if bs != block_size or dk != d or tuple(v_cache.shape[:3]) != (NB, bs, Hkv):
        raise ValueError("cache shapes do not match q / block_size")
    if block_table.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("block_table / seq_lens batch mismatch")
    if out is None:
        out = torch.empty((S, Hq, dv), dtype=q.dtype, device=dev)
    else:
        _require(out, "out", 3, dev)
        if out.dtype != q.dtype or tuple(out.shape) != (S, Hq, dv):
            raise ValueError(f"out must be {q.dtype} {(S, Hq, dv)}, got {out.dtype} "
                             f"{tuple(out.shape)}")
    return S, Hq, Hkv, d, dv, NB, block_size, block_table.shape[1], out


def paged_decode(q, k_cache, v_cache, block_table, seq_lens, block_size: int | None = None,
                 scale: float | None = None, out=None, workspace=None, stream=None):
    """One query token per sequence over a paged cache.  q [S, Hq, d];
    k_cache [NB, bs, Hkv, d]; v_cache [NB, bs, Hkv, dv]; block_table int32
    [S, max_blocks]; seq_lens int32 [S].  scale defaults to 1/sqrt(d)."""
    import torch
    lib = load_library()
    S, Hq, Hkv, d, dv, NB, block_size, maxb, out = _decode_shapes(
        q, k_cache, v_cache, block_table, seq_lens, block_size, out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = paged_decode_workspace_size(S, Hq, Hkv, dv, maxb, block_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        if not workspace.is_cuda or workspace.device != q.device:
            raise ValueError(f"workspace must be a device tensor on {q.device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
    check(lib.fa_paged_decode(_dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_table), _ptr(seq_lens), block_size, S, Hq, Hkv, d, dv,
                              NB, maxb, float(scale), _ptr(out), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


# Bytes of the static scratch behind paged_decode_noalloc (FA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 32 << 20


def paged_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, block_size: int | None = None,
                         scale: float | None = None, out=None, stream=None):
    """paged_decode through fa_paged_decode_noalloc: the split states live in
    the library's static per-GPU scratch, so the call allocates nothing when
    `out` is given.  Calls that overlap on one GPU race (one scratch per GPU)."""
    lib = load_library()
    S, Hq, Hkv, d, dv, NB, block_size, maxb, out = _decode_shapes(
        q, k_cache, v_cache, block_table, seq_lens, block_size, out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    check(lib.fa_paged_decode_noalloc(_dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(block_table), _ptr(seq_lens), block_size, S, Hq, Hkv,
                                      d, dv, NB, maxb, float(scale), _ptr(out), _stream(stream)))
    return out
