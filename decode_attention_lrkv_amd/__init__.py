"""Decode attention over a low-rank KV cache on AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C-ABI library ``liblrkv.so`` (declared in
``include/lrkv.h``).  The functions here only marshal arguments: shapes,
dtypes and pointers of torch tensors, and the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; if the library
has not been built, every call raises.

Layouts (see include/lrkv.h): keys use the row layout [B, Hkv, cap, r_K];
values use the octet layout [B, Hkv, cap/8, r_V, 8], in which each column's 8
consecutive tokens are contiguous.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "LrkvError", "library", "compress", "compress_kv", "decode_attn", "decode_workspace_bytes",
    "decode_step", "decode_step_workspace_bytes", "decode_step_partial", "decode_step_merge",
    "compress_hybrid", "compress_hybrid_workspace_bytes", "decode_attn_hybrid",
    "HybridCache", "value_cache_shape", "LIB_PATH", "decode_attn_partial", "decode_attn_merge",
    "decode_attn_latent", "oja_update", "oja_workspace_bytes", "decode_step_noalloc",
    "decode_step_noalloc_max_bytes", "decode_attn_seqlens", "decode_step_seqlens",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblrkv.so")

_F32, _BF16 = 0, 1
_KEYS, _VALUES = 0, 1


class LrkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[lrkv status {status}] {message}")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rank_k", ctypes.c_int32), ("rank_v", ctypes.c_int32),
                ("capacity", ctypes.c_int64)]


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIG = {
    "lrkv_compress": (ctypes.c_int, [_P, _P, _P, ctypes.c_int, _I32, _I32, _I32, _I32, _I64, _I64, _I64,
                                     ctypes.c_int, _P]),
    "lrkv_compress_kv": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(_Dims), _I64, _I64, ctypes.c_int, _P]),
    "lrkv_oja_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I64]),
    "lrkv_oja_update": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _I64, _F, _P, ctypes.c_size_t, _P]),
    "lrkv_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Dims), _I64, _I64]),
    "lrkv_decode_attn": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Dims), _I64, _F,
                                        ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "lrkv_decode_attn_latent": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.POINTER(_Dims), _I64, _F, ctypes.c_int,
                                               _P, ctypes.c_size_t, _P]),
    "lrkv_decode_step_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Dims), _I64]),
    "lrkv_decode_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Dims), _I64, _F,
                                        ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "lrkv_decode_attn_seqlens": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Dims), _P, _I64, _F,
                                                ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "lrkv_decode_step_seqlens": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Dims), _P,
                                                _I64, _F, ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "lrkv_decode_step_noalloc_max_bytes": (ctypes.c_size_t, []),
    "lrkv_decode_step_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Dims), _I64,
                                                _F, ctypes.c_int, _P]),
    "lrkv_decode_step_partial": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Dims), _I64, _F,
                                                ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "lrkv_decode_step_merge": (ctypes.c_int, [_P, _P, ctypes.POINTER(_Dims), _I64, ctypes.c_int, _P,
                                              ctypes.c_size_t, _P]),
    "lrkv_compress_hybrid_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Dims), _I64]),
    "lrkv_compress_hybrid": (ctypes.c_int, [_P, _P, _P, _P, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            ctypes.POINTER(_Dims), _I64, _I64, _I64, ctypes.c_int, _P,
                                            ctypes.c_size_t, _P]),
    "lrkv_decode_attn_hybrid": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _P, _P,
                                               ctypes.POINTER(_Dims), _F, ctypes.c_int, _P,
                                               ctypes.c_size_t, _P]),
    "lrkv_decode_attn_partial": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.POINTER(_Dims), _I64, _F,
                                                ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "lrkv_decode_attn_merge": (ctypes.c_int, [_P, _P, ctypes.POINTER(_Dims), _I64, ctypes.c_int, _P,
                                              ctypes.c_size_t, _P]),
    "lrkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lrkv_last_error": (ctypes.c_char_p, []),
}


def library() -> ctypes.CDLL:
    """Load liblrkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LrkvError(-1, f"{LIB_PATH} is missing: build it with "
                                "`python -c 'import __graft_entry__; __graft_entry__.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        lib = library()
        raise LrkvError(status, f"{lib.lrkv_status_string(status).decode()}: "
                                f"{lib.lrkv_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise LrkvError(1, f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise LrkvError(1, "tensors must live on the GPU")
    if not t.is_contiguous():
        raise LrkvError(1, "tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def value_cache_shape(batch: int, n_kv_heads: int, capacity: int, rank: int):
    """Shape of a value cache (octet layout) holding `capacity` tokens."""
    return (batch, n_kv_heads, capacity // 8, rank, 8)


def _dims(q_shape, n_kv_heads, head_dim, rank_k, rank_v, capacity) -> _Dims:
    return _Dims(q_shape[0], q_shape[1], n_kv_heads, head_dim, rank_k, rank_v, capacity)


def compress(x: torch.Tensor, basis: torch.Tensor, coeff: torch.Tensor, pos: int, values: bool) -> None:
    """Write coeff rows [pos, pos + T) = x @ basis (per batch and kv head).

    x [B, T, Hkv, d]; basis [Hkv, d, r]; coeff: key cache [B, Hkv, cap, r]
    (values=False) or value cache [B, Hkv, cap/8, r, 8] (values=True).
    """
    B, T, H, d = x.shape
    r = basis.shape[2]
    cap = coeff.shape[2] * (8 if values else 1)
    _check(library().lrkv_compress(_ptr(x), _ptr(basis), _ptr(coeff), _VALUES if values else _KEYS,
                                   B, H, d, r, T, pos, cap, _dtype_code(x), _stream(x.device)))


def compress_kv(xk, xv, basis_k, basis_v, coeff_k, coeff_v, pos: int) -> None:
    """Both caches at once: coeff_k rows (row layout) and coeff_v rows (octet layout) [pos, pos + T)."""
    B, T, H, d = xk.shape
    dims = _Dims(B, H, H, d, basis_k.shape[2], basis_v.shape[2], coeff_k.shape[2])
    _check(library().lrkv_compress_kv(_ptr(xk), _ptr(xv), _ptr(basis_k), _ptr(basis_v), _ptr(coeff_k),
                                      _ptr(coeff_v), ctypes.byref(dims), T, pos, _dtype_code(xk),
                                      _stream(xk.device)))


def oja_workspace_bytes(batch: int, n_kv_heads: int, head_dim: int, rank: int, n_tokens: int) -> int:
    return int(library().lrkv_oja_workspace_bytes(batch, n_kv_heads, head_dim, rank, n_tokens))


def oja_update(x: torch.Tensor, basis: torch.Tensor, eta: float, basis_bf16: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One Oja subspace step of every kv head's basis from a chunk of tokens.

    x [B, T, Hkv, d] bfloat16; basis [Hkv, d, r] float32, updated in place:
    B <- B + eta (X^T Y - B Y^T Y), Y = X B, over the chunk's tokens of all
    batch rows.  Returns basis_bf16 [Hkv, d, r] (the updated basis rounded to
    bfloat16; allocated when not given).
    """
    if x.dtype != torch.bfloat16 or basis.dtype != torch.float32:
        raise LrkvError(1, "oja_update takes bfloat16 tokens and a float32 basis")
    B, T, H, d = x.shape
    r = basis.shape[2]
    lib = library()
    ws = _workspace(int(lib.lrkv_oja_workspace_bytes(B, H, d, r, T)), x.device, workspace)
    if basis_bf16 is None:
        basis_bf16 = torch.empty(basis.shape, dtype=torch.bfloat16, device=basis.device)
    _check(lib.lrkv_oja_update(_ptr(x), _ptr(basis), _ptr(basis_bf16), B, H, d, r, T, eta, _ptr(ws), ws.numel(),
                               _stream(x.device)))
    return basis_bf16


def decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, capacity,
                           n_ctx, side_cap=0) -> int:
    dims = _Dims(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, capacity)
    return int(library().lrkv_decode_workspace_bytes(ctypes.byref(dims), n_ctx, side_cap))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    """The caller's workspace, or a new one (zeroed: the hybrid decode's
    arrival counters at its start must be zero before a first call)."""
    if workspace is not None:
        return workspace
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def decode_attn(q, basis_k, coeff_k, basis_v, coeff_v, n_ctx: int, out=None, lse=None,
                scale: float = 0.0, workspace: Optional[torch.Tensor] = None, with_lse: bool = True):
    """Decode attention over tokens [0, n_ctx) of a low-rank cache.

    q [B, Hq, d]; basis_k [Hkv, d, r_K]; coeff_k [B, Hkv, cap, r_K];
    basis_v [Hkv, d, r_V]; coeff_v [B, Hkv, cap/8, r_V, 8].
    Returns (out [B, Hq, d], lse [B, Hq] float32 or None).
    """
    B, Hq, d = q.shape
    H, _, rk = basis_k.shape
    rv = basis_v.shape[2]
    cap = coeff_k.shape[2]
    dims = _Dims(B, Hq, H, d, rk, rv, cap)
    lib = library()
    need = int(lib.lrkv_decode_workspace_bytes(ctypes.byref(dims), n_ctx, 0))
    ws = _workspace(need, q.device, workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib.lrkv_decode_attn(_ptr(q), _ptr(basis_k), _ptr(coeff_k), _ptr(basis_v), _ptr(coeff_v),
                                _ptr(out), _ptr(lse), ctypes.byref(dims), n_ctx, scale, _dtype_code(q),
                                _ptr(ws), ws.numel(), _stream(q.device)))
    return out, lse


def decode_attn_latent(q_lat, coeff_k, coeff_v, n_ctx: int, head_dim: int, out=None, lse=None, scale: float = 0.0,
                       workspace: Optional[torch.Tensor] = None, with_lse: bool = True):
    """Decode attention on latent queries, for projections that absorb the bases.

    q_lat [B, Hq, r_K]; coeff_k [B, Hkv, cap, r_K]; coeff_v [B, Hkv, cap/8, r_V, 8];
    head_dim is the model's head dimension (default scale 1/sqrt(head_dim)).
    Returns (out_lat [B, Hq, r_V], lse [B, Hq] float32 or None).
    """
    B, Hq, rk = q_lat.shape
    H, cap = coeff_k.shape[1], coeff_k.shape[2]
    rv = coeff_v.shape[3]
    dims = _Dims(B, Hq, H, head_dim, rk, rv, cap)
    lib = library()
    need = int(lib.lrkv_decode_workspace_bytes(ctypes.byref(dims), n_ctx, 0))
    ws = _workspace(need, q_lat.device, workspace)
    if out is None:
        out = torch.empty((B, Hq, rv), dtype=q_lat.dtype, device=q_lat.device)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q_lat.device)
    _check(lib.lrkv_decode_attn_latent(_ptr(q_lat), _ptr(coeff_k), _ptr(coeff_v), _ptr(out), _ptr(lse),
                                       ctypes.byref(dims), n_ctx, scale, _dtype_code(q_lat), _ptr(ws), ws.numel(),
                                       _stream(q_lat.device)))
    return out, lse


def decode_step_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, capacity,
                                n_ctx: int) -> int:
    dims = _Dims(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, capacity)
    return int(library().lrkv_decode_step_workspace_bytes(ctypes.byref(dims), n_ctx))


def decode_step(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, n_ctx: int, out=None, lse=None,
                scale: float = 0.0, workspace: Optional[torch.Tensor] = None, with_lse: bool = True,
                enc_k: Optional[torch.Tensor] = None):
    """Append the step's token at row n_ctx - 1 of both caches, then attend [0, n_ctx).

    k_new, v_new [B, Hkv, d] (or [B, 1, Hkv, d]); basis_k, basis_v decode (fold
    and lift); enc_k [Hkv, d, r_K] encodes the new key when the key transform
    is not an orthonormal basis (None: basis_k encodes; basis_v always encodes
    the value).  Other arguments as decode_attn.  Returns (out [B, Hq, d],
    lse [B, Hq] float32 or None).
    """
    B, Hq, d = q.shape
    H, _, rk = basis_k.shape
    rv = basis_v.shape[2]
    cap = coeff_k.shape[2]
    dims = _Dims(B, Hq, H, d, rk, rv, cap)
    lib = library()
    need = int(lib.lrkv_decode_step_workspace_bytes(ctypes.byref(dims), n_ctx))
    ws = _workspace(need, q.device, workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib.lrkv_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(basis_k), _ptr(coeff_k), _ptr(basis_v),
                                _ptr(coeff_v), _ptr(enc_k), _ptr(out), _ptr(lse), ctypes.byref(dims), n_ctx, scale,
                                _dtype_code(q), _ptr(ws), ws.numel(), _stream(q.device)))
    return out, lse


def _seq_lens(seq_lens: torch.Tensor, batch: int):
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != batch:
        raise LrkvError(1, f"seq_lens must be an int32 tensor of {batch} lengths")
    return _ptr(seq_lens)


def decode_attn_seqlens(q, basis_k, coeff_k, basis_v, coeff_v, seq_lens: torch.Tensor, max_seq_len: int,
                        out=None, lse=None, scale: float = 0.0, workspace: Optional[torch.Tensor] = None,
                        with_lse: bool = True):
    """decode_attn with per-sequence lengths on the device: sequence b attends
    rows [0, seq_lens[b]).  The split plan is made for max_seq_len (host), so
    a captured graph stays valid while the lengths advance."""
    B, Hq, d = q.shape
    H, _, rk = basis_k.shape
    dims = _Dims(B, Hq, H, d, rk, basis_v.shape[2], coeff_k.shape[2])
    lib = library()
    ws = _workspace(int(lib.lrkv_decode_workspace_bytes(ctypes.byref(dims), max_seq_len, 0)), q.device, workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib.lrkv_decode_attn_seqlens(_ptr(q), _ptr(basis_k), _ptr(coeff_k), _ptr(basis_v), _ptr(coeff_v),
                                        _ptr(out), _ptr(lse), ctypes.byref(dims), _seq_lens(seq_lens, B),
                                        max_seq_len, scale, _dtype_code(q), _ptr(ws), ws.numel(),
                                        _stream(q.device)))
    return out, lse


def decode_step_seqlens(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, seq_lens: torch.Tensor,
                        max_seq_len: int, out=None, lse=None, scale: float = 0.0,
                        workspace: Optional[torch.Tensor] = None, with_lse: bool = True,
                        enc_k: Optional[torch.Tensor] = None):
    """decode_step with per-sequence lengths on the device: sequence b appends
    its token at row seq_lens[b] - 1 and attends rows [0, seq_lens[b]).  The
    lengths are read, not advanced."""
    B, Hq, d = q.shape
    H, _, rk = basis_k.shape
    dims = _Dims(B, Hq, H, d, rk, basis_v.shape[2], coeff_k.shape[2])
    lib = library()
    ws = _workspace(int(lib.lrkv_decode_step_workspace_bytes(ctypes.byref(dims), max_seq_len)), q.device, workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib.lrkv_decode_step_seqlens(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(basis_k), _ptr(coeff_k),
                                        _ptr(basis_v), _ptr(coeff_v), _ptr(enc_k), _ptr(out), _ptr(lse),
                                        ctypes.byref(dims), _seq_lens(seq_lens, B), max_seq_len, scale,
                                        _dtype_code(q), _ptr(ws), ws.numel(), _stream(q.device)))
    return out, lse


def decode_step_noalloc_max_bytes() -> int:
    """Size of the library's fixed decode-step workspace (per GPU)."""
    return int(library().lrkv_decode_step_noalloc_max_bytes())


def decode_step_noalloc(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, n_ctx: int, out, lse=None,
                        scale: float = 0.0, enc_k: Optional[torch.Tensor] = None):
    """decode_step with the library's fixed workspace instead of a caller's.

    Allocates nothing: out [B, Hq, d] (and lse [B, Hq] float32, if wanted)
    must be given.  Calls on one GPU share the fixed workspace; order them on
    one stream.
    """
    B, Hq, d = q.shape
    H, _, rk = basis_k.shape
    dims = _Dims(B, Hq, H, d, rk, basis_v.shape[2], coeff_k.shape[2])
    _check(library().lrkv_decode_step_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(basis_k), _ptr(coeff_k),
                                              _ptr(basis_v), _ptr(coeff_v), _ptr(enc_k), _ptr(out), _ptr(lse),
                                              ctypes.byref(dims), n_ctx, scale, _dtype_code(q), _stream(q.device)))
    return out, lse


def compress_hybrid_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, capacity,
                                    n_tokens) -> int:
    dims = _Dims(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, capacity)
    return int(library().lrkv_compress_hybrid_workspace_bytes(ctypes.byref(dims), n_tokens))


class HybridCache:
    """Device buffers of an OjaKV-style hybrid cache (low-rank rows + full-rank side list)."""

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, capacity, side_cap,
                 device, dtype=torch.bfloat16):
        self.dims = (batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, capacity)
        self.side_cap = side_cap
        z = dict(device=device)
        self.coeff_k = torch.empty((batch, n_kv_heads, capacity, rank_k), dtype=dtype, **z)
        self.coeff_v = torch.empty(value_cache_shape(batch, n_kv_heads, capacity, rank_v), dtype=dtype, **z)
        self.k_side = torch.empty((batch, n_kv_heads, side_cap, head_dim), dtype=dtype, **z)
        self.v_side = torch.empty(value_cache_shape(batch, n_kv_heads, side_cap, head_dim), dtype=dtype, **z)
        self.side_idx = torch.empty((batch, n_kv_heads, side_cap), dtype=torch.int32, **z)
        self.n_lr = torch.zeros((batch, n_kv_heads), dtype=torch.int32, **z)
        self.n_side = torch.zeros((batch, n_kv_heads), dtype=torch.int32, **z)
        self.overflow = torch.zeros(4, dtype=torch.int32, **z)


def compress_hybrid(cache: HybridCache, k, v, basis_k, basis_v, tau: float, pos: int,
                    flags: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Append a chunk of tokens to a hybrid cache (selection + ordered compaction)."""
    B, T, H, d = k.shape
    dims = _Dims(*cache.dims)
    lib = library()
    need = int(lib.lrkv_compress_hybrid_workspace_bytes(ctypes.byref(dims), T))
    ws = _workspace(need, k.device, workspace)
    _check(lib.lrkv_compress_hybrid(_ptr(k), _ptr(v), _ptr(basis_k), _ptr(basis_v), tau,
                                    _ptr(cache.coeff_k), _ptr(cache.coeff_v), _ptr(cache.n_lr),
                                    _ptr(cache.k_side), _ptr(cache.v_side), _ptr(cache.side_idx),
                                    _ptr(cache.n_side), _ptr(flags), _ptr(cache.overflow),
                                    ctypes.byref(dims), T, pos, cache.side_cap, _dtype_code(k),
                                    _ptr(ws), ws.numel(), _stream(k.device)))
    return flags


def decode_attn_hybrid(q, basis_k, basis_v, cache: HybridCache, out=None, lse=None, scale: float = 0.0,
                       workspace: Optional[torch.Tensor] = None, with_lse: bool = True):
    """One softmax over the low-rank tokens and the side-list tokens of a hybrid cache."""
    B, Hq, d = q.shape
    dims = _Dims(*cache.dims)
    lib = library()
    need = int(lib.lrkv_decode_workspace_bytes(ctypes.byref(dims), 0, cache.side_cap))
    ws = _workspace(need, q.device, workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib.lrkv_decode_attn_hybrid(_ptr(q), _ptr(basis_k), _ptr(cache.coeff_k), _ptr(basis_v),
                                       _ptr(cache.coeff_v), _ptr(cache.n_lr), _ptr(cache.k_side),
                                       _ptr(cache.v_side), _ptr(cache.n_side), cache.side_cap,
                                       _ptr(out), _ptr(lse), ctypes.byref(dims), scale, _dtype_code(q),
                                       _ptr(ws), ws.numel(), _stream(q.device)))
    return out, lse


def decode_attn_partial(q, basis_k, coeff_k, basis_v, coeff_v, n_ctx: int, workspace: torch.Tensor,
                        scale: float = 0.0):
    """First phase of decode_attn: per-workgroup lifted partial results into `workspace`."""
    B, Hq, d = q.shape
    H, _, rk = basis_k.shape
    dims = _Dims(B, Hq, H, d, rk, basis_v.shape[2], coeff_k.shape[2])
    _check(library().lrkv_decode_attn_partial(_ptr(q), _ptr(basis_k), _ptr(coeff_k), _ptr(basis_v),
                                              _ptr(coeff_v), ctypes.byref(dims), n_ctx, scale, _dtype_code(q),
                                              _ptr(workspace), workspace.numel(), _stream(q.device)))


def decode_attn_merge(out, lse, n_ctx: int, workspace: torch.Tensor, n_kv_heads: int, rank_k: int,
                      rank_v: int, capacity: int):
    """Second phase of decode_attn: log-sum-exp merge of the partials into out and lse."""
    B, Hq, d = out.shape
    dims = _Dims(B, Hq, n_kv_heads, d, rank_k, rank_v, capacity)
    _check(library().lrkv_decode_attn_merge(_ptr(out), _ptr(lse), ctypes.byref(dims), n_ctx, _dtype_code(out),
                                            _ptr(workspace), workspace.numel(), _stream(out.device)))


def decode_step_partial(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, n_ctx: int, workspace: torch.Tensor,
                        scale: float = 0.0, enc_k: Optional[torch.Tensor] = None):
    """First phase of decode_step: append the token, partial results into `workspace`."""
    B, Hq, d = q.shape
    H, _, rk = basis_k.shape
    dims = _Dims(B, Hq, H, d, rk, basis_v.shape[2], coeff_k.shape[2])
    _check(library().lrkv_decode_step_partial(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(basis_k), _ptr(coeff_k),
                                              _ptr(basis_v), _ptr(coeff_v), _ptr(enc_k), ctypes.byref(dims), n_ctx,
                                              scale, _dtype_code(q), _ptr(workspace), workspace.numel(),
                                              _stream(q.device)))


def decode_step_merge(out, lse, n_ctx: int, workspace: torch.Tensor, n_kv_heads: int, rank_k: int, rank_v: int,
                      capacity: int):
    """Second phase of decode_step: log-sum-exp merge into out and lse."""
    B, Hq, d = out.shape
    dims = _Dims(B, Hq, n_kv_heads, d, rank_k, rank_v, capacity)
    _check(library().lrkv_decode_step_merge(_ptr(out), _ptr(lse), ctypes.byref(dims), n_ctx, _dtype_code(out),
                                            _ptr(workspace), workspace.numel(), _stream(out.device)))
