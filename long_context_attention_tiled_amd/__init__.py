"""Exact long-context attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libattn.so`` (``include/attn.h``).
Each function has the name of the C entry point it calls and does argument
marshalling only: it checks tensor dtypes/devices/shapes, allocates outputs
with PyTorch when the caller does not pass them, and enqueues the HIP kernels
on the current PyTorch stream.  Every step of the computation runs in the
library's kernels; there is no fallback.

Layouts (all tensors contiguous, on the GPU):

* ``attn_prefill``: q ``[B][S][Hq][128]``, k/v ``[B][S][Hkv][128]`` (bf16), or
  fp32 with head_dim 64/128.
* paged cache: ``k_pool [n_blocks][64][128]``, ``v_pool [n_blocks][128][64]``,
  ``block_head [n_blocks]`` int32, ``block_table [B][Hkv][max_blocks]`` int32.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import (ATTN_CP_CONTIGUOUS, ATTN_CP_STRIPED, ATTN_CP_ZIGZAG, ATTN_DEV_BAD_BLOCK,
                   ATTN_DEV_BAD_TAG, ATTN_DEV_OK, ATTN_DTYPE_BF16, ATTN_DTYPE_F32, AttnError)

__all__ = [
    "attn_prefill", "attn_chunked_prefill", "attn_kv_append", "attn_decode",
    "attn_decode_workspace_bytes", "rope_apply", "rope_apply_qk", "seq_to_head_permute", "seq_to_head_permute_qkv", "head_to_seq_permute",
    "seq_to_head_permute_qkv_rope", "cp_shard_tokens", "cp_shard", "cp_unshard",
    "attn_key_limits", "attn_prefill_limited", "attn_merge", "CP_MODES", "attn_decode_fp8",
    "attn_kv_quantize_fp8", "attn_kv_append_fp8", "attn_quantize_fp8_blocks", "attn_prefill_fp8",
    "attn_quantize_fp8_v", "attn_prefill_fp8_pv", "attn_decode_noalloc",
    "attn_status_string", "measure_mfma_rate", "mfma_rate_flops", "measure_hbm_read",
    "measure_hbm_copy",
    "AttnError", "ATTN_DEV_OK", "ATTN_DEV_BAD_TAG", "ATTN_DEV_BAD_BLOCK", "load_library",
]

HEAD_DIM = 128
BLOCK_TOKENS = 64
# context-parallel split names -> enum attn_cp_mode
CP_MODES = {"contiguous": ATTN_CP_CONTIGUOUS, "striped": ATTN_CP_STRIPED, "zigzag": ATTN_CP_ZIGZAG}


def load_library():
    return _lib.load()


def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def attn_status_string(status: int) -> str:
    return _lib.load().attn_status_string(int(status)).decode()


def attn_prefill(q, k, v, causal=True, scale=None, o=None, lse=None, stream=None):
    """Exact attention over dense tensors; returns ``(o, lse)``.

    q ``[B][S][Hq][D]``, k/v ``[B][S][Hkv][D]``; ``lse`` is ``[B][Hq][S]`` fp32
    (natural log).  bf16 needs D = 128; fp32 accepts D in {64, 128}.
    """
    torch = _torch()
    _need(q, "q")
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    dt = q.dtype
    if dt == torch.bfloat16:
        code = ATTN_DTYPE_BF16
    elif dt == torch.float32:
        code = ATTN_DTYPE_F32
    else:
        raise TypeError("q must be bf16 or fp32")
    _need(k, "k", dt, (B, S, Hkv, D))
    _need(v, "v", dt, (B, S, Hkv, D))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", dt, q.shape)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (B, Hq, S))
    scale = float(D ** -0.5) if scale is None else float(scale)
    st = _lib.load().attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, S, Hq, Hkv, D,
                                  code, int(bool(causal)), scale, _stream(stream))
    _lib.check("attn_prefill", st)
    return o, lse


def attn_kv_append(k_new, v_new, k_pool, v_pool, block_head, block_table, start_pos,
                   kv_head_base=0, dev_status=None, stream=None):
    """Write ``k_new/v_new [B][T][Hkv][128]`` at positions ``start_pos[b] + t``."""
    torch = _torch()
    _need(k_new, "k_new", torch.bfloat16)
    B, T, Hkv, D = k_new.shape
    _need(v_new, "v_new", torch.bfloat16, k_new.shape)
    n_blocks = k_pool.shape[0]
    _need(k_pool, "k_pool", torch.bfloat16, (n_blocks, BLOCK_TOKENS, D))
    _need(v_pool, "v_pool", torch.bfloat16, (n_blocks, D, BLOCK_TOKENS))
    _need(block_head, "block_head", torch.int32, (n_blocks,))
    _need(block_table, "block_table", torch.int32)
    if block_table.shape[:2] != (B, Hkv):
        raise ValueError("block_table must be [B][Hkv][max_blocks]")
    _need(start_pos, "start_pos", torch.int32, (B,))
    st = _lib.load().attn_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), n_blocks,
                                    _ptr(block_head), _ptr(block_table), block_table.shape[2],
                                    _ptr(start_pos), T, B, Hkv, D, int(kv_head_base),
                                    _ptr(dev_status), _stream(stream))
    _lib.check("attn_kv_append", st)


def attn_chunked_prefill(q, k_new, v_new, k_pool, v_pool, block_head, block_table, ctx_before,
                         kv_head_base=0, scale=None, o=None, lse=None, dev_status=None,
                         stream=None):
    """Append a chunk's K/V to the paged cache, then attend; returns ``(o, lse)``.

    q ``[B][C][Hq][128]``, k_new/v_new ``[B][C][Hkv][128]``; chunk row i sits
    at position ``ctx_before[b] + i`` and sees every cached key up to it.
    """
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    B, C, Hq, D = q.shape
    Hkv = k_new.shape[2]
    _need(k_new, "k_new", torch.bfloat16, (B, C, Hkv, D))
    _need(v_new, "v_new", torch.bfloat16, (B, C, Hkv, D))
    n_blocks = k_pool.shape[0]
    _need(k_pool, "k_pool", torch.bfloat16, (n_blocks, BLOCK_TOKENS, D))
    _need(v_pool, "v_pool", torch.bfloat16, (n_blocks, D, BLOCK_TOKENS))
    _need(block_head, "block_head", torch.int32, (n_blocks,))
    _need(block_table, "block_table", torch.int32)
    if block_table.shape[:2] != (B, Hkv):
        raise ValueError("block_table must be [B][Hkv][max_blocks]")
    _need(ctx_before, "ctx_before", torch.int32, (B,))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, q.shape)
    if lse is None:
        lse = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (B, Hq, C))
    scale = float(D ** -0.5) if scale is None else float(scale)
    st = _lib.load().attn_chunked_prefill(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), n_blocks, _ptr(block_head),
        _ptr(block_table), block_table.shape[2], _ptr(ctx_before), C, _ptr(o), _ptr(lse), B, Hq,
        Hkv, D, int(kv_head_base), scale, _ptr(dev_status), _stream(stream))
    _lib.check("attn_chunked_prefill", st)
    return o, lse


def attn_decode_workspace_bytes(B, Hq, max_blocks, split_tokens=0, D=HEAD_DIM) -> int:
    return int(_lib.load().attn_decode_workspace_bytes(B, Hq, D, max_blocks, split_tokens))


def attn_decode(q, k_pool, v_pool, block_head, block_table, ctx_len, kv_head_base=0, scale=None,
                split_tokens=0, workspace=None, o=None, lse=None, dev_status=None, stream=None):
    """One query token per request over its paged context; returns ``(o, lse)``.

    q ``[B][Hq][128]``; ``ctx_len[b]`` counts the cached tokens including the
    new one.  ``workspace`` (uint8 tensor) is allocated if not given.
    """
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    B, Hq, D = q.shape
    n_blocks = k_pool.shape[0]
    _need(k_pool, "k_pool", torch.bfloat16, (n_blocks, BLOCK_TOKENS, D))
    _need(v_pool, "v_pool", torch.bfloat16, (n_blocks, D, BLOCK_TOKENS))
    _need(block_head, "block_head", torch.int32, (n_blocks,))
    _need(block_table, "block_table", torch.int32)
    Hkv, max_blocks = block_table.shape[1], block_table.shape[2]
    if block_table.shape[0] != B:
        raise ValueError("block_table must be [B][Hkv][max_blocks]")
    _need(ctx_len, "ctx_len", torch.int32, (B,))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, q.shape)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (B, Hq))
    need = attn_decode_workspace_bytes(B, Hq, max_blocks, split_tokens, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace")
    scale = float(D ** -0.5) if scale is None else float(scale)
    st = _lib.load().attn_decode(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), n_blocks, _ptr(block_head), _ptr(block_table),
        max_blocks, _ptr(ctx_len), _ptr(o), _ptr(lse), B, Hq, Hkv, D, int(kv_head_base), scale,
        int(split_tokens), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(dev_status), _stream(stream))
    _lib.check("attn_decode", st)
    return o, lse


def attn_decode_noalloc(q, k_pool, v_pool, block_head, block_table, ctx_len, kv_head_base=0,
                        scale=None, split_tokens=0, o=None, lse=None, dev_status=None,
                        stream=None):
    """:func:`attn_decode` with the split records in the library's fixed device
    array instead of a workspace: the C call allocates nothing.  Pass ``o`` and
    ``lse`` to allocate nothing here either.  Returns ``(o, lse)``."""
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    B, Hq, D = q.shape
    n_blocks = k_pool.shape[0]
    _need(k_pool, "k_pool", torch.bfloat16, (n_blocks, BLOCK_TOKENS, D))
    _need(v_pool, "v_pool", torch.bfloat16, (n_blocks, D, BLOCK_TOKENS))
    _need(block_head, "block_head", torch.int32, (n_blocks,))
    _need(block_table, "block_table", torch.int32)
    Hkv, max_blocks = block_table.shape[1], block_table.shape[2]
    if block_table.shape[0] != B:
        raise ValueError("block_table must be [B][Hkv][max_blocks]")
    _need(ctx_len, "ctx_len", torch.int32, (B,))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, q.shape)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (B, Hq))
    scale = float(D ** -0.5) if scale is None else float(scale)
    st = _lib.load().attn_decode_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), n_blocks, _ptr(block_head), _ptr(block_table),
        max_blocks, _ptr(ctx_len), _ptr(o), _ptr(lse), B, Hq, Hkv, D, int(kv_head_base), scale,
        int(split_tokens), _ptr(dev_status), _stream(stream))
    _lib.check("attn_decode_noalloc", st)
    return o, lse


def attn_kv_quantize_fp8(k_pool, v_pool, k8_pool=None, v8_pool=None, k_scale=None, v_scale=None,
                         stream=None):
    """bf16 pools -> (k8_pool, v8_pool, k_scale, v_scale): e4m3 bytes (uint8)
    in the same layouts and one fp32 scale per token and block."""
    torch = _torch()
    n_blocks = k_pool.shape[0]
    _need(k_pool, "k_pool", torch.bfloat16, (n_blocks, BLOCK_TOKENS, HEAD_DIM))
    _need(v_pool, "v_pool", torch.bfloat16, (n_blocks, HEAD_DIM, BLOCK_TOKENS))
    dev = k_pool.device
    if k8_pool is None:
        k8_pool = torch.empty((n_blocks, BLOCK_TOKENS, HEAD_DIM), dtype=torch.uint8, device=dev)
    if v8_pool is None:
        v8_pool = torch.empty((n_blocks, HEAD_DIM, BLOCK_TOKENS), dtype=torch.uint8, device=dev)
    if k_scale is None:
        k_scale = torch.empty((n_blocks, BLOCK_TOKENS), dtype=torch.float32, device=dev)
    if v_scale is None:
        v_scale = torch.empty((n_blocks, BLOCK_TOKENS), dtype=torch.float32, device=dev)
    _need(k8_pool, "k8_pool", torch.uint8, (n_blocks, BLOCK_TOKENS, HEAD_DIM))
    _need(v8_pool, "v8_pool", torch.uint8, (n_blocks, HEAD_DIM, BLOCK_TOKENS))
    _need(k_scale, "k_scale", torch.float32, (n_blocks, BLOCK_TOKENS))
    _need(v_scale, "v_scale", torch.float32, (n_blocks, BLOCK_TOKENS))
    st = _lib.load().attn_kv_quantize_fp8(_ptr(k_pool), _ptr(v_pool), _ptr(k8_pool), _ptr(v8_pool),
                                          _ptr(k_scale), _ptr(v_scale), n_blocks, HEAD_DIM,
                                          _stream(stream))
    _lib.check("attn_kv_quantize_fp8", st)
    return k8_pool, v8_pool, k_scale, v_scale


def attn_kv_append_fp8(k_new, v_new, k8_pool, v8_pool, k_scale, v_scale, block_head, block_table,
                       start_pos, kv_head_base=0, dev_status=None, stream=None):
    """Quantise and write ``k_new/v_new [B][T][Hkv][128]`` (bf16) into the fp8
    pools at positions ``start_pos[b] + t``."""
    torch = _torch()
    _need(k_new, "k_new", torch.bfloat16)
    B, T, Hkv, D = k_new.shape
    _need(v_new, "v_new", torch.bfloat16, k_new.shape)
    n_blocks = k8_pool.shape[0]
    _need(k8_pool, "k8_pool", torch.uint8, (n_blocks, BLOCK_TOKENS, D))
    _need(v8_pool, "v8_pool", torch.uint8, (n_blocks, D, BLOCK_TOKENS))
    _need(k_scale, "k_scale", torch.float32, (n_blocks, BLOCK_TOKENS))
    _need(v_scale, "v_scale", torch.float32, (n_blocks, BLOCK_TOKENS))
    _need(block_head, "block_head", torch.int32, (n_blocks,))
    _need(block_table, "block_table", torch.int32)
    if block_table.shape[:2] != (B, Hkv):
        raise ValueError("block_table must be [B][Hkv][max_blocks]")
    _need(start_pos, "start_pos", torch.int32, (B,))
    st = _lib.load().attn_kv_append_fp8(
        _ptr(k_new), _ptr(v_new), _ptr(k8_pool), _ptr(v8_pool), _ptr(k_scale), _ptr(v_scale),
        n_blocks, _ptr(block_head), _ptr(block_table), block_table.shape[2], _ptr(start_pos), T, B,
        Hkv, D, int(kv_head_base), _ptr(dev_status), _stream(stream))
    _lib.check("attn_kv_append_fp8", st)


def attn_decode_fp8(q, k8_pool, v8_pool, k_scale, v_scale, block_head, block_table, ctx_len,
                    kv_head_base=0, scale=None, split_tokens=0, workspace=None, o=None, lse=None,
                    dev_status=None, stream=None):
    """:func:`attn_decode` over the FP8 cache of :func:`attn_kv_quantize_fp8`."""
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    B, Hq, D = q.shape
    n_blocks = k8_pool.shape[0]
    _need(k8_pool, "k8_pool", torch.uint8, (n_blocks, BLOCK_TOKENS, D))
    _need(v8_pool, "v8_pool", torch.uint8, (n_blocks, D, BLOCK_TOKENS))
    _need(k_scale, "k_scale", torch.float32, (n_blocks, BLOCK_TOKENS))
    _need(v_scale, "v_scale", torch.float32, (n_blocks, BLOCK_TOKENS))
    _need(block_head, "block_head", torch.int32, (n_blocks,))
    _need(block_table, "block_table", torch.int32)
    Hkv, max_blocks = block_table.shape[1], block_table.shape[2]
    if block_table.shape[0] != B:
        raise ValueError("block_table must be [B][Hkv][max_blocks]")
    _need(ctx_len, "ctx_len", torch.int32, (B,))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, q.shape)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (B, Hq))
    need = attn_decode_workspace_bytes(B, Hq, max_blocks, split_tokens, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace")
    scale = float(D ** -0.5) if scale is None else float(scale)
    st = _lib.load().attn_decode_fp8(
        _ptr(q), _ptr(k8_pool), _ptr(v8_pool), _ptr(k_scale), _ptr(v_scale), n_blocks,
        _ptr(block_head), _ptr(block_table), max_blocks, _ptr(ctx_len), _ptr(o), _ptr(lse), B, Hq,
        Hkv, D, int(kv_head_base), scale, int(split_tokens), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(dev_status), _stream(stream))
    _lib.check("attn_decode_fp8", st)
    return o, lse


def _signs(signs):
    """Host int8 array of the 128 rotation signs (or None) for the C ABI; the
    library checks that every entry is +1 or -1."""
    if signs is None:
        return None, None
    import numpy as np
    a = np.ascontiguousarray(np.asarray(signs, dtype=np.int64).reshape(-1).astype(np.int8))
    if a.size != 128:
        raise ValueError("signs must hold 128 values of +1 or -1")
    return a, a.ctypes.data


def attn_quantize_fp8_blocks(x, codes=None, scales=None, signs=None, stream=None):
    """bf16 ``x [..][D]`` -> (e4m3 codes uint8 ``[..][D]``, E8M0 scales uint8
    ``[..][D/32]``): one power-of-two scale per 32 consecutive elements.
    With ``signs`` (128 values +-1), each row (D = 128) is first rotated by
    the incoherent-processing transform that :func:`attn_prefill_fp8` and
    :func:`attn_prefill_fp8_pv` apply to Q with the same signs."""
    torch = _torch()
    _need(x, "x", torch.bfloat16)
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((*x.shape[:-1], D // 32), dtype=torch.uint8, device=x.device)
    _need(codes, "codes", torch.uint8, tuple(x.shape))
    _need(scales, "scales", torch.uint8, (*x.shape[:-1], D // 32))
    keep, sp = _signs(signs)
    st = _lib.load().attn_quantize_fp8_blocks(_ptr(x), _ptr(codes), _ptr(scales), rows, D, sp,
                                              _stream(stream))
    del keep
    _lib.check("attn_quantize_fp8_blocks", st)
    return codes, scales


def attn_prefill_fp8(q, k8, k_scale, v, causal=True, scale=None, o=None, lse=None, signs=None,
                     stream=None):
    """Prefill with FP8 scores: q, v bf16 ``[B][S][H][128]``, k8 / k_scale from
    :func:`attn_quantize_fp8_blocks` on K (with the same ``signs``, when Q is
    to be rotated); returns ``(o, lse)``."""
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    B, S, Hq, D = q.shape
    Hkv = v.shape[2]
    _need(k8, "k8", torch.uint8, (B, S, Hkv, D))
    _need(k_scale, "k_scale", torch.uint8, (B, S, Hkv, D // 32))
    _need(v, "v", torch.bfloat16, (B, S, Hkv, D))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, q.shape)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (B, Hq, S))
    scale = float(D ** -0.5) if scale is None else float(scale)
    keep, sp = _signs(signs)
    st = _lib.load().attn_prefill_fp8(_ptr(q), _ptr(k8), _ptr(k_scale), _ptr(v), _ptr(o),
                                      _ptr(lse), B, S, Hq, Hkv, D, int(bool(causal)), scale, sp,
                                      _stream(stream))
    del keep
    _lib.check("attn_prefill_fp8", st)
    return o, lse


def attn_quantize_fp8_v(v, v8t=None, v_scale=None, stream=None):
    """bf16 ``v [B][S][Hkv][128]`` -> (e4m3 ``v8t [B][Hkv][128][S64]``, E8M0
    ``v_scale [B][Hkv][S64/64][256]``), S64 = S rounded up to 64: one
    power-of-two scale per (dim, 32 consecutive keys), the layout
    :func:`attn_prefill_fp8_pv` reads."""
    torch = _torch()
    _need(v, "v", torch.bfloat16)
    B, S, Hkv, D = v.shape
    s64 = (S + 63) // 64 * 64
    if v8t is None:
        v8t = torch.empty((B, Hkv, D, s64), dtype=torch.uint8, device=v.device)
    if v_scale is None:
        v_scale = torch.empty((B, Hkv, s64 // 64, 256), dtype=torch.uint8, device=v.device)
    _need(v8t, "v8t", torch.uint8, (B, Hkv, D, s64))
    _need(v_scale, "v_scale", torch.uint8, (B, Hkv, s64 // 64, 256))
    st = _lib.load().attn_quantize_fp8_v(_ptr(v), _ptr(v8t), _ptr(v_scale), B, S, Hkv, D,
                                         _stream(stream))
    _lib.check("attn_quantize_fp8_v", st)
    return v8t, v_scale


def attn_prefill_fp8_pv(q, k8, k_scale, v8t, v_scale, causal=True, scale=None, o=None, lse=None,
                        signs=None, stream=None):
    """Prefill with both products on FP8: q bf16 ``[B][S][Hq][128]``, k8 /
    k_scale from :func:`attn_quantize_fp8_blocks` on K (with the same
    ``signs``, when Q is to be rotated), v8t / v_scale from
    :func:`attn_quantize_fp8_v`; returns ``(o, lse)``."""
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    B, S, Hq, D = q.shape
    Hkv = k8.shape[2]
    s64 = (S + 63) // 64 * 64
    _need(k8, "k8", torch.uint8, (B, S, Hkv, D))
    _need(k_scale, "k_scale", torch.uint8, (B, S, Hkv, D // 32))
    _need(v8t, "v8t", torch.uint8, (B, Hkv, D, s64))
    _need(v_scale, "v_scale", torch.uint8, (B, Hkv, s64 // 64, 256))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, q.shape)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (B, Hq, S))
    scale = float(D ** -0.5) if scale is None else float(scale)
    keep, sp = _signs(signs)
    st = _lib.load().attn_prefill_fp8_pv(_ptr(q), _ptr(k8), _ptr(k_scale), _ptr(v8t),
                                         _ptr(v_scale), _ptr(o), _ptr(lse), B, S, Hq, Hkv, D,
                                         int(bool(causal)), scale, sp, _stream(stream))
    del keep
    _lib.check("attn_prefill_fp8_pv", st)
    return o, lse


def rope_apply(x, positions, base=10000.0, stream=None):
    """Rotate ``x [S][H][D]`` (bf16) in place at absolute ``positions [S]`` (int32)."""
    torch = _torch()
    _need(x, "x", torch.bfloat16)
    S, H, D = x.shape
    _need(positions, "positions", torch.int32, (S,))
    st = _lib.load().rope_apply(_ptr(x), _ptr(positions), S, H, D, float(base), _stream(stream))
    _lib.check("rope_apply", st)
    return x


def rope_apply_qk(q, k, positions, base=10000.0, stream=None):
    """Rotate ``q [S][Hq][D]`` and ``k [S][Hkv][D]`` (bf16) in place at the same
    absolute ``positions [S]`` (int32), in one launch."""
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be [S][H][D]")
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    _need(k, "k", torch.bfloat16, (S, Hkv, D))
    _need(positions, "positions", torch.int32, (S,))
    st = _lib.load().rope_apply_qk(_ptr(q), _ptr(k), _ptr(positions), S, Hq, Hkv, D, float(base),
                                   _stream(stream))
    _lib.check("rope_apply_qk", st)
    return q, k


def seq_to_head_permute_qkv(q, k, v, rank, outs=None, stream=None):
    """Relayout of Q, K and V (``[SP][S_loc][H][D]`` each, K and V with the
    same head count) for ``rank`` in one launch; returns ``(q_out, k_out, v_out)``."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    SP, S_loc, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (SP, S_loc, Hkv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [SP][S_loc][Hkv][D] with q's SP, S_loc and D")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k and v must share a dtype")
    if Hq % SP or Hkv % SP:
        raise ValueError("head counts must be divisible by SP")
    if outs is None:
        outs = (torch.empty((SP * S_loc, Hq // SP, D), dtype=q.dtype, device=q.device),
                torch.empty((SP * S_loc, Hkv // SP, D), dtype=q.dtype, device=q.device),
                torch.empty((SP * S_loc, Hkv // SP, D), dtype=q.dtype, device=q.device))
    qo, ko, vo = outs
    _need(qo, "q_out", q.dtype, (SP * S_loc, Hq // SP, D))
    _need(ko, "k_out", q.dtype, (SP * S_loc, Hkv // SP, D))
    _need(vo, "v_out", q.dtype, (SP * S_loc, Hkv // SP, D))
    st = _lib.load().seq_to_head_permute_qkv(_ptr(q), _ptr(k), _ptr(v), _ptr(qo), _ptr(ko), _ptr(vo),
                                             SP, S_loc, Hq, Hkv, D, int(rank), q.element_size(),
                                             _stream(stream))
    _lib.check("seq_to_head_permute_qkv", st)
    return qo, ko, vo


def seq_to_head_permute_qkv_rope(q, k, v, rank, positions, base=10000.0, outs=None, stream=None):
    """:func:`seq_to_head_permute_qkv` of bf16 ``q, k, v`` with RoPE at
    ``positions [SP*S_loc]`` (int32, absolute position of each output token)
    applied to Q and K in the same pass; returns ``(q_out, k_out, v_out)``."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16)
    SP, S_loc, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (SP, S_loc, Hkv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [SP][S_loc][Hkv][D] with q's SP, S_loc and D")
    if Hq % SP or Hkv % SP:
        raise ValueError("head counts must be divisible by SP")
    _need(positions, "positions", torch.int32, (SP * S_loc,))
    if outs is None:
        outs = tuple(torch.empty((SP * S_loc, H // SP, D), dtype=q.dtype, device=q.device)
                     for H in (Hq, Hkv, Hkv))
    qo, ko, vo = outs
    _need(qo, "q_out", q.dtype, (SP * S_loc, Hq // SP, D))
    _need(ko, "k_out", q.dtype, (SP * S_loc, Hkv // SP, D))
    _need(vo, "v_out", q.dtype, (SP * S_loc, Hkv // SP, D))
    st = _lib.load().seq_to_head_permute_qkv_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(qo), _ptr(ko), _ptr(vo), _ptr(positions), SP, S_loc, Hq,
        Hkv, D, int(rank), float(base), _stream(stream))
    _lib.check("seq_to_head_permute_qkv_rope", st)
    return qo, ko, vo


def seq_to_head_permute(x, rank, out=None, stream=None):
    """``x [SP][S_loc][H_tot][D]`` -> ``out [SP*S_loc][H_tot/SP][D]`` for ``rank``."""
    torch = _torch()
    _need(x, "x")
    SP, S_loc, H_tot, D = x.shape
    if H_tot % SP:
        raise ValueError("H_tot must be divisible by SP")
    if out is None:
        out = torch.empty((SP * S_loc, H_tot // SP, D), dtype=x.dtype, device=x.device)
    _need(out, "out", x.dtype, (SP * S_loc, H_tot // SP, D))
    st = _lib.load().seq_to_head_permute(_ptr(x), _ptr(out), SP, S_loc, H_tot, D, int(rank),
                                         x.element_size(), _stream(stream))
    _lib.check("seq_to_head_permute", st)
    return out


def head_to_seq_permute(x, SP, H_tot, rank, out=None, stream=None):
    """``x [SP*S_loc][H_tot/SP][D]`` (rank's heads) -> rank's head slice of
    ``out [SP][S_loc][H_tot][D]``; the other slices of ``out`` are left as
    they are (a new ``out`` is zero-filled first)."""
    torch = _torch()
    _need(x, "x")
    T, H_loc, D = x.shape
    if H_tot % SP or H_tot // SP != H_loc or T % SP:
        raise ValueError("x must be [SP*S_loc][H_tot/SP][D]")
    S_loc = T // SP
    if out is None:
        out = torch.zeros((SP, S_loc, H_tot, D), dtype=x.dtype, device=x.device)
    _need(out, "out", x.dtype, (SP, S_loc, H_tot, D))
    st = _lib.load().head_to_seq_permute(_ptr(x), _ptr(out), SP, S_loc, H_tot, D, int(rank),
                                         x.element_size(), _stream(stream))
    _lib.check("head_to_seq_permute", st)
    return out


def _cp_mode(mode):
    if mode not in CP_MODES:
        raise ValueError(f"mode must be one of {sorted(CP_MODES)}")
    return CP_MODES[mode]


def cp_shard_tokens(S, N, rank, mode) -> int:
    """Tokens that CP rank ``rank`` of ``N`` holds under ``mode`` (host only)."""
    n = _lib.load().cp_shard_tokens(int(S), int(N), int(rank), _cp_mode(mode))
    if n < 0:
        _lib.check("cp_shard_tokens", -n)
    return n


def cp_shard(x, N, rank, mode, out=None, positions=None, stream=None):
    """Rank's tokens of ``x [S][H][D]`` -> ``(out [n][H][D], positions [n] int32)``."""
    torch = _torch()
    _need(x, "x")
    S, H, D = x.shape
    n = cp_shard_tokens(S, N, rank, mode)
    if out is None:
        out = torch.empty((n, H, D), dtype=x.dtype, device=x.device)
    _need(out, "out", x.dtype, (n, H, D))
    if positions is None:
        positions = torch.empty((n,), dtype=torch.int32, device=x.device)
    _need(positions, "positions", torch.int32, (n,))
    st = _lib.load().cp_shard(_ptr(x), _ptr(out), _ptr(positions), S, H, D, x.element_size(),
                              int(N), int(rank), _cp_mode(mode), _stream(stream))
    _lib.check("cp_shard", st)
    return out, positions


def cp_unshard(x, S, N, rank, mode, out=None, stream=None):
    """``x [n][H][D]`` of rank back into its rows of ``out [S][H][D]`` (other
    rows untouched; a new ``out`` is zero-filled first)."""
    torch = _torch()
    _need(x, "x")
    n, H, D = x.shape
    if n != cp_shard_tokens(S, N, rank, mode):
        raise ValueError("x does not hold this rank's token count")
    if out is None:
        out = torch.zeros((S, H, D), dtype=x.dtype, device=x.device)
    _need(out, "out", x.dtype, (S, H, D))
    st = _lib.load().cp_unshard(_ptr(x), _ptr(out), S, H, D, x.element_size(), int(N), int(rank),
                                _cp_mode(mode), _stream(stream))
    _lib.check("cp_unshard", st)
    return out


def attn_key_limits(q_pos, k_pos, out=None, stream=None):
    """``key_limit[b][i] = #{j : k_pos[b][j] <= q_pos[b][i]}`` (int32; k_pos
    ascending); ``q_pos [B][Sq]`` or ``[Sq]``, ``k_pos`` likewise."""
    torch = _torch()
    qp = q_pos if q_pos.dim() == 2 else q_pos[None]
    kp = k_pos if k_pos.dim() == 2 else k_pos[None]
    B, Sq = qp.shape
    Sk = kp.shape[1]
    _need(qp, "q_pos", torch.int32, (B, Sq))
    _need(kp, "k_pos", torch.int32, (B, Sk))
    if out is None:
        out = torch.empty((B, Sq), dtype=torch.int32, device=qp.device)
    _need(out, "key_limit", torch.int32, (B, Sq))
    st = _lib.load().attn_key_limits(_ptr(qp), _ptr(kp), _ptr(out), B, Sq, Sk, _stream(stream))
    _lib.check("attn_key_limits", st)
    return out


def attn_prefill_limited(q, k, v, key_limit, scale=None, o=None, lse=None, accumulate=False,
                         stream=None):
    """bf16 attention where row i of batch b sees keys ``[0, key_limit[b][i])``;
    q ``[B][Sq][Hq][128]``, k/v ``[B][Sk][Hkv][128]``; returns ``(o, lse)``.
    With ``accumulate``, ``o``/``lse`` hold a partial over other keys and this
    call merges into them in place."""
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    _need(k, "k", torch.bfloat16, (B, Sk, Hkv, D))
    _need(v, "v", torch.bfloat16, (B, Sk, Hkv, D))
    _need(key_limit, "key_limit", torch.int32, (B, Sq))
    if accumulate and (o is None or lse is None):
        raise ValueError("accumulate needs the partial to merge into: pass o and lse")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, q.shape)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (B, Hq, Sq))
    scale = float(D ** -0.5) if scale is None else float(scale)
    st = _lib.load().attn_prefill_limited(_ptr(q), _ptr(k), _ptr(v), _ptr(key_limit), _ptr(o),
                                          _ptr(lse), B, Sq, Sk, Hq, Hkv, D, scale,
                                          int(bool(accumulate)), _stream(stream))
    _lib.check("attn_prefill_limited", st)
    return o, lse


def attn_merge(o_a, lse_a, o_b, lse_b, o=None, lse=None, stream=None):
    """Merge two normalised partials (bf16 O ``[B][S][H][D]``, fp32 LSE
    ``[B][H][S]``) of the same rows; ``o``/``lse`` may be ``o_a``/``lse_a``."""
    torch = _torch()
    _need(o_a, "o_a", torch.bfloat16)
    B, S, H, D = o_a.shape
    _need(o_b, "o_b", torch.bfloat16, (B, S, H, D))
    _need(lse_a, "lse_a", torch.float32, (B, H, S))
    _need(lse_b, "lse_b", torch.float32, (B, H, S))
    if o is None:
        o = torch.empty_like(o_a)
    _need(o, "o", torch.bfloat16, (B, S, H, D))
    if lse is None:
        lse = torch.empty_like(lse_a)
    _need(lse, "lse", torch.float32, (B, H, S))
    st = _lib.load().attn_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse),
                                B, S, H, D, _stream(stream))
    _lib.check("attn_merge", st)
    return o, lse


def mfma_rate_flops(n_wg, iters) -> int:
    """Floating-point operations of one :func:`measure_mfma_rate` launch."""
    return int(n_wg) * 8 * int(iters) * 4 * 32768


def measure_mfma_rate(n_wg=1024, iters=65536, seed=1, a_from_lds=False, out=None, stream=None):
    """Enqueue one launch of the sustained-MFMA yardstick (bf16 32x32x16 MFMA
    on random operands, ``mfma_rate_flops(n_wg, iters)`` flops; with
    ``a_from_lds`` each MFMA's A operand is read from LDS just before it);
    ``out`` is a float32 device buffer of ``n_wg * 512`` elements.  Time it
    with events on ``stream``."""
    torch = _torch()
    if n_wg < 1 or n_wg > 65536 or iters < 4 or iters > (1 << 24) or iters % 4:
        raise ValueError("n_wg must be in [1, 65536] and iters a multiple of 4 in [4, 2^24]")
    if out is None:
        out = torch.empty(n_wg * 512, dtype=torch.float32, device="cuda")
    _need(out, "out", torch.float32, (n_wg * 512,))
    st = _lib.load().attn_measure_mfma_rate(_ptr(out), int(n_wg), int(iters), int(seed) & 0xFFFFFFFF,
                                            int(bool(a_from_lds)), _stream(stream))
    _lib.check("attn_measure_mfma_rate", st)
    return out


def measure_hbm_read(buf, waves=4096, out=None, stream=None):
    """Enqueue one streaming read of the device tensor ``buf`` (16-byte
    aligned) by ``waves`` waves; returns ``(out, bytes_read)``."""
    torch = _torch()
    _need(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(waves * 64, dtype=torch.int32, device=buf.device)
    _need(out, "out", torch.int32, (waves * 64,))
    lib = _lib.load()
    st = lib.attn_measure_hbm_read(_ptr(buf), nbytes, _ptr(out), int(waves), _stream(stream))
    _lib.check("attn_measure_hbm_read", st)
    return out, int(lib.attn_measure_hbm_read_bytes(nbytes, int(waves)))


def measure_hbm_copy(src, dst, stream=None):
    """Enqueue a streaming copy of ``src`` into ``dst`` (same byte size,
    16-byte aligned; ``dst`` may be ``src`` itself, any other overlap is
    refused); returns the bytes copied."""
    _need(src, "src")
    _need(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    st = _lib.load().attn_measure_hbm_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream))
    _lib.check("attn_measure_hbm_copy", st)
    return nbytes
