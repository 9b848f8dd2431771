"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws random numbers and arranges them into the layouts the
attention library consumes (dense tensors, shard tensors, paged KV pools with
block tables and head tags).  It performs none of the attention arithmetic:
no scores, no softmax, no rotary embedding, no relayout of the method.  Both
``oracle/`` and the GPU tests receive the exact same arrays from here.

Storage conventions
-------------------
* bf16 tensors are numpy ``uint16`` arrays holding the bf16 bit patterns
  (round-to-nearest-even from fp32 draws).  ``torch`` consumers view them as
  ``torch.bfloat16``; the oracle widens the bit patterns itself.
* fp32 tensors are numpy ``float32``.
* Paged KV pools: ``k_pool[n_blocks][64][D]`` (token-major) and
  ``v_pool[n_blocks][D][64]`` (dimension-major), both bf16 bits, with
  ``block_table[B][Hkv][max_blocks]`` int32 physical block ids (-1 where
  unused) and ``block_head[n_blocks]`` int32 global KV-head tags (-1 for
  blocks that hold nothing).
"""
from __future__ import annotations

import numpy as np

BLOCK_TOKENS = 64
BF16_NAN_BITS = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# bf16 bit conversion (representation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    """N(0,1) draws rounded to bf16, generated in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(size=e - s, dtype=np.float32))
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Dense workloads
# --------------------------------------------------------------------------
def tiny_exact(seed: int = 1, S: int = 256, D: int = 64):
    """1 batch, 1 head, S queries and keys, fp32 N(0,1), scale 1/sqrt(D)."""
    rng = np.random.default_rng(seed)
    q = normal_f32(rng, (1, S, 1, D))
    k = normal_f32(rng, (1, S, 1, D))
    v = normal_f32(rng, (1, S, 1, D))
    return dict(q=q, k=k, v=v, scale=float(1.0 / np.sqrt(D)))


def dense_bf16(seed: int, B: int, S: int, Hq: int, Hkv: int, D: int = 128):
    """Dense bf16 Q [B][S][Hq][D], K/V [B][S][Hkv][D], N(0,1); positions 0..S-1."""
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (B, S, Hq, D))
    k = normal_bf16(rng, (B, S, Hkv, D))
    v = normal_bf16(rng, (B, S, Hkv, D))
    pos = np.arange(S, dtype=np.int32)
    return dict(q=q, k=k, v=v, positions=pos, scale=float(1.0 / np.sqrt(D)))


def causal_gqa(seed: int = 2, S: int = 32768, Hq: int = 16, Hkv: int = 2, D: int = 128):
    """One sequence-parallel shard's heads: batch 1, full sequence, causal GQA."""
    return dense_bf16(seed, 1, S, Hq, Hkv, D)


def ulysses_shards(seed: int = 3, SP: int = 4, S_loc: int = 16384, Hq_tot: int = 64,
                   Hkv_tot: int = 8, D: int = 128):
    """Sequence-sharded inputs as they sit before the head relayout.

    Shard k holds tokens whose global positions are ``S_loc*k + s``.
    Q is ``[SP][S_loc][Hq_tot][D]``, K/V are ``[SP][S_loc][Hkv_tot][D]``.
    """
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (SP, S_loc, Hq_tot, D))
    k = normal_bf16(rng, (SP, S_loc, Hkv_tot, D))
    v = normal_bf16(rng, (SP, S_loc, Hkv_tot, D))
    shard_pos = (np.arange(SP, dtype=np.int64)[:, None] * S_loc
                 + np.arange(S_loc, dtype=np.int64)[None, :]).astype(np.int32)
    return dict(q=q, k=k, v=v, shard_positions=shard_pos, SP=SP, S_loc=S_loc,
                scale=float(1.0 / np.sqrt(D)))


# --------------------------------------------------------------------------
# Paged KV cache construction
# --------------------------------------------------------------------------
def n_blocks_for(tokens: int) -> int:
    return (int(tokens) + BLOCK_TOKENS - 1) // BLOCK_TOKENS


def scatter_into_pool(k_pool, v_pool, blk, k_tok, v_tok, slot0: int = 0):
    """Place up to 64 consecutive tokens (``[n][D]`` bf16 bits) into block ``blk``
    starting at slot ``slot0``; V goes in dimension-major."""
    n = k_tok.shape[0]
    k_pool[blk, slot0:slot0 + n, :] = k_tok
    v_pool[blk, :, slot0:slot0 + n] = v_tok.T


def decode_cache(seed: int = 4, B: int = 32, ctx_lo: int = 8192, ctx_hi: int = 131072,
                 Hq: int = 16, Hkv: int = 2, D: int = 128, kv_head_base: int = 0,
                 ctx_lens=None, extra_blocks: int = 0, keep_contiguous: bool = True):
    """Single-token decode over a head-sharded paged cache.

    Context lengths are integers drawn uniformly from [ctx_lo, ctx_hi] (both
    ends included) unless ``ctx_lens`` is given.  Physical block ids are a
    seeded permutation over the pool.  Unused slots of partially filled blocks,
    and whole spare blocks, are filled with NaN so that a kernel reading past
    ``ctx_len`` is caught.
    """
    rng = np.random.default_rng(seed)
    if ctx_lens is None:
        ctx_lens = rng.integers(ctx_lo, ctx_hi, size=B, endpoint=True)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    nb = np.array([n_blocks_for(c) for c in ctx_lens], dtype=np.int64)
    max_blocks = int(nb.max()) if B else 0
    n_used = int(nb.sum()) * Hkv
    n_blocks = n_used + extra_blocks
    perm = rng.permutation(n_blocks).astype(np.int32)
    q = normal_bf16(rng, (B, Hq, D))
    k_pool = np.full((n_blocks, BLOCK_TOKENS, D), BF16_NAN_BITS, dtype=np.uint16)
    v_pool = np.full((n_blocks, D, BLOCK_TOKENS), BF16_NAN_BITS, dtype=np.uint16)
    table = np.full((B, Hkv, max(max_blocks, 1)), -1, dtype=np.int32)
    tags = np.full((n_blocks,), -1, dtype=np.int32)
    k_seq, v_seq = [], []
    nxt = 0
    for b in range(B):
        ctx = int(ctx_lens[b])
        kb = normal_bf16(rng, (ctx, Hkv, D))
        vb = normal_bf16(rng, (ctx, Hkv, D))
        for g in range(Hkv):
            for j in range(int(nb[b])):
                blk = int(perm[nxt]); nxt += 1
                table[b, g, j] = blk
                tags[blk] = kv_head_base + g
                t0, t1 = j * BLOCK_TOKENS, min(ctx, (j + 1) * BLOCK_TOKENS)
                scatter_into_pool(k_pool, v_pool, blk, kb[t0:t1, g], vb[t0:t1, g])
        if keep_contiguous:
            k_seq.append(kb)
            v_seq.append(vb)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=table, block_head=tags,
                ctx_len=ctx_lens.astype(np.int32), max_blocks=max(max_blocks, 1),
                k_seq=k_seq, v_seq=v_seq, kv_head_base=kv_head_base,
                scale=float(1.0 / np.sqrt(D)), Hq=Hq, Hkv=Hkv, D=D)


class BlockAllocator:
    """Free-list allocator of physical KV blocks, in the order blocks are requested."""

    def __init__(self, n_blocks: int, seed: int | None = None):
        ids = np.arange(n_blocks, dtype=np.int32)
        if seed is not None:
            ids = np.random.default_rng(seed).permutation(ids).astype(np.int32)
        self.free = list(ids[::-1])

    def alloc(self) -> int:
        return int(self.free.pop())


def chunked_prefill(seed: int = 5, B: int = 4, S: int = 131072, C: int = 8192,
                    Hq: int = 16, Hkv: int = 2, D: int = 128, kv_head_base: int = 0):
    """Requests processed in C-token chunks against a growing paged cache.

    Returns full per-request Q/K/V (``[B][S][H][D]``), an empty pool large
    enough for every request, and a block table whose entries are assigned from
    a free list as chunks complete (requests advance in lockstep, so blocks
    interleave across requests and heads).  Tags are written at assignment.
    """
    d = dense_bf16(seed, B, S, Hq, Hkv, D)
    nb = n_blocks_for(S)
    n_blocks = B * Hkv * nb
    alloc = BlockAllocator(n_blocks)
    table = np.full((B, Hkv, nb), -1, dtype=np.int32)
    tags = np.full((n_blocks,), -1, dtype=np.int32)
    n_chunks = (S + C - 1) // C
    for c in range(n_chunks):
        j0 = (c * C) // BLOCK_TOKENS
        j1 = n_blocks_for(min(S, (c + 1) * C))
        for b in range(B):
            for g in range(Hkv):
                for j in range(j0, j1):
                    if table[b, g, j] < 0:
                        blk = alloc.alloc()
                        table[b, g, j] = blk
                        tags[blk] = kv_head_base + g
    d.update(block_table=table, block_head=tags, n_blocks=n_blocks, max_blocks=nb,
             C=C, n_chunks=n_chunks, kv_head_base=kv_head_base, Hq=Hq, Hkv=Hkv, D=D)
    return d


def sample_rows(rng_seed: int, S: int, n: int, forced=()):
    """Sorted unique query-row sample: ``n`` seeded rows plus the forced ones."""
    rng = np.random.default_rng(rng_seed)
    n = min(n, S)
    rows = set(int(r) for r in rng.choice(S, size=n, replace=False))
    rows.update(int(r) for r in forced if 0 <= int(r) < S)
    return np.array(sorted(rows), dtype=np.int64)
