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

import concurrent.futures as cf
import os

import numpy as np

BLOCK_TOKENS = 64
BF16_NAN_BITS = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# bf16 bit conversion (representation only)
# --------------------------------------------------------------------------
CHUNK = 1 << 22          # elements per independently seeded draw chunk


def _pool_size() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).reshape(-1)
    out = np.empty(u.shape, dtype=np.uint16)
    for s in range(0, u.size, CHUNK):
        c = u[s:s + CHUNK]
        lsb = (c >> np.uint32(16)) & np.uint32(1)
        # finite inputs: c + 0x7FFF + lsb cannot wrap (largest is 0xFF7FFFFF)
        out[s:s + CHUNK] = ((c + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x.reshape(-1))
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _seq(seed) -> np.random.SeedSequence:
    return seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)


def normal_f32(seed, shape) -> np.ndarray:
    """N(0,1) fp32 draws.  Chunk i of the flattened array comes from child i
    of the seed sequence, so the result does not depend on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    n_chunks = (n + CHUNK - 1) // CHUNK
    children = _seq(seed).spawn(n_chunks)

    def fill(i):
        np.random.default_rng(children[i]).standard_normal(
            out=out[i * CHUNK:min(n, (i + 1) * CHUNK)], dtype=np.float32)

    if n_chunks > 1:
        with cf.ThreadPoolExecutor(_pool_size()) as ex:
            list(ex.map(fill, range(n_chunks)))
    elif n_chunks == 1:
        fill(0)
    return out.reshape(shape)


def normal_bf16(seed, shape) -> np.ndarray:
    """N(0,1) draws rounded to bf16 bits (see :func:`normal_f32`)."""
    x = normal_f32(seed, shape).reshape(-1)
    out = np.empty(x.size, dtype=np.uint16)
    starts = list(range(0, x.size, CHUNK))

    def conv(s):
        out[s:s + CHUNK] = f32_to_bf16_bits(x[s:s + CHUNK])

    if len(starts) > 1:
        with cf.ThreadPoolExecutor(_pool_size()) as ex:
            list(ex.map(conv, starts))
    elif starts:
        conv(0)
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Dense workloads
# --------------------------------------------------------------------------
def tiny_exact(seed: int = 1, S: int = 256, D: int = 64):
    """1 batch, 1 head, S queries and keys, fp32 N(0,1), scale 1/sqrt(D)."""
    sq, sk, sv = _seq(seed).spawn(3)
    q = normal_f32(sq, (1, S, 1, D))
    k = normal_f32(sk, (1, S, 1, D))
    v = normal_f32(sv, (1, S, 1, D))
    return dict(q=q, k=k, v=v, scale=float(1.0 / np.sqrt(D)))


def dense_bf16(seed: int, B: int, S: int, Hq: int, Hkv: int, D: int = 128):
    """Dense bf16 Q [B][S][Hq][D], K/V [B][S][Hkv][D], N(0,1); positions 0..S-1."""
    sq, sk, sv = _seq(seed).spawn(3)
    q = normal_bf16(sq, (B, S, Hq, D))
    k = normal_bf16(sk, (B, S, Hkv, D))
    v = normal_bf16(sv, (B, S, Hkv, D))
    pos = np.arange(S, dtype=np.int32)
    return dict(q=q, k=k, v=v, positions=pos, scale=float(1.0 / np.sqrt(D)))


def dense_bf16_outliers(seed: int, B: int, S: int, Hq: int, Hkv: int, D: int = 128,
                        n_channels: int = 4, q_gain: float = 8.0, k_gain: float = 2.0):
    """dense_bf16 with a few outlier channels, the way a handful of feature
    dimensions dominate the queries and keys of trained models: the same
    ``n_channels`` head dims (a seeded choice) of every Q row are multiplied
    by ``q_gain`` and of every K row by ``k_gain`` before rounding to bf16.
    With the defaults the scores have a standard deviation of about 3 (in
    natural-log units, after 1/sqrt(D)).  V is N(0, 1)."""
    sq, sk, sv, sc = _seq(seed).spawn(4)
    ch = np.random.default_rng(sc).choice(D, size=n_channels, replace=False)
    gq = np.ones(D, np.float32)
    gk = np.ones(D, np.float32)
    gq[ch], gk[ch] = q_gain, k_gain
    q = f32_to_bf16_bits(normal_f32(sq, (B, S, Hq, D)) * gq)
    k = f32_to_bf16_bits(normal_f32(sk, (B, S, Hkv, D)) * gk)
    v = normal_bf16(sv, (B, S, Hkv, D))
    pos = np.arange(S, dtype=np.int32)
    return dict(q=q, k=k, v=v, positions=pos, scale=float(1.0 / np.sqrt(D)), channels=np.sort(ch))


def hadamard_signs(seed: int, D: int = 128) -> np.ndarray:
    """The random signs (+1 / -1, int8) of the incoherent-processing rotation."""
    return np.random.default_rng(_seq(seed)).choice(np.array([-1, 1], np.int8), size=D)


def causal_gqa(seed: int = 2, S: int = 32768, Hq: int = 16, Hkv: int = 2, D: int = 128):
    """One sequence-parallel shard's heads: batch 1, full sequence, causal GQA."""
    return dense_bf16(seed, 1, S, Hq, Hkv, D)


def ulysses_shards(seed: int = 3, SP: int = 4, S_loc: int = 16384, Hq_tot: int = 64,
                   Hkv_tot: int = 8, D: int = 128):
    """Sequence-sharded inputs as they sit before the head relayout.

    Shard k holds tokens whose global positions are ``S_loc*k + s``.
    Q is ``[SP][S_loc][Hq_tot][D]``, K/V are ``[SP][S_loc][Hkv_tot][D]``.
    """
    sq, sk, sv = _seq(seed).spawn(3)
    q = normal_bf16(sq, (SP, S_loc, Hq_tot, D))
    k = normal_bf16(sk, (SP, S_loc, Hkv_tot, D))
    v = normal_bf16(sv, (SP, S_loc, Hkv_tot, D))
    shard_pos = (np.arange(SP, dtype=np.int64)[:, None] * S_loc
                 + np.arange(S_loc, dtype=np.int64)[None, :]).astype(np.int32)
    return dict(q=q, k=k, v=v, shard_positions=shard_pos, SP=SP, S_loc=S_loc,
                scale=float(1.0 / np.sqrt(D)))


# --------------------------------------------------------------------------
# Paged KV cache construction
# --------------------------------------------------------------------------
def n_blocks_for(tokens: int) -> int:
    return (int(tokens) + BLOCK_TOKENS - 1) // BLOCK_TOKENS


def _fill_pool(k_pool, v_pool, ids, k_tok, v_tok):
    """Place ``n`` consecutive tokens (``[n][D]`` bf16 bits, n <= 64*len(ids))
    into blocks ``ids`` in order; V is stored dimension-major.  Slots past
    ``n`` in the last block are left as they are."""
    n, D = k_tok.shape
    nb = len(ids)
    full = n // BLOCK_TOKENS
    if full:
        kb = k_tok[:full * BLOCK_TOKENS].reshape(full, BLOCK_TOKENS, D)
        vb = v_tok[:full * BLOCK_TOKENS].reshape(full, BLOCK_TOKENS, D)
        k_pool[ids[:full]] = kb
        v_pool[ids[:full]] = vb.transpose(0, 2, 1)
    rest = n - full * BLOCK_TOKENS
    if rest:
        assert nb == full + 1
        k_pool[ids[full], :rest] = k_tok[full * BLOCK_TOKENS:]
        v_pool[ids[full], :, :rest] = v_tok[full * BLOCK_TOKENS:].T


def decode_cache(seed: int = 4, B: int = 32, ctx_lo: int = 8192, ctx_hi: int = 131072,
                 Hq: int = 16, Hkv: int = 2, D: int = 128, kv_head_base: int = 0,
                 ctx_lens=None, extra_blocks: int = 0, keep_contiguous: bool = True,
                 with_content: bool = True):
    """Single-token decode over a head-sharded paged cache.

    Context lengths are integers drawn uniformly from [ctx_lo, ctx_hi] (both
    ends included) unless ``ctx_lens`` is given.  Physical block ids are a
    seeded permutation over the pool; request b's blocks for local KV head g
    come next in that permutation, logical block by logical block.  Unused
    slots of partially filled blocks, and whole spare blocks, are NaN so that
    a kernel reading past ``ctx_len`` is caught.  With ``with_content=False``
    only the structure (lengths, table, tags, q) is built and the pools are
    left to the caller.
    """
    s_meta, s_q, s_kv = _seq(seed).spawn(3)
    rng = np.random.default_rng(s_meta)
    if ctx_lens is None:
        ctx_lens = rng.integers(ctx_lo, ctx_hi, size=B, endpoint=True)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    nb = np.array([n_blocks_for(c) for c in ctx_lens], dtype=np.int64)
    max_blocks = max(int(nb.max()) if B else 0, 1)
    n_blocks = int(nb.sum()) * Hkv + extra_blocks
    perm = rng.permutation(n_blocks).astype(np.int32)
    q = normal_bf16(s_q, (B, Hq, D))
    if with_content:
        k_pool = np.full((n_blocks, BLOCK_TOKENS, D), BF16_NAN_BITS, dtype=np.uint16)
        v_pool = np.full((n_blocks, D, BLOCK_TOKENS), BF16_NAN_BITS, dtype=np.uint16)
    else:
        k_pool = v_pool = None
    table = np.full((B, Hkv, max_blocks), -1, dtype=np.int32)
    tags = np.full((n_blocks,), -1, dtype=np.int32)
    kv_seeds = s_kv.spawn(2 * B) if B else []
    k_seq, v_seq = [], []
    nxt = 0
    for b in range(B):
        ctx = int(ctx_lens[b])
        if with_content:
            kb = normal_bf16(kv_seeds[2 * b], (ctx, Hkv, D))
            vb = normal_bf16(kv_seeds[2 * b + 1], (ctx, Hkv, D))
        for g in range(Hkv):
            ids = perm[nxt:nxt + nb[b]]
            nxt += int(nb[b])
            table[b, g, :nb[b]] = ids
            tags[ids] = kv_head_base + g
            if with_content:
                _fill_pool(k_pool, v_pool, ids, kb[:, g], vb[:, g])
        if keep_contiguous and with_content:
            k_seq.append(kb)
            v_seq.append(vb)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=table, block_head=tags,
                n_blocks=n_blocks,
                ctx_len=ctx_lens.astype(np.int32), max_blocks=max_blocks,
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


def chunked_block_table(B: int, S: int, C: int, Hkv: int, kv_head_base: int = 0):
    """Block table of requests processed in C-token chunks: entries are taken
    from a free list as chunks complete (requests advance in lockstep, so
    blocks interleave across requests and heads); tags are set at assignment.
    Returns (block_table [B][Hkv][ceil(S/64)], block_head [n_blocks], n_blocks)."""
    nb = n_blocks_for(S)
    n_blocks = B * Hkv * nb
    alloc = BlockAllocator(n_blocks)
    table = np.full((B, Hkv, nb), -1, dtype=np.int32)
    tags = np.full((n_blocks,), -1, dtype=np.int32)
    for c in range((S + C - 1) // C):
        j0 = (c * C) // BLOCK_TOKENS
        j1 = n_blocks_for(min(S, (c + 1) * C))
        for b in range(B):
            for g in range(Hkv):
                for j in range(j0, j1):
                    if table[b, g, j] < 0:
                        blk = alloc.alloc()
                        table[b, g, j] = blk
                        tags[blk] = kv_head_base + g
    return table, tags, n_blocks


def chunked_prefill(seed: int = 5, B: int = 4, S: int = 131072, C: int = 8192,
                    Hq: int = 16, Hkv: int = 2, D: int = 128, kv_head_base: int = 0):
    """Requests processed in C-token chunks against a growing paged cache:
    full per-request Q/K/V (``[B][S][H][D]``), the pool size, and the block
    table of :func:`chunked_block_table`."""
    d = dense_bf16(seed, B, S, Hq, Hkv, D)
    table, tags, n_blocks = chunked_block_table(B, S, C, Hkv, kv_head_base)
    d.update(block_table=table, block_head=tags, n_blocks=n_blocks, max_blocks=table.shape[2],
             C=C, n_chunks=(S + C - 1) // C, kv_head_base=kv_head_base, Hq=Hq, Hkv=Hkv, D=D)
    return d


def sample_rows(seed: int, S: int, n: int, forced=()):
    """Sorted unique query-row sample: ``n`` seeded rows plus the forced ones."""
    rng = np.random.default_rng(seed)
    n = min(n, S)
    rows = set(int(r) for r in rng.choice(S, size=n, replace=False))
    rows.update(int(r) for r in forced if 0 <= int(r) < S)
    return np.array(sorted(rows), dtype=np.int64)
