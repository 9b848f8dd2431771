"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The HIP product path
(``long_context_attention_tiled_amd``) never imports it, and this package
never imports that one; both only share the seeded inputs of ``synth``.

What it computes (each function cites the passage it follows):

* :func:`attention` — the naive definition of attention ("Flash Attention and
  distributed inference", §18.2) evaluated row by row with the three-pass
  softmax of §18.3, in fp64 (C library ``liboracle.so``).
* :func:`rope` — rotary embedding at absolute global positions (Ulysses
  inference article, §3.2 and §5.3).  Pairing and frequency schedule are a
  reading (rotate-half, ``base**(-2i/D)``); parity of that reading is pinned
  only by textbook RoPE properties, not by the pages.
* :func:`permute` — the sequence-shard -> head-shard relayout of the same
  article's §2.2; :func:`unpermute` — the reverse exchange of the same
  section for the attention output (head shard back to sequence shards).
* :func:`paged_gather` — read-back of the head-sharded paged KV cache of the
  article's §2.3.
* :func:`partial_attention` / :func:`lse_merge` — the rescale identity of
  §18.3 applied to key ranges; used only to cross-check :func:`attention`.
* :mod:`oracle.fp8` — OCP e4m3 encode/decode and the per-token quantisation
  of the paged KV cache (the FP8 cache variant; format reading stated there).
* :func:`cp_tokens` — which tokens each context-parallel rank holds under the
  contiguous (ring), striped (round-robin) and zigzag (in-seq-split) splits
  of "LLM推理中的多卡切分" §3.5 / §3.5.1.
* :func:`attention_positions` — attention whose causal mask is stated on
  token positions, for such shards; :func:`merge_normalized` combines
  normalised partial results (O, LSE) with the same rescale identity.

Inputs may be float64, float32, or uint16 arrays of bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (fp64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_attention_rows.argtypes = [vp, i32, vp, i32, vp, i32, i64, i64, i64, i64, i64,
                                              i64, vp, dbl, vp, vp]
        lib.oracle_attention_rows.restype = i32
        lib.oracle_attention_positions.argtypes = [vp, i32, vp, i32, vp, i32, i64, i64, i64, i64,
                                                   i64, i64, vp, vp, dbl, vp, vp]
        lib.oracle_attention_positions.restype = i32
        lib.oracle_rope.argtypes = [vp, i32, vp, i64, i64, i64, dbl, vp]
        lib.oracle_rope.restype = i32
        lib.oracle_permute.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64]
        lib.oracle_permute.restype = i32
        lib.oracle_unpermute.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64]
        lib.oracle_unpermute.restype = i32
        lib.oracle_paged_gather.argtypes = [vp, vp, i64, vp, i64, i64, i64, vp, i64, i64, vp, vp]
        lib.oracle_paged_gather.restype = i32
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return 0
    if a.dtype == np.float32:
        return 1
    if a.dtype == np.uint16:
        return 2
    raise TypeError(f"oracle: unsupported dtype {a.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def widen(a: np.ndarray) -> np.ndarray:
    """fp64 view of an input array (bf16 bit patterns widened exactly)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def num_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------
# Attention (naive definition, three-pass softmax)
# ---------------------------------------------------------------------------
def attention_rows(q_rows, k, v, key_limit, scale):
    """Attention of selected rows.

    q_rows: [B][R][Hq][D]; k, v: [B][Sk][Hkv][D]; key_limit: [B][R] number of
    leading keys each row may see.  Returns (out [B][R][Hq][D] fp64,
    lse [B][Hq][R] fp64).
    """
    q_rows = np.ascontiguousarray(q_rows)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    B, R, Hq, D = q_rows.shape
    Bk, Sk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape:
        raise ValueError("oracle: shape mismatch")
    lim = np.ascontiguousarray(np.broadcast_to(np.asarray(key_limit, dtype=np.int64), (B, R)))
    out = np.empty((B, R, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)
    rc = _load().oracle_attention_rows(_ptr(q_rows), _dtype_code(q_rows), _ptr(k), _dtype_code(k),
                                       _ptr(v), _dtype_code(v), B, R, Sk, Hq, Hkv, D, _ptr(lim),
                                       float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_rows failed ({rc})")
    return out, lse


def attention(q, k, v, scale, causal=False, rows=None):
    """Dense attention over ``[B][S][H][D]`` tensors for the given query rows.

    Non-causal rows see every key; causal row i sees keys 0..i (global token
    indices, the full-sequence mask of the Ulysses article §5.3).
    Returns (out [B][R][Hq][D], lse [B][Hq][R]).
    """
    B, Sq = q.shape[0], q.shape[1]
    rows = np.arange(Sq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    q_rows = np.ascontiguousarray(q[:, rows])
    if causal:
        lim = np.broadcast_to(rows[None, :] + 1, (B, rows.size))
    else:
        lim = np.full((B, rows.size), k.shape[1], dtype=np.int64)
    return attention_rows(q_rows, k, v, lim, scale)


def decode_attention(q, k_seq, v_seq, ctx_len, scale):
    """One new query per request over its whole cached context.

    q: [B][Hq][D]; k_seq[b], v_seq[b]: [ctx_b][Hkv][D] contiguous per request.
    Every key 0..ctx_len-1 is visible (the new token's own K/V included).
    Returns (out [B][Hq][D], lse [B][Hq]).
    """
    B = q.shape[0]
    outs, lses = [], []
    for b in range(B):
        n = int(ctx_len[b])
        o, l = attention_rows(q[b:b + 1, None], k_seq[b][None, :n], v_seq[b][None, :n],
                              np.array([[n]]), scale)
        outs.append(o[0, 0])
        lses.append(l[0, :, 0])
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------
# Rotary embedding, relayout, paged gather
# ---------------------------------------------------------------------------
def rope(x, positions, base=10000.0):
    """fp64 rotary embedding of ``x`` ``[S][H][D]`` at absolute ``positions``."""
    x = np.ascontiguousarray(x)
    S, H, D = x.shape
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64))
    if pos.shape != (S,):
        raise ValueError("oracle: positions must be [S]")
    out = np.empty((S, H, D), dtype=np.float64)
    rc = _load().oracle_rope(_ptr(x), _dtype_code(x), _ptr(pos), S, H, D, float(base), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_rope failed ({rc})")
    return out


def permute(x, rank):
    """``[SP][S_loc][H_tot][D]`` -> ``[SP*S_loc][H_tot/SP][D]`` for ``rank``."""
    x = np.ascontiguousarray(x)
    SP, S_loc, H_tot, D = x.shape
    if H_tot % SP:
        raise ValueError("oracle: H_tot must be divisible by SP")
    out = np.empty((SP * S_loc, H_tot // SP, D), dtype=x.dtype)
    rc = _load().oracle_permute(_ptr(x), _ptr(out), SP, S_loc, H_tot, D, int(rank), x.itemsize)
    if rc != 0:
        raise RuntimeError(f"oracle_permute failed ({rc})")
    return out


def unpermute(x, SP, H_tot, rank, out=None):
    """``[SP*S_loc][H_tot/SP][D]`` of ``rank`` -> its head slice of
    ``out [SP][S_loc][H_tot][D]`` (other slices untouched; zeros if ``out``
    is not given)."""
    x = np.ascontiguousarray(x)
    T, H_loc, D = x.shape
    if H_tot % SP or H_tot // SP != H_loc or T % SP:
        raise ValueError("oracle: shape mismatch")
    S_loc = T // SP
    if out is None:
        out = np.zeros((SP, S_loc, H_tot, D), dtype=x.dtype)
    elif out.shape != (SP, S_loc, H_tot, D) or out.dtype != x.dtype or not out.flags.c_contiguous:
        raise ValueError("oracle: bad out")
    rc = _load().oracle_unpermute(_ptr(x), _ptr(out), SP, S_loc, H_tot, D, int(rank), x.itemsize)
    if rc != 0:
        raise RuntimeError(f"oracle_unpermute failed ({rc})")
    return out


def paged_gather(k_pool, v_pool, block_table, n_tok, T_max=None):
    """Read a paged cache back into ``[B][T_max][Hkv][D]`` K and V (bit copies)."""
    k_pool = np.ascontiguousarray(k_pool, dtype=np.uint16)
    v_pool = np.ascontiguousarray(v_pool, dtype=np.uint16)
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    n_tok = np.ascontiguousarray(np.asarray(n_tok, dtype=np.int64))
    B, Hkv, max_blocks = table.shape
    n_blocks, bt, D = k_pool.shape
    T_max = int(n_tok.max()) if T_max is None else int(T_max)
    k_out = np.zeros((B, T_max, Hkv, D), dtype=np.uint16)
    v_out = np.zeros((B, T_max, Hkv, D), dtype=np.uint16)
    rc = _load().oracle_paged_gather(_ptr(k_pool), _ptr(v_pool), n_blocks, _ptr(table), B, Hkv,
                                     max_blocks, _ptr(n_tok), T_max, D, _ptr(k_out), _ptr(v_out))
    if rc != 0:
        raise RuntimeError(f"oracle_paged_gather failed ({rc})")
    return k_out, v_out


# ---------------------------------------------------------------------------
# Key-range partials and their merge (rescale identity, §18.3)
# ---------------------------------------------------------------------------
def attention_positions(q, k, v, q_pos, k_pos, scale):
    """Attention of ``q [B][Sq][Hq][D]`` over ``k, v [B][Sk][Hkv][D]`` where a
    query at position P attends the keys at positions <= P ("LLM推理中的多卡切分"
    §3.5: the causal mask between two ranks' shards).  ``q_pos [B][Sq]``,
    ``k_pos [B][Sk]``.  Returns (out [B][Sq][Hq][D], lse [B][Hq][Sq]); rows
    with no allowed key get NaN and -inf."""
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape:
        raise ValueError("oracle: shape mismatch")
    qp = np.ascontiguousarray(np.broadcast_to(np.asarray(q_pos, dtype=np.int64), (B, Sq)))
    kp = np.ascontiguousarray(np.broadcast_to(np.asarray(k_pos, dtype=np.int64), (B, Sk)))
    out = np.empty((B, Sq, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64)
    rc = _load().oracle_attention_positions(_ptr(q), _dtype_code(q), _ptr(k), _dtype_code(k),
                                            _ptr(v), _dtype_code(v), B, Sq, Sk, Hq, Hkv, D,
                                            _ptr(qp), _ptr(kp), float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_positions failed ({rc})")
    return out, lse


CP_MODES = ("contiguous", "striped", "zigzag")


def cp_tokens(S, N, mode, rank):
    """Ascending token indices that context-parallel rank ``rank`` of ``N``
    holds for a sequence of ``S`` tokens ("LLM推理中的多卡切分" §3.5, §3.5.1):

    * ``contiguous`` — ring attention's split into N consecutive blocks;
    * ``striped`` — round-robin: the tokens with index mod N == rank
      (S % N == 0, the stated constraint);
    * ``zigzag`` — in-seq-split: the sequence cut into 2N consecutive blocks,
      rank i taking blocks i and 2N-1-i (S >= 2N, the stated constraint).

    Block boundaries where S is not a multiple of the block count are a
    reading: block b spans [floor(b*S/n), floor((b+1)*S/n)).
    """
    if not (0 <= rank < N):
        raise ValueError("oracle: rank out of range")
    bound = lambda b, n: (b * S) // n
    if mode == "contiguous":
        if S < N:
            raise ValueError("oracle: S < N")
        return np.arange(bound(rank, N), bound(rank + 1, N), dtype=np.int64)
    if mode == "striped":
        if S % N:
            raise ValueError("oracle: S % N != 0")
        return np.arange(rank, S, N, dtype=np.int64)
    if mode == "zigzag":
        if S < 2 * N:
            raise ValueError("oracle: S < 2N")
        a, b = rank, 2 * N - 1 - rank
        return np.concatenate([np.arange(bound(a, 2 * N), bound(a + 1, 2 * N)),
                               np.arange(bound(b, 2 * N), bound(b + 1, 2 * N))]).astype(np.int64)
    raise ValueError(f"oracle: unknown CP mode {mode!r}")


def merge_normalized(parts):
    """Combine normalised partials [(O_s, LSE_s)] of the same queries over
    disjoint key sets: M = max LSE_s, w_s = exp(LSE_s - M),
    O = sum w_s O_s / sum w_s, LSE = M + ln sum w_s (the rescale identity of
    "Flash Attention and distributed inference" §18.3).  Partials with
    LSE = -inf (no key) get weight 0; if all do, O = 0 and LSE = -inf.
    Layouts: O [B][S][H][D] with LSE [B][H][S] (the attention outputs), or
    any O [..., D] with LSE [...]."""
    Os = [np.asarray(O, dtype=np.float64) for O, _ in parts]
    Ls = [np.asarray(L, dtype=np.float64) for _, L in parts]
    four = Os[0].ndim == 4 and Ls[0].ndim == 3
    if four:
        Ls = [np.swapaxes(L, 1, 2) for L in Ls]      # -> [B][S][H]
    M = np.max(np.stack(Ls), axis=0)
    Ms = np.where(np.isfinite(M), M, 0.0)
    num = np.zeros(Os[0].shape)
    den = np.zeros(M.shape)
    for O, L in zip(Os, Ls):
        live = np.isfinite(L)
        w = np.where(live, np.exp(np.where(live, L, 0.0) - Ms), 0.0)
        num = num + w[..., None] * np.where(live[..., None], O, 0.0)
        den = den + w
    safe = np.where(den > 0, den, 1.0)
    O = np.where(den[..., None] > 0, num / safe[..., None], 0.0)
    lse = np.where(den > 0, Ms + np.log(safe), -np.inf)
    if four:
        lse = np.swapaxes(lse, 1, 2)
    return O, lse


def partial_attention(q_vec, k_rows, v_rows, scale):
    """Unnormalised partial of one query over a key range.

    Returns (m, l, o): m = max score, l = sum exp(s - m), o = sum exp(s - m) v.
    An empty range gives (-inf, 0, zeros).
    """
    q_vec = widen(np.asarray(q_vec))
    k_rows = widen(np.asarray(k_rows))
    v_rows = widen(np.asarray(v_rows))
    if k_rows.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(q_vec.shape[-1])
    s = scale * (k_rows @ q_vec)
    m = float(np.max(s))
    w = np.exp(s - m)
    return m, float(np.sum(w)), w @ v_rows


def lse_merge(parts):
    """Combine partials: M = max m_s, w_s = exp(m_s - M), O = sum w_s o_s / sum w_s l_s."""
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    M = float(np.max(ms))
    num = np.zeros_like(parts[0][2], dtype=np.float64)
    den = 0.0
    for m, l, o in parts:
        if m == -np.inf:
            continue
        w = np.exp(m - M)
        num = num + w * o
        den += w * l
    return num / den, M + np.log(den)
