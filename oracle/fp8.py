"""FP8 (OCP e4m3) quantisation of the KV cache — TEST INFRASTRUCTURE ONLY.

Written from the format definition, not from any implementation.  Where the
pages mention quantised attention they leave the number format open: the
FP8 path of "Flash Attention and distributed inference" (FA3 section)
quantises blocks to 8-bit floats, and the Ulysses inference article (§5.4)
stores a KV cache quantised in groups.  Reading taken here: the OCP 8-bit
e4m3 format (the one gfx950 implements), with one fp32 scale per group of
one token's head vector (a K row or a V column of a 64-token block).

e4m3: sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field
0 holds the subnormals m * 2^-9; fields 1..15 hold (1 + m/8) * 2^(e-7),
except e = 15, m = 7, which is NaN.  There are no infinities; the largest
finite magnitude is 448.

Quantising a group x: scale = amax(|x|) / 448 (fp32 division), each
element y = x / scale (fp32 division), rounded to the nearest e4m3 value
with ties to the even code, magnitudes at or above 448 saturating to 448.
A group of zeros gets scale 0 and codes 0.  Dequantised value:
decode(code) * scale.
"""
from __future__ import annotations

import numpy as np


def _magnitudes() -> np.ndarray:
    """Value of codes 0 .. 126 (sign bit clear, NaN code 127 excluded)."""
    vals = []
    for c in range(127):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3_MAG = _magnitudes()          # ascending
E4M3_MAX = 448.0


def fp8_e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, E4M3_MAG[np.minimum(c & 0x7F, 126)])
    return np.where(c & 0x80, -mag, mag)


def fp8_e4m3_encode(x) -> np.ndarray:
    """Values -> uint8 codes: nearest e4m3 value, ties to the even code,
    saturating at +-448; the sign bit is the sign bit of x (so -0 and
    negative values that round to zero give 0x80).  Finite inputs only."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle: fp8 encode of a non-finite value")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(E4M3_MAG, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - E4M3_MAG[lo]
    d_hi = E4M3_MAG[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(E4M3_MAG[hi] == a, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def quantize_groups(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantise each group (last axis) of fp32-representable values.
    Returns (codes uint8, same shape; scale fp32, shape[:-1])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)            # fp32 division, as the kernel
    codes = fp8_e4m3_encode(y)
    codes = np.where((scale > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def dequantize_groups(codes, scale) -> np.ndarray:
    return fp8_e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def quantize_kv_pool(k_pool_bits, v_pool_bits):
    """Paged bf16 pools -> fp8 pools with one scale per token and block.

    k_pool [n][64][D] (token-major): group = one token's K row.
    v_pool [n][D][64] (dimension-major): group = one token's V column.
    Returns (k8 [n][64][D], v8 [n][D][64], k_scale [n][64], v_scale [n][64]).
    """
    kb = np.asarray(k_pool_bits, dtype=np.uint16)
    vb = np.asarray(v_pool_bits, dtype=np.uint16)
    kf = (kb.astype(np.uint32) << 16).view(np.float32)
    vf = (vb.astype(np.uint32) << 16).view(np.float32)
    k8, ks = quantize_groups(kf)
    v8t, vs = quantize_groups(np.swapaxes(vf, 1, 2))        # [n][64][D]: token groups
    return k8, np.ascontiguousarray(np.swapaxes(v8t, 1, 2)), ks, vs


def gather_dequantized(k8, v8, k_scale, v_scale, block_table, ctx_len, requests=None):
    """Per request b (all, or those listed in ``requests``), the dequantised K
    and V of its first ctx_len[b] tokens in order, [ctx][Hkv][D] fp64 each:
    token t of KV head g sits in slot t % 64 of physical block
    block_table[b][g][t // 64] (the paged layout of the Ulysses inference
    article, §2.3).  Only the blocks of those requests are dequantised."""
    table = np.asarray(block_table)
    B, Hkv, _ = table.shape
    D = np.asarray(k8).shape[2]
    ks, vs = [], []
    for b in (range(B) if requests is None else requests):
        T = int(ctx_len[b])
        nb = (T + 63) // 64
        kb = np.empty((T, Hkv, D))
        vb = np.empty((T, Hkv, D))
        for g in range(Hkv):
            blk = table[b, g, :nb]
            k = dequantize_groups(k8[blk], k_scale[blk])                        # [nb][64][D]
            v = dequantize_groups(np.swapaxes(v8[blk], 1, 2), v_scale[blk])     # [nb][64][D]
            kb[:, g] = k.reshape(nb * 64, D)[:T]
            vb[:, g] = v.reshape(nb * 64, D)[:T]
        ks.append(kb)
        vs.append(vb)
    return ks, vs


# ---------------------------------------------------------------------------
# FP8 scores for prefill: power-of-two block scales
# ---------------------------------------------------------------------------
# FA3's FP8 path ("Flash Attention and distributed inference", §18.5) runs the
# attention matmuls on FP8 operands with block quantisation; the pages give no
# format or scale rule.  Reading taken here: QK^T in OCP e4m3, each block of 32
# consecutive head dimensions of one token (one query row, or one key row)
# with its own scale 2^e, e the smallest integer with amax <= 448 * 2^e (so the
# block's largest magnitude lands in (224, 448] and nothing saturates); codes
# are x / 2^e rounded to the nearest e4m3 value, ties to even.  A block of
# zeros gets e = -127 and zero codes.  The query row is multiplied by
# c = scale * log2(e) in fp32 before it is quantised, so the scores come out in
# log2 units and the softmax is taken in base 2; P V stays in bf16.
E8M0_BIAS = 127
BLOCK = 32


def block_exponents(x, block=BLOCK):
    """e per block of ``block`` values along the last axis: the smallest
    integer with max|x| <= 448 * 2^e (fp32 inputs, so the test is exact in
    fp64); -127 for an all-zero block."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x.reshape(*x.shape[:-1], -1, block)), axis=-1)
    e = np.full(amax.shape, -E8M0_BIAS, dtype=np.int64)
    nz = amax > 0
    # frexp: amax = m * 2^E with m in [0.5, 1); the candidate 2^(E-9) times 448
    # is 0.875 * 2^E, so e = E - 9 exactly when amax <= 0.875 * 2^E
    m, E = np.frexp(amax[nz])
    e[nz] = np.maximum(np.where(m <= 0.875, E - 9, E - 8), -E8M0_BIAS)   # E8M0 floor 2^-127
    return e


def quantize_blocks(x, block=BLOCK):
    """(codes uint8 [...][D], exponents int [...][D/block]) of fp32 values."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    e = block_exponents(x, block)
    scaled = x.reshape(*x.shape[:-1], -1, block) / np.exp2(e)[..., None]   # exact: powers of two
    codes = fp8_e4m3_encode(scaled).reshape(x.shape)
    return codes.astype(np.uint8), e


def dequantize_blocks(codes, e, block=BLOCK):
    c = fp8_e4m3_decode(codes)
    v = c.reshape(*c.shape[:-1], -1, block) * np.exp2(np.asarray(e, dtype=np.float64))[..., None]
    return v.reshape(c.shape)


def e8m0_bytes(e):
    """Scale exponents as E8M0 bytes (2^(byte - 127))."""
    return (np.asarray(e, dtype=np.int64) + E8M0_BIAS).astype(np.uint8)


def query_multiplier(scale):
    """The fp32 factor the query rows are multiplied by: fp32(scale) * fp32(log2 e),
    rounded to fp32."""
    return np.float32(np.float32(scale) * np.float32(1.4426950408889634))


# ---------------------------------------------------------------------------
# Incoherent processing: Q and K rotated before they are quantised
# ---------------------------------------------------------------------------
# FA3's FP8 path (same section) pairs block quantisation with incoherent
# processing: Q and K are multiplied by one random orthogonal matrix before
# quantisation, which leaves Q K^T unchanged and spreads a few large channels
# over all of them.  The pages name the step and give no matrix.  Reading
# taken here: M = diag(s) H, H the 128 x 128 Sylvester-Hadamard matrix
# (H[i][j] = (-1)^popcount(i & j), entries +-1) and s a vector of +-1 signs
# the caller draws; x -> x M for each 128-dim row.  H H^T = 128 I, so
# (q M)(k M)^T = 128 q.k, and the query multiplier becomes c / 128 (exact: a
# power of two).  Arithmetic, fixed so that quantised codes are reproducible:
# the signs are applied to the bf16 values (exact), x H is the fast
# Walsh-Hadamard transform in fp32 taken in the usual butterfly order (span
# 1, 2, 4, ..., 64; element i with bit `span` clear pairs with i + span and
# the pair becomes (a + b, a - b)), and the query is then multiplied by
# c / 128 in fp32 (one rounding) before it is block-quantised.  V is not
# rotated.
HADAMARD_D = 128


def hadamard_matrix(n=HADAMARD_D):
    """Sylvester-Hadamard matrix of order n (a power of two), by doubling:
    H_2n = [[H, H], [H, -H]]."""
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_rotate(x, signs):
    """x [..][128] (fp32 values) -> (s * x) H in fp32 by butterflies, in the
    order stated above."""
    s = np.asarray(signs)
    if s.shape != (HADAMARD_D,) or not np.all(np.abs(s) == 1):
        raise ValueError("oracle: signs must be 128 values of +-1")
    y = (np.asarray(x, dtype=np.float32) * s.astype(np.float32)).astype(np.float32)
    lead = y.shape[:-1]
    span = 1
    while span < HADAMARD_D:
        y = y.reshape(*lead, HADAMARD_D // (2 * span), 2, span)
        a, b = y[..., 0, :], y[..., 1, :]
        y = np.stack([(a + b).astype(np.float32), (a - b).astype(np.float32)], axis=-2)
        span *= 2
    return y.reshape(*lead, HADAMARD_D)


def prefill_fp8_operands(q_bits, k_bits, scale, signs=None):
    """Dequantised fp64 Q'' [..][D] (of q * c, log2 units) and K'' [..][D] from
    bf16 bit patterns, following the reading above; with ``signs`` (128 values
    +-1), Q and K are first rotated as stated above (then Q'' approximates
    (q M) c / 128 and K'' approximates k M, whose product is c q.k)."""
    qf = (np.asarray(q_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    kf = (np.asarray(k_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    c = query_multiplier(scale)
    if signs is not None:
        qf, kf = hadamard_rotate(qf, signs), hadamard_rotate(kf, signs)
        c = np.float32(c / np.float32(HADAMARD_D))
    qs = (qf * c).astype(np.float32)                 # fp32 product, as the kernel
    qc, qe = quantize_blocks(qs)
    kc, ke = quantize_blocks(kf)
    return dequantize_blocks(qc, qe), dequantize_blocks(kc, ke)


def quantize_rotated_rows(x_bits, signs):
    """K rows [..][128] bf16 bits -> (codes, exponents) of x M: the rotated
    rows block-quantised (what the K quantiser with signs stores)."""
    xf = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return quantize_blocks(hadamard_rotate(xf, signs))


def attention_fp8(q_bits, k_bits, v_bits, scale, causal=False, rows=None, signs=None):
    """What the FP8-score prefill computes, in fp64: attention over the
    dequantised Q'' (already in log2 units) and K'' with base-2 softmax,
    i.e. weights 2^(q''.k''), and V as given (bf16).  q [B][S][Hq][D],
    k/v [B][S][Hkv][D] bf16 bits.  Returns (out [B][R][Hq][D], lse [B][Hq][R])
    with lse in natural-log units.  Causal row i sees keys 0..i."""
    import oracle
    B, S = q_bits.shape[:2]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    qd, kd = prefill_fp8_operands(np.ascontiguousarray(np.asarray(q_bits)[:, rows]), k_bits, scale,
                                  signs)
    lim = (np.broadcast_to(rows[None, :] + 1, (B, rows.size)) if causal
           else np.full((B, rows.size), np.asarray(k_bits).shape[1], dtype=np.int64))
    # exp(ln 2 * s) = 2^s: the natural-log softmax of ln2-scaled scores
    return oracle.attention_rows(qd, kd, v_bits, lim, float(np.log(2.0)))


def dequantized_v_keys(v_bits):
    """V [B][S][Hkv][D] bf16 bits -> fp64 V'' with each (dim, block of 32
    consecutive keys) quantised by the power-of-two rule above (the FP8 P V
    reading: the key axis is the contraction axis of P V, so V's blocks run
    along keys).  Keys past the last multiple of 32 form a shorter block as if
    padded with zeros."""
    v = (np.asarray(v_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    B, S, H, D = v.shape
    Sp = -(-S // BLOCK) * BLOCK
    vt = np.zeros((B, H, D, Sp), np.float32)
    vt[..., :S] = np.transpose(v, (0, 2, 3, 1))
    c, e = quantize_blocks(vt)
    return np.ascontiguousarray(np.transpose(dequantize_blocks(c, e)[..., :S], (0, 3, 1, 2)))


def attention_fp8_pv(q_bits, k_bits, v_bits, scale, causal=False, rows=None, signs=None):
    """What the FP8-score, FP8-P.V prefill computes before P is rounded:
    attention_fp8 with V replaced by V'' (dequantised along keys).  The
    kernel also rounds the weights P to e4m3 before P V, which depends on its
    running reference maximum; that rounding is bounded in the tests, not
    modelled here."""
    import oracle
    B, S = q_bits.shape[:2]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    qd, kd = prefill_fp8_operands(np.ascontiguousarray(np.asarray(q_bits)[:, rows]), k_bits, scale,
                                  signs)
    lim = (np.broadcast_to(rows[None, :] + 1, (B, rows.size)) if causal
           else np.full((B, rows.size), np.asarray(k_bits).shape[1], dtype=np.int64))
    return oracle.attention_rows(qd, kd, dequantized_v_keys(v_bits), lim, float(np.log(2.0)))
