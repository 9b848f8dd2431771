"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test states what it pins and the basis: a closed form, an identity the
pages state, a worked example printed on the pages (``tests/golden``), or a
textbook property.  A plausible slip in the oracle (dropped scale, wrong sign,
swapped K/V, wrong GQA head map, causal off-by-one, wrong rotary pairing or
frequency) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(rng, *shape):
    return rng.standard_normal(size=shape)


# ---------------------------------------------------------------------------
# Attention: closed forms
# ---------------------------------------------------------------------------
def test_two_key_closed_form():
    """Two keys: weights are a logistic of the scaled score gap (pins scale,
    sign, K vs V roles).  softmax([a, b]) = [1/(1+e^(b-a)), 1/(1+e^(a-b))]."""
    rng = np.random.default_rng(11)
    D = 8
    q = rand(rng, 1, 1, 1, D)
    k = rand(rng, 1, 2, 1, D)
    v = rand(rng, 1, 2, 1, D)
    scale = 0.37
    a = scale * float(q[0, 0, 0] @ k[0, 0, 0])
    b = scale * float(q[0, 0, 0] @ k[0, 1, 0])
    w0 = 1.0 / (1.0 + math.exp(b - a))
    w1 = 1.0 / (1.0 + math.exp(a - b))
    want = w0 * v[0, 0, 0] + w1 * v[0, 1, 0]
    out, lse = oracle.attention(q, k, v, scale)
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=0, atol=1e-14)
    assert abs(lse[0, 0, 0] - (max(a, b) + math.log(math.exp(a - max(a, b)) + math.exp(b - max(a, b))))) < 1e-14


def test_uniform_scores_give_mean_of_v():
    """q = 0 makes every score 0, so the output is the mean of V and
    LSE = ln(n) (definition of softmax, §18.3)."""
    rng = np.random.default_rng(12)
    n, D = 37, 16
    q = np.zeros((1, 3, 2, D))
    k = rand(rng, 1, n, 2, D)
    v = rand(rng, 1, n, 2, D)
    out, lse = oracle.attention(q, k, v, 0.25)
    for h in range(2):
        np.testing.assert_allclose(out[0, :, h], np.broadcast_to(v[0, :, h].mean(0), (3, D)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(n), atol=1e-14)


def test_single_key_returns_v():
    """One visible key: output is that key's V and LSE is its scaled score."""
    rng = np.random.default_rng(13)
    D = 32
    q = rand(rng, 2, 1, 4, D)
    k = rand(rng, 2, 1, 1, D)
    v = rand(rng, 2, 1, 1, D)
    out, lse = oracle.attention(q, k, v, 0.5)
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(out[b, 0, h], v[b, 0, 0], atol=0)
            assert abs(lse[b, h, 0] - 0.5 * float(q[b, 0, h] @ k[b, 0, 0])) < 1e-13


def test_causal_row0_and_row1():
    """Causal row 0 sees only key 0 (returns V[0]); row 1 sees exactly keys 0
    and 1 (two-key closed form) — pins the j <= i convention."""
    rng = np.random.default_rng(14)
    S, D = 9, 8
    q = rand(rng, 1, S, 1, D)
    k = rand(rng, 1, S, 1, D)
    v = rand(rng, 1, S, 1, D)
    scale = 0.3
    out, _ = oracle.attention(q, k, v, scale, causal=True)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 0], atol=0)
    a = scale * float(q[0, 1, 0] @ k[0, 0, 0])
    b = scale * float(q[0, 1, 0] @ k[0, 1, 0])
    w0 = 1.0 / (1.0 + math.exp(b - a))
    np.testing.assert_allclose(out[0, 1, 0], w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0], atol=1e-14)


def test_shift_invariance_and_needle():
    """Adding a constant to every score of a row leaves softmax unchanged;
    a key with an overwhelming score returns its value (needle)."""
    rng = np.random.default_rng(15)
    n, D = 50, 16
    q = rand(rng, 1, 1, 1, D)
    k = rand(rng, 1, n, 1, D)
    v = rand(rng, 1, n, 1, D)
    # shift: append a coordinate with q = 1 and identical k -> every score += c*scale
    q2 = np.concatenate([q, np.ones((1, 1, 1, 1))], axis=-1)
    k2 = np.concatenate([k, np.full((1, n, 1, 1), 5.0)], axis=-1)
    v2 = np.concatenate([v, np.zeros((1, n, 1, 1))], axis=-1)
    o1, _ = oracle.attention(q, k, v, 0.2)
    o2, _ = oracle.attention(q2, k2, v2, 0.2)
    np.testing.assert_allclose(o2[0, 0, 0, :D], o1[0, 0, 0], atol=1e-14)
    kn = k.copy()
    kn[0, 17, 0] = 400.0 * q[0, 0, 0] / np.linalg.norm(q[0, 0, 0])
    o3, _ = oracle.attention(q, kn, v, 1.0)
    np.testing.assert_allclose(o3[0, 0, 0], v[0, 17, 0], atol=1e-12)


# ---------------------------------------------------------------------------
# Attention: identities and independent formulations
# ---------------------------------------------------------------------------
def online_softmax_attention(qv, K, V, scale):
    """Streaming form of §18.3, element by element: running max m and
    denominator l with rescaling of the output accumulator, divided once at
    the end.  Written here independently of the oracle."""
    m, l = -math.inf, 0.0
    acc = np.zeros(V.shape[-1])
    for j in range(K.shape[0]):
        x = scale * float(qv @ K[j])
        m_new = max(m, x)
        corr = math.exp(m - m_new) if m != -math.inf else 0.0
        l = l * corr + math.exp(x - m_new)
        acc = acc * corr + math.exp(x - m_new) * V[j]
        m = m_new
    return acc / l, m + math.log(l)


def test_three_pass_equals_online_recurrence():
    """The three-pass oracle equals the online recurrence (the pages state the
    two are mathematically identical)."""
    rng = np.random.default_rng(16)
    S, D = 60, 24
    q = rand(rng, 1, S, 2, D)
    k = rand(rng, 1, S, 1, D) * 3.0
    v = rand(rng, 1, S, 1, D)
    out, lse = oracle.attention(q, k, v, 0.2, causal=True)
    for i in [0, 1, 7, 31, 59]:
        for h in range(2):
            o_ref, l_ref = online_softmax_attention(q[0, i, h], k[0, :i + 1, 0], v[0, :i + 1, 0], 0.2)
            np.testing.assert_allclose(out[0, i, h], o_ref, rtol=1e-12, atol=1e-13)
            assert abs(lse[0, h, i] - l_ref) < 1e-12


def test_bruteforce_matrix_form_small():
    """Full-matrix softmax(Q K^T * scale) V in numpy (the naive form of §18.2)
    agrees with the row-wise oracle for N <= 64, causal and not."""
    rng = np.random.default_rng(17)
    for S, D, causal in [(1, 4, False), (16, 8, True), (64, 64, False), (64, 32, True)]:
        q = rand(rng, 1, S, 1, D)
        k = rand(rng, 1, S, 1, D)
        v = rand(rng, 1, S, 1, D)
        s = (q[0, :, 0] @ k[0, :, 0].T) * 0.125
        if causal:
            s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
        a = np.exp(s - s.max(1, keepdims=True))
        a /= a.sum(1, keepdims=True)
        out, _ = oracle.attention(q, k, v, 0.125, causal=causal)
        np.testing.assert_allclose(out[0, :, 0], a @ v[0, :, 0], rtol=1e-12, atol=1e-13)


def test_pure_python_fsum_tiny():
    """Pure-Python loops with math.fsum for N <= 16 (independent of numpy)."""
    rng = np.random.default_rng(18)
    S, D = 16, 5
    q = rand(rng, 1, S, 1, D)
    k = rand(rng, 1, S, 1, D)
    v = rand(rng, 1, S, 1, D)
    out, _ = oracle.attention(q, k, v, 0.7, causal=True)
    for i in range(S):
        sc = [0.7 * math.fsum(q[0, i, 0, d] * k[0, j, 0, d] for d in range(D)) for j in range(i + 1)]
        mx = max(sc)
        e = [math.exp(x - mx) for x in sc]
        z = math.fsum(e)
        for d in range(D):
            want = math.fsum(e[j] / z * v[0, j, 0, d] for j in range(i + 1))
            assert abs(out[0, i, 0, d] - want) < 1e-13


def test_gqa_equals_mha_with_repeated_kv():
    """Query head h reads KV head h // (Hq/Hkv): GQA equals MHA with each KV
    head repeated group-size times (pins the head map)."""
    rng = np.random.default_rng(19)
    S, Hq, Hkv, D = 12, 8, 2, 16
    q = rand(rng, 1, S, Hq, D)
    k = rand(rng, 1, S, Hkv, D)
    v = rand(rng, 1, S, Hkv, D)
    out, lse = oracle.attention(q, k, v, 0.3, causal=True)
    kr = np.repeat(k, Hq // Hkv, axis=2)
    vr = np.repeat(v, Hq // Hkv, axis=2)
    out2, lse2 = oracle.attention(q, kr, vr, 0.3, causal=True)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)
    # and differs from the wrong (modulo) mapping
    kw = np.tile(k, (1, 1, Hq // Hkv, 1))
    vw = np.tile(v, (1, 1, Hq // Hkv, 1))
    out3, _ = oracle.attention(q, kw, vw, 0.3, causal=True)
    assert np.abs(out3 - out).max() > 1e-3


def test_split_merge_equals_unsplit():
    """Partials over key ranges merged by the rescale identity of §18.3 equal
    the unsplit three-pass result, including an empty range."""
    rng = np.random.default_rng(20)
    n, D = 300, 16
    q = rand(rng, 1, 1, 1, D)
    k = rand(rng, 1, n, 1, D) * 2
    v = rand(rng, 1, n, 1, D)
    out, lse = oracle.attention(q, k, v, 0.25)
    cuts = [0, 64, 64, 130, 257, 300]
    parts = [oracle.partial_attention(q[0, 0, 0], k[0, a:b, 0], v[0, a:b, 0], 0.25)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, l = oracle.lse_merge(parts)
    np.testing.assert_allclose(o, out[0, 0, 0], rtol=1e-12, atol=1e-14)
    assert abs(l - lse[0, 0, 0]) < 1e-12


def test_chunked_rows_equal_causal_rows():
    """A chunk row i at cache offset c sees keys 0..c+i, i.e. exactly causal
    row c+i of the concatenated sequence (chunked prefill, multi-GPU
    partitioning article §2.2)."""
    rng = np.random.default_rng(21)
    S, C, D = 40, 8, 8
    q = rand(rng, 1, S, 2, D)
    k = rand(rng, 1, S, 1, D)
    v = rand(rng, 1, S, 1, D)
    full, _ = oracle.attention(q, k, v, 0.4, causal=True)
    for c0 in range(0, S, C):
        rows = np.arange(C)
        lim = (c0 + rows + 1)[None, :]
        o, _ = oracle.attention_rows(q[:, c0:c0 + C], k, v, lim, 0.4)
        np.testing.assert_array_equal(o, full[:, c0:c0 + C])


def test_empty_row_is_nan_with_minus_inf_lse():
    q = np.ones((1, 1, 1, 4))
    k = np.ones((1, 3, 1, 4))
    out, lse = oracle.attention_rows(q, k, k, np.zeros((1, 1), np.int64), 1.0)
    assert np.isnan(out).all() and lse[0, 0, 0] == -np.inf


def test_bf16_inputs_widen_exactly():
    """bf16 bit patterns are widened exactly (no re-rounding) on the way in."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((1, 20, 1, 8)).astype(np.float32)
    xb = synth.f32_to_bf16_bits(x)
    xf = synth.bf16_bits_to_f32(xb).astype(np.float64)
    o1, l1 = oracle.attention(xb, xb, xb, 0.3, causal=True)
    o2, l2 = oracle.attention(xf, xf, xf, 0.3, causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ---------------------------------------------------------------------------
# Rotary embedding
# ---------------------------------------------------------------------------
def test_rope_closed_form_d2_and_d4():
    """D=2: theta_0 = 1, so position p rotates (x0, x1) by p radians
    counter-clockwise.  D=4, base 10000: pairs (0,2) at theta 1 and (1,3) at
    theta 10000^(-1/2) = 0.01 (the rotate-half reading)."""
    x = np.array([[[0.3, -1.2]]])
    for p in [0, 1, 5, 1000]:
        got = oracle.rope(x, [p])
        c, s = math.cos(p), math.sin(p)
        np.testing.assert_allclose(got[0, 0], [0.3 * c + 1.2 * s, -1.2 * c + 0.3 * s], atol=1e-15)
    x4 = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    p = 7
    got = oracle.rope(x4, [p])
    c0, s0 = math.cos(7.0), math.sin(7.0)
    c1, s1 = math.cos(0.07), math.sin(0.07)
    want = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    np.testing.assert_allclose(got[0, 0], want, atol=1e-14)


def test_rope_identity_norm_and_relative_position():
    """R(0) = I; rotations keep the norm; <R(p)q, R(p')k> depends only on
    p - p' (textbook RoPE properties; shifts up to 2^17)."""
    rng = np.random.default_rng(23)
    D = 128
    x = rng.standard_normal((3, 2, D))
    np.testing.assert_array_equal(oracle.rope(x, [0, 0, 0]), x)
    r = oracle.rope(x, [5, 70000, 131071])
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for p, pk, t in [(10, 3, 1000), (65535, 0, 65536), (100, 90000, 31)]:
        a = float(oracle.rope(q, [p])[0, 0] @ oracle.rope(k, [pk])[0, 0])
        b = float(oracle.rope(q, [p + t])[0, 0] @ oracle.rope(k, [pk + t])[0, 0])
        assert abs(a - b) < 1e-9 * np.linalg.norm(q) * np.linalg.norm(k)


# ---------------------------------------------------------------------------
# Relayout
# ---------------------------------------------------------------------------
def _read_golden(name):
    spec = {}
    heads = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "rank":
                heads[int(parts[1])] = [int(x) for x in parts[3:]]
            else:
                spec[parts[0]] = int(parts[1])
    return spec, heads


def test_permute_worked_example():
    """The article's worked example: SP=4, 16-token shards, 8 heads; after the
    exchange rank r holds heads 2r, 2r+1 for all 64 tokens in global order."""
    spec, heads = _read_golden("ulysses_relayout_example.txt")
    SP, S_loc, H, D = spec["SP"], spec["S_loc"], spec["H_tot"], 3
    code = np.zeros((SP, S_loc, H, D), dtype=np.int64)
    for k_ in range(SP):
        for s in range(S_loc):
            for h in range(H):
                for d in range(D):
                    code[k_, s, h, d] = ((k_ * 100 + s) * 100 + h) * 100 + d
    for r in range(SP):
        out = oracle.permute(code, r)
        assert out.shape == (spec["tokens_after"], spec["heads_after"], D)
        for t in range(spec["tokens_after"]):
            for hl, hg in enumerate(heads[r]):
                for d in range(D):
                    assert out[t, hl, d] == ((t // S_loc * 100 + t % S_loc) * 100 + hg) * 100 + d


def test_permute_all_ranks_is_a_bijection():
    rng = np.random.default_rng(24)
    SP, S_loc, H, D = 4, 5, 8, 6
    x = rng.integers(0, 2**16, size=(SP, S_loc, H, D), dtype=np.uint16)
    outs = [oracle.permute(x, r) for r in range(SP)]
    # stack heads back: rank r's heads are global heads r*H/SP .. (r+1)*H/SP - 1
    full = np.concatenate(outs, axis=1)          # [SP*S_loc][H][D]
    np.testing.assert_array_equal(full.reshape(SP, S_loc, H, D), x)


def test_unpermute_worked_example_reversed():
    """The reverse exchange of the same worked example: rank r holds heads
    2r, 2r+1 of all 64 tokens; sending every rank's heads back must leave
    shard k with tokens 16k .. 16k+15 and all 8 heads, each head at its
    global index."""
    spec, heads = _read_golden("ulysses_relayout_example.txt")
    SP, S_loc, H, D = spec["SP"], spec["S_loc"], spec["H_tot"], 3
    T = spec["tokens_after"]
    code = lambda t, h, d: (t * 100 + h) * 100 + d
    out = np.full((SP, S_loc, H, D), -1, dtype=np.int64)
    for r in range(SP):
        x = np.array([[[code(t, hg, d) for d in range(D)] for hg in heads[r]] for t in range(T)],
                     dtype=np.int64)
        oracle.unpermute(x, SP, H, r, out=out)
    for k_ in range(SP):
        for s in range(S_loc):
            for h in range(H):
                for d in range(D):
                    assert out[k_, s, h, d] == code(k_ * S_loc + s, h, d)


def test_unpermute_inverts_permute_and_touches_only_its_heads():
    rng = np.random.default_rng(25)
    SP, S_loc, H, D = 4, 5, 8, 6
    x = rng.integers(0, 2**16, size=(SP, S_loc, H, D), dtype=np.uint16)
    back = np.zeros_like(x)
    for r in range(SP):
        before = back.copy()
        oracle.unpermute(oracle.permute(x, r), SP, H, r, out=back)
        changed = np.argwhere((back != before).any(axis=-1))
        assert set(int(h) for h in changed[:, 2]) <= set(range(r * H // SP, (r + 1) * H // SP))
    np.testing.assert_array_equal(back, x)


# ---------------------------------------------------------------------------
# Context-parallel splits and the position-stated causal mask
# ---------------------------------------------------------------------------
def test_cp_maps_worked_examples():
    """The splits the CP section prints: ring (12 tokens, 4 GPUs), striped (16
    tokens, 4 GPUs) and the zigzag block layout 0 7 1 6 2 5 3 4 (one token
    per block)."""
    n = 0
    with open(os.path.join(GOLDEN, "cp_index_maps.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, toks = line.split(":")
            mode, S, N, r = head.split()
            want = [int(t) for t in toks.split()]
            assert list(oracle.cp_tokens(int(S), int(N), mode, int(r))) == want, line
            n += 1
    assert n == 12


@pytest.mark.parametrize("mode", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("S,N", [(16, 4), (48, 4), (40, 2), (64, 8)])
def test_cp_maps_partition_and_balance(mode, S, N):
    """Every token belongs to exactly one rank, each rank's list ascends, and
    the zigzag and striped splits balance causal work as the section says
    (zigzag exactly when S % 2N == 0: sum of (t+1) equal over ranks)."""
    parts = [oracle.cp_tokens(S, N, mode, r) for r in range(N)]
    allt = np.concatenate(parts)
    assert np.array_equal(np.sort(allt), np.arange(S))
    for p_ in parts:
        assert np.all(np.diff(p_) > 0)
    work = [int(np.sum(p_ + 1)) for p_ in parts]
    if mode == "zigzag" and S % (2 * N) == 0:
        assert len(set(work)) == 1
    if mode == "striped":
        assert max(work) - min(work) <= S // N * (N - 1)
    if mode == "contiguous" and S >= 2 * N:
        assert work[-1] > work[0]          # the imbalance the section points out


def test_attention_positions_is_causal_on_the_full_sequence():
    d = synth.dense_bf16(seed=31, B=1, S=70, Hq=4, Hkv=2, D=16)
    pos = np.arange(70)
    o1, l1 = oracle.attention_positions(d["q"], d["k"], d["v"], pos, pos, d["scale"])
    o2, l2 = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def test_attention_positions_brute_force():
    """Against a full-matrix numpy softmax with the mask built from positions
    (scattered, unsorted query and key positions; one query sees no key)."""
    rng = np.random.default_rng(32)
    Sq, Sk, D = 9, 11, 8
    q = rng.standard_normal((1, Sq, 1, D))
    k = rng.standard_normal((1, Sk, 1, D))
    v = rng.standard_normal((1, Sk, 1, D))
    qp = rng.permutation(40)[:Sq]
    kp = rng.permutation(40)[:Sk]
    qp[0] = min(kp) - 1 if min(kp) > 0 else qp[0]
    o, l = oracle.attention_positions(q, k, v, qp, kp, 0.3)
    for i in range(Sq):
        vis = kp <= qp[i]
        if not vis.any():
            assert np.isnan(o[0, i, 0]).all() and l[0, 0, i] == -np.inf
            continue
        s = 0.3 * (k[0, vis, 0] @ q[0, i, 0])
        w = np.exp(s - s.max())
        assert np.allclose(o[0, i, 0], (w / w.sum()) @ v[0, vis, 0], rtol=0, atol=1e-12)
        assert abs(l[0, 0, i] - (s.max() + np.log(w.sum()))) < 1e-12


@pytest.mark.parametrize("mode", ["contiguous", "striped", "zigzag"])
def test_cp_partials_merge_to_the_causal_rows(mode):
    """Ring attention on one rank: its queries against every rank's key
    shard, merged by LSE, equal the causal attention rows of its tokens;
    and the normalised merge agrees with the unnormalised one."""
    S, N = 48, 4
    d = synth.dense_bf16(seed=33, B=1, S=S, Hq=4, Hkv=2, D=16)
    for r in range(N):
        tq = oracle.cp_tokens(S, N, mode, r)
        parts = []
        for s_ in range(N):
            tk = oracle.cp_tokens(S, N, mode, s_)
            parts.append(oracle.attention_positions(d["q"][:, tq], d["k"][:, tk], d["v"][:, tk], tq,
                                                    tk, d["scale"]))
        o, l = oracle.merge_normalized(parts)
        ref, ref_l = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True, rows=tq)
        assert np.allclose(o, ref, rtol=0, atol=1e-12) and np.allclose(l, ref_l, rtol=0, atol=1e-12)
    # one row through the unnormalised identity as well
    q0 = oracle.widen(d["q"][0, S - 1, 0])
    raw = [oracle.partial_attention(q0, d["k"][0, tk, 0], d["v"][0, tk, 0], d["scale"])
           for tk in (np.arange(0, 20), np.arange(20, 48))]
    o_u, l_u = oracle.lse_merge(raw)
    o_n, l_n = oracle.merge_normalized([(p_[2] / p_[1], p_[0] + np.log(p_[1])) for p_ in raw])
    assert np.allclose(o_u, o_n, rtol=0, atol=1e-12) and abs(l_u - l_n) < 1e-12


# ---------------------------------------------------------------------------
# FP8 (OCP e4m3) KV quantisation
# ---------------------------------------------------------------------------
from oracle import fp8  # noqa: E402


def test_fp8_decode_matches_the_format_definition():
    """Closed-form values of e4m3: bias 7, subnormals m*2^-9, max 448, one
    NaN pattern per sign, no infinities."""
    dec = fp8.fp8_e4m3_decode
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
            0x39: 1.125, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in want.items():
        assert dec([c])[0] == v, hex(c)
    assert np.isnan(dec([0x7F])[0]) and np.isnan(dec([0xFF])[0])
    assert np.signbit(dec([0x80])[0])
    finite = dec(np.arange(256, dtype=np.uint8))
    assert np.sum(np.isnan(finite)) == 2 and np.nanmax(finite) == 448.0


def test_fp8_encode_inverts_decode_and_rounds_to_nearest_even():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(fp8.fp8_e4m3_encode(fp8.fp8_e4m3_decode(codes)), codes)
    enc = lambda v: int(fp8.fp8_e4m3_encode([v])[0])
    assert enc(1.0625) == 0x38            # tie between 1 (0x38) and 1.125 (0x39): even
    assert enc(1.1875) == 0x3A            # tie between 1.125 and 1.25: even
    assert enc(1.0626) == 0x39
    assert enc(2.0 ** -10) == 0x00        # tie between 0 and the smallest subnormal
    assert enc(3 * 2.0 ** -10) == 0x02    # tie between 1 and 2 * 2^-9: even
    assert enc(464.0) == 0x7E and enc(1e6) == 0x7E and enc(-1e6) == 0xFE   # saturate
    assert enc(-1e-30) == 0x80


def test_fp8_error_bound():
    rng = np.random.default_rng(40)
    x = np.exp(rng.uniform(np.log(2.0 ** -6), np.log(448.0), 20000)) * rng.choice([-1, 1], 20000)
    y = fp8.fp8_e4m3_decode(fp8.fp8_e4m3_encode(x))
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -4)            # half an ulp, normal range
    xs = rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000)
    ys = fp8.fp8_e4m3_decode(fp8.fp8_e4m3_encode(xs))
    assert np.all(np.abs(ys - xs) <= 2.0 ** -10)                      # half a subnormal step


def test_fp8_group_quantisation():
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((50, 128)) * np.exp(rng.uniform(-8, 8, (50, 1)))).astype(np.float32)
    x[3] = 0.0
    codes, scale = fp8.quantize_groups(x)
    assert scale[3] == 0 and np.all(codes[3] == 0)
    y = fp8.dequantize_groups(codes, scale)
    amax = np.abs(x).max(axis=1)
    assert np.all(np.abs(y - x) <= 2.0 ** -4 * amax[:, None] + 1e-30)
    i = np.argmax(np.abs(x), axis=1)
    assert np.all((codes[np.arange(50), i] & 0x7F)[amax > 0] == 0x7E)      # the max maps to 448


def test_fp8_pool_groups_are_k_rows_and_v_columns():
    """K groups are token rows of a block, V groups are token columns of the
    dimension-major V block: scaling token j by 2^j scales exactly its group."""
    row = synth.bf16_bits_to_f32(synth.normal_bf16(42, (128,)))
    f = np.broadcast_to(row, (1, 64, 128)).astype(np.float32)     # the same vector per token
    tok = 2.0 ** np.arange(64, dtype=np.float32)
    kb = synth.f32_to_bf16_bits(f * tok[None, :, None])
    vb = synth.f32_to_bf16_bits(np.swapaxes(f, 1, 2) * tok[None, None, :])
    k8, v8, ks, vs = fp8.quantize_kv_pool(kb, vb)
    assert np.allclose(ks[0] / ks[0, 0], tok) and np.allclose(vs[0] / vs[0, 0], tok)
    assert np.array_equal(k8, np.swapaxes(v8, 1, 2))     # same values per token, transposed


# ---------------------------------------------------------------------------
# Paged cache read-back
# ---------------------------------------------------------------------------
def test_paged_gather_hand_example():
    """Two requests, one KV head, 64-token blocks placed at hand-chosen
    physical ids; V blocks are dimension-major."""
    D = 2
    k_pool = np.zeros((3, 64, D), np.uint16)
    v_pool = np.zeros((3, D, 64), np.uint16)
    k_pool[2, 5] = [7, 8]
    v_pool[2, :, 5] = [9, 10]
    k_pool[0, 1] = [1, 2]
    v_pool[0, :, 1] = [3, 4]
    table = np.array([[[1, 2]], [[0, -1]]], np.int32)     # b0: blocks 1,2 ; b1: block 0
    ko, vo = oracle.paged_gather(k_pool, v_pool, table, [70, 2], 70)
    assert list(ko[0, 64 + 5, 0]) == [7, 8] and list(vo[0, 69, 0]) == [9, 10]
    assert list(ko[1, 1, 0]) == [1, 2] and list(vo[1, 1, 0]) == [3, 4]


def test_paged_gather_roundtrip_decode_cache():
    c = synth.decode_cache(seed=5, B=3, ctx_lens=[1, 64, 200], Hq=4, Hkv=2, D=16)
    ko, vo = oracle.paged_gather(c["k_pool"], c["v_pool"], c["block_table"], c["ctx_len"])
    for b, n in enumerate(c["ctx_len"]):
        np.testing.assert_array_equal(ko[b, :n], c["k_seq"][b])
        np.testing.assert_array_equal(vo[b, :n], c["v_seq"][b])
    bad = c["block_table"].copy()
    bad[0, 0, 0] = 10**6
    with pytest.raises(RuntimeError):
        oracle.paged_gather(c["k_pool"], c["v_pool"], bad, c["ctx_len"])


# ---------------------------------------------------------------------------
# Decode over per-request contexts, and the dequantising gather of the FP8 cache
# ---------------------------------------------------------------------------
def _softmax_matrix_decode(q, k_seq, v_seq, ctx_len, scale, group):
    """numpy full-matrix form, head by head: softmax(scale * K q) V over the
    first ctx_len keys, KV head h // group (an independent formulation of the
    naive attention of "Flash Attention and distributed inference" §18.2)."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        n = int(ctx_len[b])
        for h in range(Hq):
            K = k_seq[b][:n, h // group]
            V = v_seq[b][:n, h // group]
            s = scale * (K @ q[b, h])
            w = np.exp(s - s.max())
            out[b, h] = (w / w.sum()) @ V
            lse[b, h] = s.max() + np.log(w.sum())
    return out, lse


def test_decode_attention_brute_force_and_closed_forms():
    """Three requests of 1, 64 and 70 keys (a partial last block), GQA 2:1:
    every one of the ctx_len keys is visible and no other (Ulysses inference
    article §2.3: the head-sharded cache holds the whole history; the new
    token's own K/V included).  Also the single-key closed form (O = V_0,
    LSE = s_0) and q = 0 -> mean of the ctx_len values."""
    rng = np.random.default_rng(90)
    Hq, Hkv, D, scale = 4, 2, 8, 0.5
    ctx = np.array([1, 64, 70])
    q = rand(rng, 3, Hq, D)
    k_seq = [rand(rng, n + 5, Hkv, D) for n in ctx]     # 5 trailing keys that must not count
    v_seq = [rand(rng, n + 5, Hkv, D) for n in ctx]
    out, lse = oracle.decode_attention(q, k_seq, v_seq, ctx, scale)
    ref, ref_lse = _softmax_matrix_decode(q, k_seq, v_seq, ctx, scale, Hq // Hkv)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)
    for h in range(Hq):                                   # ctx = 1: V_0 and its score
        np.testing.assert_allclose(out[0, h], v_seq[0][0, h // 2], rtol=0, atol=1e-15)
        assert abs(lse[0, h] - scale * q[0, h] @ k_seq[0][0, h // 2]) <= 1e-14
    z, zl = oracle.decode_attention(np.zeros_like(q), k_seq, v_seq, ctx, scale)
    for b, n in enumerate(ctx):
        for h in range(Hq):
            np.testing.assert_allclose(z[b, h], v_seq[b][:n, h // 2].mean(axis=0), atol=1e-14)
            assert abs(zl[b, h] - np.log(n)) <= 1e-13


def test_gather_dequantized_hand_example():
    """Literal values: one KV head, request 0 owns blocks 2 then 0 (a
    shuffled table), request 1 owns block 1; 70 and 3 tokens.  e4m3 codes
    0x38 = 1, 0x40 = 2, 0xB8 = -1 (the format's closed forms) times the
    token's scale.  K token t sits in row t % 64 of its block, V token t in
    column t % 64 of the dimension-major V block."""
    D = 2
    k8 = np.zeros((3, 64, D), np.uint8)
    v8 = np.zeros((3, D, 64), np.uint8)
    ks = np.zeros((3, 64), np.float32)
    vs = np.zeros((3, 64), np.float32)
    k8[2, 0] = [0x38, 0x40]; ks[2, 0] = 0.5          # request 0, token 0
    v8[2, :, 0] = [0x40, 0xB8]; vs[2, 0] = 0.25
    k8[0, 5] = [0xB8, 0x38]; ks[0, 5] = 4.0          # request 0, token 69
    v8[0, :, 5] = [0x38, 0x38]; vs[0, 5] = 3.0
    k8[1, 2] = [0x40, 0x40]; ks[1, 2] = 1.5          # request 1, token 2
    v8[1, :, 2] = [0xB8, 0x40]; vs[1, 2] = 2.0
    table = np.array([[[2, 0]], [[1, -1]]], np.int32)
    kq, vq = fp8.gather_dequantized(k8, v8, ks, vs, table, [70, 3])
    assert kq[0].shape == (70, 1, D) and kq[1].shape == (3, 1, D)
    assert list(kq[0][0, 0]) == [0.5, 1.0] and list(vq[0][0, 0]) == [0.5, -0.25]
    assert list(kq[0][69, 0]) == [-4.0, 4.0] and list(vq[0][69, 0]) == [3.0, 3.0]
    assert list(kq[1][2, 0]) == [3.0, 3.0] and list(vq[1][2, 0]) == [-2.0, 4.0]
    assert not kq[0][1:69].any() and not vq[1][:2].any()
    only1 = fp8.gather_dequantized(k8, v8, ks, vs, table, [70, 3], requests=[1])
    assert len(only1[0]) == 1 and np.array_equal(only1[0][0], kq[1])


def test_gather_dequantized_equals_paged_gather_then_dequantize():
    """On a seeded shuffled cache (partial tails, NaN-free codes, 2 KV heads):
    the dequantising gather equals the pinned paged gather of the codes
    followed by the pinned group dequantisation, token by token.  The scales
    are routed through the same gather as slot indices."""
    c = synth.decode_cache(seed=91, B=3, ctx_lens=[1, 64, 150], Hq=4, Hkv=2, D=16)
    unused = lambda pool: np.where(pool == synth.BF16_NAN_BITS, np.uint16(0), pool)
    k8, v8, ks, vs = fp8.quantize_kv_pool(unused(c["k_pool"]), unused(c["v_pool"]))
    n, D = k8.shape[0], k8.shape[2]
    kc, vc = oracle.paged_gather(k8.astype(np.uint16), v8.astype(np.uint16), c["block_table"],
                                 c["ctx_len"])
    slot = np.arange(n * 64, dtype=np.uint16).reshape(n, 64, 1)     # index of (block, slot)
    si, _ = oracle.paged_gather(slot, np.swapaxes(slot, 1, 2), c["block_table"], c["ctx_len"])
    kq, vq = fp8.gather_dequantized(k8, v8, ks, vs, c["block_table"], c["ctx_len"])
    for b, T in enumerate(c["ctx_len"]):
        idx = si[b, :T, :, 0].astype(np.int64)                       # [T][Hkv]
        k_ref = fp8.fp8_e4m3_decode(kc[b, :T]) * ks.reshape(-1)[idx][..., None]
        v_ref = fp8.fp8_e4m3_decode(vc[b, :T]) * vs.reshape(-1)[idx][..., None]
        np.testing.assert_array_equal(kq[b], k_ref)
        np.testing.assert_array_equal(vq[b], v_ref)
    # and the values are the quantised versions of the tokens placed there
    for b, T in enumerate(c["ctx_len"]):
        x = synth.bf16_bits_to_f32(c["k_seq"][b]).astype(np.float64)
        assert np.all(np.abs(kq[b] - x) <= 2.0 ** -4 * np.abs(x).max(axis=-1, keepdims=True))


# ---------------------------------------------------------------------------
# FP8 scores for prefill: power-of-two block scales (reading in oracle/fp8.py)
# ---------------------------------------------------------------------------
def _block(v, *rest):
    b = np.zeros(32)
    b[0] = v
    b[1:1 + len(rest)] = rest
    return b


def test_fp8_block_exponent_closed_forms():
    """e is the smallest integer with amax <= 448 * 2^e: 448 -> 0, 449 -> 1,
    224 -> -1, 224.5 -> 0, 1 -> -8 (1.75 >= 1 > 0.875), 2^-130 -> clamped to
    -127, zeros -> -127."""
    x = np.stack([_block(448.0), _block(449.0), _block(-224.0), _block(224.5), _block(1.0, -0.5),
                  _block(2.0 ** -130), np.zeros(32)])
    assert fp8.block_exponents(x).ravel().tolist() == [0, 1, -1, 0, -8, -127, -127]
    assert fp8.e8m0_bytes([0, -8, -127, 127]).tolist() == [127, 119, 0, 254]


def test_fp8_block_quantisation_values():
    """Codes of a block follow x / 2^e through the e4m3 table: with amax 1,
    e = -8 and 1 -> 256 (0x78), -0.5 -> -128 (0xF0), 2^-8 -> 1 (0x38),
    3 * 2^-10 -> 0.75 = 1.5 * 2^-1 (0x34); a 448 block keeps 448 -> 0x7E."""
    codes, e = fp8.quantize_blocks(np.stack([_block(1.0, -0.5, 2.0 ** -8, 3 * 2.0 ** -10),
                                             _block(448.0, 1.0)]))
    assert e.tolist() == [[-8], [0]]
    assert codes[0, :4].tolist() == [0x78, 0xF0, 0x38, 0x34]
    assert codes[1, :2].tolist() == [0x7E, 0x38]
    assert not codes[0, 4:].any()


def test_fp8_block_quantisation_invariance_and_error_bound():
    """Scaling a block by 2^j keeps its codes and moves e by j; every value is
    within half an e4m3 step: 2^-4 |x| in the normal range, 2^-10 * 2^e below."""
    rng = np.random.default_rng(95)
    x = (rng.standard_normal((40, 128)) * np.exp(rng.uniform(-20, 20, (40, 1)))).astype(np.float32)
    c, e = fp8.quantize_blocks(x)
    for j in (-5, 3, 17):
        c2, e2 = fp8.quantize_blocks((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c2, c) and np.array_equal(e2, e + j)
    y = fp8.dequantize_blocks(c, e)
    step = np.repeat(np.exp2(e.astype(np.float64)), 32, axis=-1)
    xd = x.astype(np.float64)
    normal = np.abs(xd) >= 2.0 ** -6 * step
    assert np.all(np.abs(y - xd)[normal] <= 2.0 ** -4 * np.abs(xd)[normal])
    assert np.all(np.abs(y - xd)[~normal] <= 2.0 ** -10 * step[~normal])
    # the block maximum keeps full range: it lands in (224, 448] before rounding
    blk = np.abs(xd).reshape(40, 4, 32).max(-1) / np.exp2(e)
    assert np.all((blk > 224) & (blk <= 448))


def test_attention_fp8_closed_forms():
    """Base-2 softmax of the dequantised scores: one key gives O = V_0 and
    LSE = ln2 * (q''.k''); two keys give weights 1 / (1 + 2^(s1 - s0))."""
    rng = np.random.default_rng(96)
    q = synth.normal_bf16(97, (1, 1, 1, 64))
    k = synth.normal_bf16(98, (1, 2, 1, 64))
    v = synth.normal_bf16(99, (1, 2, 1, 64))
    qd, kd = fp8.prefill_fp8_operands(q, k, 0.125)
    s = kd[0, :, 0] @ qd[0, 0, 0]                                     # log2 units
    o1, l1 = fp8.attention_fp8(q, k[:, :1], v[:, :1], 0.125)
    np.testing.assert_allclose(o1[0, 0, 0], oracle.widen(v)[0, 0, 0], rtol=0, atol=1e-15)
    assert abs(l1[0, 0, 0] - np.log(2) * s[0]) <= 1e-12
    o2, l2 = fp8.attention_fp8(q, k, v, 0.125)
    w0 = 1.0 / (1.0 + 2.0 ** (s[1] - s[0]))
    vv = oracle.widen(v)[0, :, 0]
    np.testing.assert_allclose(o2[0, 0, 0], w0 * vv[0] + (1 - w0) * vv[1], rtol=1e-12, atol=1e-13)
    assert rng is not None


def test_fp8_operands_are_the_scaled_query_and_the_key():
    """Q'' is q * scale * log2(e) and K'' is k, each within half an e4m3 step
    of its block (2^-4 relative in the normal range)."""
    d = synth.dense_bf16(seed=101, B=1, S=64, Hq=2, Hkv=1, D=128)
    qd, kd = fp8.prefill_fp8_operands(d["q"], d["k"], d["scale"])
    q = oracle.widen(d["q"]) * d["scale"] * np.log2(np.e)
    k = oracle.widen(d["k"])
    for got, want in ((qd, q), (kd, k)):
        blk = np.abs(want).reshape(*want.shape[:-1], 4, 32).max(-1, keepdims=True)
        tol = np.maximum(2.0 ** -4 * np.abs(want), 2.0 ** -10 * blk.repeat(32, -1).reshape(want.shape) / 224)
        assert np.all(np.abs(got - want) <= tol * (1 + 1e-6))


def test_attention_fp8_close_to_exact_attention():
    """With the dequantised operands fixed (pinned above), each row's weights
    differ from the exact softmax weights by at most a factor e^(2 Delta),
    Delta = ln2 * max_j |s''_j - s_j| (log2-unit scores), so
    |O_fp8 - O| <= (e^(2 Delta) - 1) max|v|; checked on 128 causal rows."""
    d = synth.dense_bf16(seed=100, B=1, S=128, Hq=2, Hkv=1, D=128)
    o8, _ = fp8.attention_fp8(d["q"], d["k"], d["v"], d["scale"], causal=True)
    o, _ = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True)
    qd, kd = fp8.prefill_fp8_operands(d["q"], d["k"], d["scale"])
    s8 = np.einsum("ihd,jd->ihj", qd[0], kd[0, :, 0])
    s = np.einsum("ihd,jd->ihj", oracle.widen(d["q"])[0], oracle.widen(d["k"])[0, :, 0]) \
        * d["scale"] * np.log2(np.e)
    vmax = np.abs(oracle.widen(d["v"])).max()
    for i in range(128):
        delta = np.log(2) * np.abs(s8[i, :, :i + 1] - s[i, :, :i + 1]).max()
        assert np.abs(o8[0, i] - o[0, i]).max() <= (np.exp(2 * delta) - 1) * vmax + 1e-12
    assert np.abs(o8 - o).max() > 0          # the quantisation is not a no-op


def test_fp8_v_blocks_run_along_keys():
    """V'' quantises each (dim, 32-key block): scaling one dimension of the keys
    of one block by 2^j scales exactly those values by 2^j; a block of keys
    is quantised independently of its neighbours (a huge value in keys 0..31
    leaves keys 32..63 untouched); a ragged tail is a block of its own."""
    rng = np.random.default_rng(102)
    v = rng.standard_normal((1, 70, 1, 64)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(v)
    base = fp8.dequantized_v_keys(bits)
    w = synth.bf16_bits_to_f32(bits).copy()
    w[0, 32:64, 0, 5] *= np.float32(8.0)
    got = fp8.dequantized_v_keys(synth.f32_to_bf16_bits(w))
    np.testing.assert_array_equal(got[0, 32:64, 0, 5], 8 * base[0, 32:64, 0, 5])
    mask = np.ones_like(got, bool)
    mask[0, 32:64, 0, 5] = False
    np.testing.assert_array_equal(got[mask], base[mask])
    w2 = synth.bf16_bits_to_f32(bits).copy()
    w2[0, 3, 0, :] = 1e6
    got2 = fp8.dequantized_v_keys(synth.f32_to_bf16_bits(w2))
    np.testing.assert_array_equal(got2[0, 32:], base[0, 32:])
    assert not np.array_equal(got2[0, :32], base[0, :32])
    # keys 64..69 form their own block: quantised with their own maximum
    tail = synth.bf16_bits_to_f32(bits)[0, 64:, 0, :].astype(np.float64)
    c, e = fp8.quantize_blocks(np.concatenate([tail, np.zeros((26, 64))]).T.astype(np.float32))
    np.testing.assert_array_equal(base[0, 64:, 0, :], fp8.dequantize_blocks(c, e).T[:6])
    v2 = synth.bf16_bits_to_f32(bits).astype(np.float64)
    assert np.all(np.abs(base - v2) <= 2.0 ** -4 * np.abs(v2) + 2.0 ** -10 * np.abs(v2).max())


def test_attention_fp8_pv_uses_the_key_blocked_v():
    """attention_fp8_pv = attention_fp8 with V'' in place of V (one-key row:
    O = V''_0)."""
    d = synth.dense_bf16(seed=103, B=1, S=40, Hq=2, Hkv=1, D=64)
    o, _ = fp8.attention_fp8_pv(d["q"], d["k"], d["v"], d["scale"], causal=True)
    vdd = fp8.dequantized_v_keys(d["v"])
    np.testing.assert_allclose(o[0, 0, :, :], np.broadcast_to(vdd[0, 0, 0], (2, 64)), atol=1e-15)
    o8, _ = fp8.attention_fp8(d["q"], d["k"], d["v"], d["scale"], causal=True)
    assert 0 < np.abs(o - o8).max() < 0.2


def test_hadamard_matrix_and_transform():
    """The rotation of incoherent processing: hadamard_matrix is Sylvester's
    (scipy.linalg.hadamard), H H^T = 128 I; hadamard_rotate(x, s) equals
    (s * x) H exactly for small-integer rows (exact in fp32) with random
    signs, and maps e_i to s_i times row i of H."""
    import scipy.linalg
    H = fp8.hadamard_matrix()
    Hs = scipy.linalg.hadamard(128)
    np.testing.assert_array_equal(H, Hs)
    np.testing.assert_array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    s = synth.hadamard_signs(110)
    assert s.dtype == np.int8 and set(np.unique(s).tolist()) == {-1, 1}
    x = np.random.default_rng(110).integers(-64, 65, (5, 128)).astype(np.float32)
    np.testing.assert_array_equal(fp8.hadamard_rotate(x, s).astype(np.float64),
                                  (x.astype(np.float64) * s) @ Hs)
    for i in (0, 1, 77, 127):
        e = np.zeros(128, np.float32)
        e[i] = 1
        np.testing.assert_array_equal(fp8.hadamard_rotate(e, s), s[i] * Hs[i])
    with pytest.raises(ValueError):
        fp8.hadamard_rotate(x, np.ones(128) * 2)


def test_rotated_fp8_operands():
    """With signs, Q'' is (q M) * c / 128 and K'' is k M (M = diag(s) H, the
    rotation computed independently in fp64 here), each within half an e4m3
    step of its block; and (q M).(k M) = 128 q.k, so the scores are kept."""
    import scipy.linalg
    d = synth.dense_bf16_outliers(seed=111, B=1, S=64, Hq=2, Hkv=1)
    s = synth.hadamard_signs(111)
    M = np.diag(s.astype(np.float64)) @ scipy.linalg.hadamard(128)
    qd, kd = fp8.prefill_fp8_operands(d["q"], d["k"], d["scale"], signs=s)
    c = float(fp8.query_multiplier(d["scale"]))
    q, k = oracle.widen(d["q"]), oracle.widen(d["k"])
    qm, km = q @ M * (c / 128), k @ M
    for got, want in ((qd, qm), (kd, km)):
        blk = np.abs(want).reshape(*want.shape[:-1], 4, 32).max(-1, keepdims=True)
        tol = np.maximum(2.0 ** -4 * np.abs(want), 2.0 ** -10 * blk.repeat(32, -1).reshape(want.shape) / 224)
        assert np.all(np.abs(got - want) <= tol * (1 + 1e-5) + 1e-6 * blk.repeat(32, -1).reshape(want.shape))
    np.testing.assert_allclose(np.einsum("bshd,bthd->bsht", q @ M, k @ M),
                               128 * np.einsum("bshd,bthd->bsht", q, k), rtol=1e-9, atol=1e-9)


def test_rotation_lowers_fp8_error_on_outlier_channels():
    """What incoherent processing is for: on inputs whose Q and K carry a
    few outlier channels, the FP8-score attention with the rotation is at
    least 1.6 times closer to exact attention (relative L2) than without it;
    on N(0, 1) inputs the two errors are within 10% of each other."""
    s = synth.hadamard_signs(112)
    def err(d, signs):
        o, _ = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True)
        o8, _ = fp8.attention_fp8(d["q"], d["k"], d["v"], d["scale"], causal=True, signs=signs)
        return np.linalg.norm(o8 - o) / np.linalg.norm(o)
    d = synth.dense_bf16_outliers(seed=112, B=1, S=256, Hq=2, Hkv=1)
    assert err(d, None) > 1.6 * err(d, s)
    d0 = synth.dense_bf16(seed=112, B=1, S=256, Hq=2, Hkv=1, D=128)
    assert abs(err(d0, None) / err(d0, s) - 1) < 0.1
