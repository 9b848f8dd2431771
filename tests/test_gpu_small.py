"""GPU parity at small sizes: every kernel against the fp64 oracle.

Shapes span several tiles and ragged tails; every output element is compared.
All calls go through the C ABI of libattn (via the thin binding).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import BF16_ATOL, assert_attention_close, bits, log, to_dev, to_np64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lcat = pytest.importorskip("long_context_attention_tiled_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lcat.load_library()


# ---------------------------------------------------------------------------
# seq -> head relayout (bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("SP,S_loc,H,D,dtype", [
    (4, 16, 8, 128, np.uint16),      # the article's worked example, bf16 payload
    (4, 37, 64, 128, np.uint16),     # 64 global heads, ragged token count
    (2, 5, 4, 3, np.uint8),          # odd run length -> element path
    (4, 9, 8, 6, np.float64),
    (8, 3, 16, 4, np.int32),
])
def test_permute_bit_exact(SP, S_loc, H, D, dtype):
    log(f"permute SP={SP} S_loc={S_loc} H={H} D={D} {np.dtype(dtype).name}")
    rng = np.random.default_rng(100 + SP + S_loc)
    if np.dtype(dtype).kind == "f":
        x = rng.standard_normal((SP, S_loc, H, D)).astype(dtype)
    else:
        x = rng.integers(0, np.iinfo(dtype).max, size=(SP, S_loc, H, D), dtype=dtype)
    xd = torch.from_numpy(x).cuda()
    for r in range(SP):
        out = lcat.seq_to_head_permute(xd, r)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), oracle.permute(x, r))


@pytest.mark.parametrize("SP,S_loc,H,D,dtype", [
    (4, 16, 8, 128, np.uint16),      # the article's worked example, bf16 payload
    (4, 37, 64, 128, np.uint16),     # 64 global heads, ragged token count
    (2, 5, 4, 3, np.uint8),          # odd run length -> element path
    (4, 9, 8, 6, np.float64),
    (8, 3, 16, 4, np.int32),
])
def test_unpermute_bit_exact(SP, S_loc, H, D, dtype):
    """head -> sequence relayout of every rank into one pre-filled buffer:
    after each call the buffer equals the oracle's, so the other ranks'
    slices are untouched, and after all ranks it is the full output."""
    log(f"unpermute SP={SP} S_loc={S_loc} H={H} D={D} {np.dtype(dtype).name}")
    rng = np.random.default_rng(200 + SP + S_loc)
    draw = ((lambda shape: rng.standard_normal(shape).astype(dtype)) if np.dtype(dtype).kind == "f"
            else (lambda shape: rng.integers(0, np.iinfo(dtype).max, size=shape, dtype=dtype)))
    ref = draw((SP, S_loc, H, D))                 # arbitrary prior contents
    outd = torch.from_numpy(ref.copy()).cuda()
    for r in range(SP):
        x = draw((SP * S_loc, H // SP, D))
        lcat.head_to_seq_permute(torch.from_numpy(x).cuda(), SP, H, r, out=outd)
        torch.cuda.synchronize()
        oracle.unpermute(x, SP, H, r, out=ref)
        np.testing.assert_array_equal(outd.cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def _rope_ref_bits_close(got_bits, ref):
    """GPU bf16 vs fp64 reference: within one bf16 ulp plus the fp32 rotation
    error (about 1e-7 absolute, which dominates only where the two rotation
    terms cancel), and the correctly rounded value for (almost) every element."""
    got = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    err = np.abs(got - ref)
    bound = np.abs(ref) * 2.0 ** -7 + 1e-6
    assert np.all(err <= bound), f"max excess {np.max(err - bound):.3g}"
    exact = synth.f32_to_bf16_bits(ref.astype(np.float32))
    frac = np.mean(got_bits == exact)
    assert frac > 0.99, f"only {frac:.4f} correctly rounded"


@pytest.mark.parametrize("SP,S_loc,Hq,Hkv,D,dtype", [(4, 37, 64, 8, 128, np.uint16),
                                                     (2, 5, 4, 2, 3, np.uint16),
                                                     (8, 3, 16, 8, 4, np.float64)])
def test_permute_qkv_bit_exact(SP, S_loc, Hq, Hkv, D, dtype):
    """Q, K and V relayout in one launch equals three oracle relayouts; the
    second and third shapes are not 16-byte runs (element path)."""
    rng = np.random.default_rng(SP * 100 + S_loc)
    mk = lambda H: rng.integers(0, 2 ** 16, size=(SP, S_loc, H, D)).astype(dtype)
    qs, ks, vs = mk(Hq), mk(Hkv), mk(Hkv)
    for rank in (0, SP - 1):
        qo, ko, vo = lcat.seq_to_head_permute_qkv(to_dev(qs), to_dev(ks), to_dev(vs), rank)
        torch.cuda.synchronize()
        for got, x in ((qo, qs), (ko, ks), (vo, vs)):
            g = bits(got) if got.dtype == torch.bfloat16 else got.cpu().numpy()
            assert np.array_equal(g, oracle.permute(x, rank))


@pytest.mark.parametrize("SP,S_loc,Hq,Hkv,D", [(4, 37, 64, 8, 128), (2, 5, 4, 2, 16),
                                             (8, 3, 16, 8, 256), (1, 700, 16, 2, 128),
                                             (4, 33, 4, 4, 64)])
def test_permute_qkv_rope(SP, S_loc, Hq, Hkv, D):
    """Relayout + RoPE in one pass: Q and K against the oracle's rotation of
    the oracle's relayout, V bit for bit against the relayout; and the whole
    output bit for bit equal to the two-step path (relayout, then RoPE)."""
    log(f"permute+rope SP={SP} S_loc={S_loc} Hq={Hq} Hkv={Hkv} D={D}")
    seed = 300 + SP * 10 + S_loc
    qs = synth.normal_bf16(seed, (SP, S_loc, Hq, D))
    ks = synth.normal_bf16(seed + 1, (SP, S_loc, Hkv, D))
    vs = synth.normal_bf16(seed + 2, (SP, S_loc, Hkv, D))
    pos = np.random.default_rng(seed).integers(0, 2 ** 17, SP * S_loc).astype(np.int32)
    posd = to_dev(pos)
    for rank in (0, SP - 1):
        qo, ko, vo = lcat.seq_to_head_permute_qkv_rope(to_dev(qs), to_dev(ks), to_dev(vs), rank,
                                                       posd)
        q2, k2, v2 = lcat.seq_to_head_permute_qkv(to_dev(qs), to_dev(ks), to_dev(vs), rank)
        lcat.rope_apply(q2, posd)
        lcat.rope_apply(k2, posd)
        torch.cuda.synchronize()
        _rope_ref_bits_close(bits(qo), oracle.rope(oracle.permute(qs, rank), pos))
        _rope_ref_bits_close(bits(ko), oracle.rope(oracle.permute(ks, rank), pos))
        assert np.array_equal(bits(vo), oracle.permute(vs, rank))
        for a, b in ((qo, q2), (ko, k2), (vo, v2)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_rope_matches_oracle_large_positions():
    S, H, D = 1000, 16, 128
    log("rope S=1000 H=16 positions up to 131k")
    x = synth.normal_bf16(200, (S, H, D))
    pos = (np.arange(S, dtype=np.int64) * 131).astype(np.int32)
    xd = to_dev(x)
    lcat.rope_apply(xd, to_dev(pos))
    torch.cuda.synchronize()
    _rope_ref_bits_close(bits(xd), oracle.rope(x, pos))


def test_rope_local_positions_fail_negative_control():
    """Local positions (0..S_loc-1 on every shard) must NOT reproduce the
    global-position result beyond the first shard (the article's §5.3 bug)."""
    S_loc, H, D = 64, 2, 128
    x = synth.normal_bf16(201, (2 * S_loc, H, D))
    glob = np.arange(2 * S_loc, dtype=np.int32)
    loc = np.concatenate([np.arange(S_loc), np.arange(S_loc)]).astype(np.int32)
    a, b = to_dev(x), to_dev(x)
    lcat.rope_apply(a, to_dev(glob))
    lcat.rope_apply(b, to_dev(loc))
    torch.cuda.synchronize()
    assert torch.equal(a[:S_loc], b[:S_loc])
    assert (a[S_loc:].float() - b[S_loc:].float()).abs().max().item() > 0.1


def test_rope_commutes_with_relayout():
    """RoPE on each shard with its global positions, then the relayout, equals
    the relayout then RoPE at positions 0..S-1 (bit for bit)."""
    SP, S_loc, H, D = 4, 48, 16, 128
    x = synth.normal_bf16(202, (SP, S_loc, H, D))
    shard_pos = (np.arange(SP)[:, None] * S_loc + np.arange(S_loc)[None]).astype(np.int32)
    for r in range(SP):
        a = to_dev(x)
        for k_ in range(SP):
            lcat.rope_apply(a[k_], to_dev(shard_pos[k_]))
        pa = lcat.seq_to_head_permute(a, r)
        pb = lcat.seq_to_head_permute(to_dev(x), r)
        lcat.rope_apply(pb, to_dev(np.arange(SP * S_loc, dtype=np.int32)))
        torch.cuda.synchronize()
        assert torch.equal(pa, pb)


@pytest.mark.parametrize("S,Hq,Hkv,D", [(1, 16, 2, 128), (300, 16, 2, 128), (4099, 16, 2, 128),
                                         (77, 8, 8, 64), (130, 32, 1, 256)])
def test_rope_apply_qk_equals_two_calls(S, Hq, Hkv, D):
    """Q and K rotated in one launch equal rope_apply on each tensor bit for
    bit, and Q matches the oracle; positions reach 2^17 and are not
    consecutive."""
    q = synth.normal_bf16(230 + S, (S, Hq, D))
    k = synth.normal_bf16(231 + S, (S, Hkv, D))
    pos = np.random.default_rng(232 + S).integers(0, 1 << 17, S).astype(np.int32)
    qa, ka, pd = to_dev(q), to_dev(k), to_dev(pos)
    lcat.rope_apply_qk(qa, ka, pd)
    qb, kb = to_dev(q), to_dev(k)
    lcat.rope_apply(qb, pd)
    lcat.rope_apply(kb, pd)
    torch.cuda.synchronize()
    assert torch.equal(qa, qb) and torch.equal(ka, kb)
    _rope_ref_bits_close(bits(qa), oracle.rope(q, pos))
    _rope_ref_bits_close(bits(ka), oracle.rope(k, pos))


# ---------------------------------------------------------------------------
# fp32 exact path
# ---------------------------------------------------------------------------
def test_tiny_exact_fp32_config():
    """1 x 1 x 256 x 64 fp32, non-causal, scale 1/8: max abs error <= 1e-3
    over every output (the article's §3.5 alignment threshold)."""
    c = synth.tiny_exact()
    log("fp32 tiny exact 256x64")
    o, lse = lcat.attn_prefill(to_dev(c["q"]), to_dev(c["k"]), to_dev(c["v"]), causal=False,
                               scale=c["scale"])
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(c["q"], c["k"], c["v"], c["scale"])
    err = np.abs(to_np64(o) - ref).max()
    log(f"  max abs err {err:.3g}")
    assert err <= 1e-3
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-3


@pytest.mark.parametrize("S,Hq,Hkv,D,causal", [(200, 4, 2, 128, True), (130, 2, 1, 64, True),
                                              (65, 3, 3, 128, False)])
def test_fp32_ragged(S, Hq, Hkv, D, causal):
    rng = np.random.default_rng(300 + S)
    q = rng.standard_normal((2, S, Hq, D)).astype(np.float32)
    k = rng.standard_normal((2, S, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((2, S, Hkv, D)).astype(np.float32)
    scale = D ** -0.5
    o, lse = lcat.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, scale, causal=causal)
    assert np.abs(to_np64(o) - ref).max() <= 1e-3
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-3


# ---------------------------------------------------------------------------
# bf16 MFMA prefill
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S,Hq,Hkv,causal", [
    (1, 16, 2, True), (63, 16, 2, True), (64, 16, 2, True), (65, 16, 2, True),
    (300, 16, 2, True), (300, 16, 2, False), (200, 2, 2, True), (200, 4, 2, True),
    (200, 8, 2, False), (257, 32, 2, True), (129, 16, 16, True),
])
def test_prefill_bf16_all_rows(S, Hq, Hkv, causal):
    log(f"prefill bf16 S={S} Hq={Hq} Hkv={Hkv} causal={causal}")
    d = synth.dense_bf16(seed=400 + S + Hq, B=2, S=S, Hq=Hq, Hkv=Hkv)
    o, lse = lcat.attn_prefill(to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"]), causal=causal)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=causal)
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="prefill")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")


def test_prefill_needle():
    """One key per query row is planted as a large multiple of that row's
    query: the output must be (close to) that key's value row."""
    S, Hq, Hkv = 256, 16, 2
    rng = np.random.default_rng(501)
    q = rng.standard_normal((1, S, Hq, 128)).astype(np.float32)
    q[:, :, 1:] = q[:, :, :1]           # all heads of a group share the query
    k = rng.standard_normal((1, S, Hkv, 128)).astype(np.float32) * 0.1
    v = rng.standard_normal((1, S, Hkv, 128)).astype(np.float32)
    rows = np.arange(100, S)
    needle = rows - 60                  # one distinct earlier key per row
    for g in range(Hkv):
        k[0, needle, g] = 4.0 * q[0, rows, 0]
    qb, kb, vb = (synth.f32_to_bf16_bits(a) for a in (q, k, v))
    o, _ = lcat.attn_prefill(to_dev(qb), to_dev(kb), to_dev(vb), causal=True)
    torch.cuda.synchronize()
    got = to_np64(o)[0, rows]
    want = synth.bf16_bits_to_f32(vb)[0, needle].astype(np.float64)
    for h in range(Hq):
        assert np.abs(got[:, h] - want[:, h // (Hq // Hkv)]).max() < 0.05


def test_prefill_closed_forms():
    """Closed forms on the kernel itself (no oracle): q = 0 makes every score
    0, so causal row i returns the mean of V[0..i] with LSE = ln(i+1); causal
    row 0 returns V[0] exactly whatever q is; a single key returns V[0] with
    LSE = scale * q.k0."""
    S, Hq, Hkv = 300, 16, 2
    g = Hq // Hkv
    d = synth.dense_bf16(seed=950, B=1, S=S, Hq=Hq, Hkv=Hkv)
    v64 = synth.bf16_bits_to_f32(d["v"]).astype(np.float64)[0]          # [S][Hkv][D]
    mean = np.cumsum(v64, axis=0) / np.arange(1, S + 1)[:, None, None]
    zero_q = np.zeros_like(d["q"])
    o, lse = lcat.attn_prefill(to_dev(zero_q), to_dev(d["k"]), to_dev(d["v"]), causal=True)
    torch.cuda.synchronize()
    want = np.repeat(mean, g, axis=1)[None]                                # [1][S][Hq][D]
    want_lse = np.broadcast_to(np.log(np.arange(1, S + 1))[None, None, :], (1, Hq, S))
    assert_attention_close(to_np64(o), want, lse.cpu().numpy(), want_lse, what="q = 0")
    # causal row 0 sees only key 0: P = 1 exactly, so O is V[0] bit for bit
    o, _ = lcat.attn_prefill(to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"]), causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o)[0, 0], np.repeat(d["v"][0, 0], g, axis=0))
    # a single key
    d1 = synth.dense_bf16(seed=951, B=2, S=1, Hq=Hq, Hkv=Hkv)
    o, lse = lcat.attn_prefill(to_dev(d1["q"]), to_dev(d1["k"]), to_dev(d1["v"]), causal=False)
    torch.cuda.synchronize()
    q64, k64 = (synth.bf16_bits_to_f32(d1[n]).astype(np.float64) for n in ("q", "k"))
    s0 = np.einsum("bhd,bhd->bh", q64[:, 0], np.repeat(k64[:, 0], g, axis=1)) * d1["scale"]
    assert np.array_equal(bits(o)[:, 0], np.repeat(d1["v"][:, 0], g, axis=1))
    assert_attention_close(to_np64(o), np.repeat(synth.bf16_bits_to_f32(d1["v"]).astype(np.float64),
                                                 g, axis=2), lse.cpu().numpy(), s0[:, :, None],
                           what="single key")


def test_prefill_deterministic():
    d = synth.dense_bf16(seed=502, B=1, S=500, Hq=16, Hkv=2)
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    o1, l1 = lcat.attn_prefill(q, k, v)
    o2, l2 = lcat.attn_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)



def _stepped_scores(seed, B, S, Hq, Hkv, step_keys, step=13.0, D=128):
    """bf16 inputs whose scaled scores climb by about `step` (natural-log
    units, i.e. ~18.8 in log2 units) every `step_keys` keys: every query row
    shares one direction u (plus 10% noise) and key t is the multiple of u
    that puts it on its level, plus N(0, 0.3^2) noise.  The running maximum
    of a row then jumps far past any lazy-rescale bound deep inside the key
    loop, not only in its first or last tile; with steps every 128 keys the
    total climb passes 2^128, so exponentials taken against a stale maximum
    would overflow fp32."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D)
    scale = 1.0 / np.sqrt(D)
    q = u + 0.1 * rng.standard_normal((B, S, Hq, D))
    coef = step * (np.arange(S) // step_keys) / (scale * (u @ u))
    k = coef[None, :, None, None] * u + 0.3 * rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    q, k, v = (synth.f32_to_bf16_bits(a.astype(np.float32)) for a in (q, k, v))
    return dict(q=q, k=k, v=v, scale=scale)


@pytest.mark.parametrize("S,B,Hq,Hkv,causal,stepped", [
    (2048, 1, 16, 2, True, False), (1100, 2, 16, 2, False, False), (2048, 1, 16, 2, True, True),
    (1100, 2, 16, 2, False, True), (1500, 1, 8, 2, True, False), (1300, 1, 4, 4, True, True),
])
def test_prefill_bf16_long_rows(S, B, Hq, Hkv, causal, stepped):
    """Sequences long enough for the interleaved key loop (five or more
    full tiles before the diagonal), every row against the oracle; the
    stepped inputs make that loop take its exact-maximum recovery path."""
    log(f"prefill bf16 long S={S} B={B} Hq={Hq} Hkv={Hkv} causal={causal} stepped={stepped}")
    d = (_stepped_scores(800 + S, B, S, Hq, Hkv, step_keys=128) if stepped
         else synth.dense_bf16(seed=800 + S, B=B, S=S, Hq=Hq, Hkv=Hkv))
    o, lse = lcat.attn_prefill(to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"]), causal=causal)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=causal)
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="prefill")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")

@pytest.mark.parametrize("S,B,Hq,Hkv", [
    (4096, 1, 16, 2), (4096, 2, 16, 2), (8192, 1, 8, 1), (5000, 1, 16, 2), (4096, 3, 16, 2),
])
def test_causal_work_order_covers_every_row(S, B, Hq, Hkv):
    """Causal prefill hands its work items (query block x batch x KV head) to
    workgroups in an XCD-aware order: generations of 32 consecutive query
    blocks per XCD, the XCDs of one KV head alternating direction between
    generations.  The shapes take 1 and 2 whole generations with 2, 4 and 8
    XCDs per KV head, a partial last generation, and a batch x head count
    that does not divide 8 (plain order).  The order must be a bijection:
    with outputs pre-filled with NaN, all three prefill kernels write every
    row of every head; bf16 rows are checked against the oracle, and the
    FP8 outputs must stay close to the bf16 ones."""
    log(f"work order S={S} B={B} Hq={Hq} Hkv={Hkv}")
    d = synth.dense_bf16(seed=600 + S + B, B=B, S=S, Hq=Hq, Hkv=Hkv)
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    k8, ks = lcat.attn_quantize_fp8_blocks(k)
    v8t, vs = lcat.attn_quantize_fp8_v(v)
    runs = {
        "bf16": lambda o, l: lcat.attn_prefill(q, k, v, causal=True, o=o, lse=l),
        "fp8": lambda o, l: lcat.attn_prefill_fp8(q, k8, ks, v, causal=True, scale=d["scale"],
                                                  o=o, lse=l),
        "fp8_pv": lambda o, l: lcat.attn_prefill_fp8_pv(q, k8, ks, v8t, vs, causal=True,
                                                        scale=d["scale"], o=o, lse=l),
    }
    outs = {}
    for name, run in runs.items():
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, S), float("nan"), device=q.device)
        run(o, lse)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any().item(), f"{name}: output rows left unwritten"
        assert not torch.isnan(lse).any().item(), f"{name}: LSE entries left unwritten"
        outs[name] = o.float()
    rows = synth.sample_rows(601, S, 96, [0, 31, 32, S // 2, S - 1])
    ref, ref_lse = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    o16, l16 = runs["bf16"](None, None)
    torch.cuda.synchronize()
    assert_attention_close(to_np64(o16[:, sel]), ref, l16[:, :, sel].cpu().numpy(), ref_lse,
                           what="work order")
    for name in ("fp8", "fp8_pv"):
        rel = (torch.linalg.vector_norm(outs[name] - outs["bf16"]) /
               torch.linalg.vector_norm(outs["bf16"])).item()
        log(f"  {name}: rel-L2 against bf16 {rel:.3g}")
        assert rel < 0.1, (name, rel)


# ---------------------------------------------------------------------------
# decode over the paged cache
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("split", [64, 128, 0])
def test_decode_all_rows(split):
    ctx = [1, 2, 63, 64, 65, 127, 128, 1000, 3001]
    log(f"decode ctx={ctx} split={split}")
    c = synth.decode_cache(seed=600, B=len(ctx), ctx_lens=ctx, Hq=16, Hkv=2, kv_head_base=2,
                           extra_blocks=5)
    dev_status = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, lse = lcat.attn_decode(to_dev(c["q"]), to_dev(c["k_pool"]), to_dev(c["v_pool"]),
                              to_dev(c["block_head"]), to_dev(c["block_table"]),
                              to_dev(c["ctx_len"]), kv_head_base=2, split_tokens=split,
                              dev_status=dev_status)
    torch.cuda.synchronize()
    assert dev_status.item() == 0
    ref, ref_lse = oracle.decode_attention(c["q"], c["k_seq"], c["v_seq"], c["ctx_len"], c["scale"])
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="decode")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")


@pytest.mark.parametrize("ctx,pieces", [
    ([8192] * 4, 256),                      # W = 1024 units: 256 waves, 4 units each
    ([8192] * 8 + [4096], 512),             # W = 2176: 512 waves
    ([8192] * 12 + [1000], 768),            # W = 3104: 768 waves (the launch)
    ([8192] * 7 + [65, 1, 0, 9000], 512),   # ragged tails and an empty request in the mix
])
def test_decode_piece_count_regimes(ctx, pieces):
    """The equal-share split cuts the W = sum(Hkv * blocks) units into
    256 * floor(W / 1024) pieces, clamped to [256, 768]; each regime
    against the oracle (every row) and against fixed 256-key splits."""
    W = sum(2 * ((c + 63) // 64) for c in ctx)
    assert min(768, max(256, (W // 1024) * 256)) == pieces
    log(f"decode pieces={pieces} W={W} ctx={ctx}")
    c = synth.decode_cache(seed=605, B=len(ctx), ctx_lens=ctx, Hq=16, Hkv=2, extra_blocks=1)
    args = [to_dev(c[k]) for k in ("q", "k_pool", "v_pool", "block_head", "block_table", "ctx_len")]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, lse = lcat.attn_decode(*args, dev_status=st)
    of, lf = lcat.attn_decode(*args, split_tokens=256)
    torch.cuda.synchronize()
    assert st.item() == 0
    nz = [i for i, n in enumerate(ctx) if n > 0]
    ref, ref_lse = oracle.decode_attention(c["q"][nz], [c["k_seq"][i] for i in nz],
                                           [c["v_seq"][i] for i in nz], c["ctx_len"][nz],
                                           c["scale"])
    for got_o, got_l, what in ((o, lse, "equal-share"), (of, lf, "fixed splits")):
        go, gl = to_np64(got_o), got_l.cpu().numpy()
        assert_attention_close(go[nz], ref, gl[nz], ref_lse, what=what)
        for i in set(range(len(ctx))) - set(nz):   # empty request: o = 0, lse = -inf
            assert not go[i].any() and np.isneginf(gl[i]).all()


@pytest.mark.parametrize("group", [1, 4, 16])
def test_decode_group_sizes(group):
    Hkv = 2
    c = synth.decode_cache(seed=601, B=3, ctx_lens=[5, 300, 129], Hq=group * Hkv, Hkv=Hkv)
    o, lse = lcat.attn_decode(to_dev(c["q"]), to_dev(c["k_pool"]), to_dev(c["v_pool"]),
                              to_dev(c["block_head"]), to_dev(c["block_table"]),
                              to_dev(c["ctx_len"]), split_tokens=128)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_attention(c["q"], c["k_seq"], c["v_seq"], c["ctx_len"], c["scale"])
    assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="decode group")


def test_decode_batch_order_and_block_placement_invariance():
    """The article's state-persistence check: reordering the requests of a
    batch permutes the outputs bit for bit; moving blocks to other physical
    ids (same tags) leaves them unchanged bit for bit."""
    c = synth.decode_cache(seed=602, B=6, ctx_lens=[70, 500, 64, 1, 999, 2048], Hq=16, Hkv=2)
    args = [to_dev(c[k]) for k in ("q", "k_pool", "v_pool", "block_head", "block_table", "ctx_len")]
    o, lse = lcat.attn_decode(*args, split_tokens=256)
    perm = np.array([3, 0, 5, 1, 4, 2])
    pargs = [args[0][perm], args[1], args[2], args[3], args[4][perm].contiguous(), args[5][perm].contiguous()]
    o2, lse2 = lcat.attn_decode(*pargs, split_tokens=256)
    # move every block to a new physical id
    nb = c["k_pool"].shape[0]
    mv = np.random.default_rng(9).permutation(nb)
    inv = np.argsort(mv)
    kp2 = c["k_pool"][inv]
    vp2 = c["v_pool"][inv]
    tags2 = c["block_head"][inv]
    tab2 = np.where(c["block_table"] >= 0, mv[np.maximum(c["block_table"], 0)], -1).astype(np.int32)
    o3, lse3 = lcat.attn_decode(args[0], to_dev(kp2), to_dev(vp2), to_dev(tags2), to_dev(tab2),
                                args[5], split_tokens=256)
    torch.cuda.synchronize()
    assert torch.equal(o2, o[perm]) and torch.equal(lse2, lse[perm])
    assert torch.equal(o3, o) and torch.equal(lse3, lse)


def test_decode_equal_share_split_crosses_requests():
    """Automatic split: the blocks of all (request, KV head) segments are
    shared out equally among a fixed number of waves, so one wave's range can
    start and end inside segments and cover several; empty requests give
    o = 0 and lse = -inf.  Checked against the oracle row by row and against
    a fixed 256-key split of the same cache."""
    ctx = [0, 1, 8192, 64, 3000, 0, 777, 5000, 4096, 65] * 4   # 2680 (request, head, block) units
    log(f"decode equal-share split, {len(ctx)} requests")
    c = synth.decode_cache(seed=604, B=len(ctx), ctx_lens=ctx, Hq=16, Hkv=2, extra_blocks=3)
    args = [to_dev(c[k]) for k in ("q", "k_pool", "v_pool", "block_head", "block_table", "ctx_len")]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, lse = lcat.attn_decode(*args, split_tokens=0, dev_status=st)
    o2, lse2 = lcat.attn_decode(*args, split_tokens=256)
    torch.cuda.synchronize()
    assert st.item() == 0
    nz = [i for i, n in enumerate(ctx) if n > 0]
    z = [i for i, n in enumerate(ctx) if n == 0]
    ref, ref_lse = oracle.decode_attention(c["q"][nz], [c["k_seq"][i] for i in nz],
                                           [c["v_seq"][i] for i in nz], c["ctx_len"][nz], c["scale"])
    got = to_np64(o)
    got_lse = lse.cpu().numpy()
    e, r = assert_attention_close(got[nz], ref, got_lse[nz], ref_lse, what="equal-share decode")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")
    assert np.all(got[z] == 0.0) and np.all(np.isneginf(got_lse[z]))
    assert np.abs(got - to_np64(o2)).max() <= 1.6e-2   # two bf16 roundings of the same O
    assert np.abs(got_lse[nz] - lse2.cpu().numpy()[nz]).max() <= 1e-4


def test_decode_bad_tag_and_block_are_reported():
    c = synth.decode_cache(seed=603, B=2, ctx_lens=[200, 100], Hq=16, Hkv=2)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    tags = c["block_head"].copy()
    tags[c["block_table"][1, 1, 0]] = 7
    lcat.attn_decode(to_dev(c["q"]), to_dev(c["k_pool"]), to_dev(c["v_pool"]), to_dev(tags),
                     to_dev(c["block_table"]), to_dev(c["ctx_len"]), dev_status=st)
    torch.cuda.synchronize()
    assert st.item() == lcat.ATTN_DEV_BAD_TAG
    st.zero_()
    tab = c["block_table"].copy()
    tab[0, 0, 2] = 10 ** 6
    lcat.attn_decode(to_dev(c["q"]), to_dev(c["k_pool"]), to_dev(c["v_pool"]),
                     to_dev(c["block_head"]), to_dev(tab), to_dev(c["ctx_len"]), dev_status=st)
    torch.cuda.synchronize()
    assert st.item() == lcat.ATTN_DEV_BAD_BLOCK


# ---------------------------------------------------------------------------
# context parallelism on one GPU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("S,N,H,D,dtype", [(48, 4, 16, 128, np.int16), (50, 4, 2, 128, np.int16),
                                           (64, 8, 1, 3, np.int16), (40, 2, 3, 8, np.float32)])
def test_cp_shard_round_trip(mode, S, N, H, D, dtype):
    """Each rank's shard equals the oracle's token list of the full tensor bit
    for bit, positions are those tokens, and unsharding every rank rebuilds
    the full tensor (rows of other ranks untouched in between)."""
    if mode == "striped" and S % N:
        pytest.skip("striped needs S % N == 0")
    log(f"cp shard {mode} S={S} N={N} H={H} D={D}")
    rng = np.random.default_rng(S * 10 + N)
    x = rng.integers(-2 ** 15, 2 ** 15, size=(S, H, D)).astype(np.int16)
    if dtype == np.float32:
        x = rng.standard_normal((S, H, D)).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    back = torch.zeros_like(xd)
    for r in range(N):
        toks = oracle.cp_tokens(S, N, mode, r)
        sh, pos = lcat.cp_shard(xd, N, r, mode)
        torch.cuda.synchronize()
        assert np.array_equal(sh.cpu().numpy(), x[toks])
        assert np.array_equal(pos.cpu().numpy(), toks)
        lcat.cp_unshard(sh, S, N, r, mode, out=back)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), x)


def test_key_limits_count_keys_at_or_before_each_query():
    rng = np.random.default_rng(900)
    B, Sq, Sk = 2, 300, 257
    qp = np.sort(rng.integers(0, 5000, size=(B, Sq)), axis=1).astype(np.int32)
    kp = np.sort(rng.choice(5000, size=(B, Sk), replace=True), axis=1).astype(np.int32)
    qp[0, :5] = -3                         # before every key
    lim = lcat.attn_key_limits(to_dev(qp), to_dev(kp))
    torch.cuda.synchronize()
    want = np.array([[int(np.sum(kp[b] <= p_)) for p_ in qp[b]] for b in range(B)])
    assert np.array_equal(lim.cpu().numpy(), want)


@pytest.mark.parametrize("Sq,Sk", [(700, 900), (333, 64), (256, 1500)])
def test_prefill_limited_vs_oracle(Sq, Sk):
    """Rows attend a caller-given prefix of the keys (nondecreasing limits,
    some zero, some ragged, some past Sk); rows with no key give O = 0 and
    LSE = -inf."""
    log(f"prefill limited Sq={Sq} Sk={Sk}")
    B, Hq, Hkv = 2, 16, 2
    rng = np.random.default_rng(Sq + Sk)
    sq_, sk_, sv_ = np.random.SeedSequence(Sq * Sk).spawn(3)
    q = synth.normal_bf16(sq_, (B, Sq, Hq, 128))
    k = synth.normal_bf16(sk_, (B, Sk, Hkv, 128))
    v = synth.normal_bf16(sv_, (B, Sk, Hkv, 128))
    lim = np.sort(rng.integers(0, Sk + 40, size=(B, Sq)), axis=1).astype(np.int32)
    lim[:, : Sq // 10] = 0
    o, lse = lcat.attn_prefill_limited(to_dev(q), to_dev(k), to_dev(v), to_dev(lim))
    torch.cuda.synchronize()
    eff = np.minimum(lim, Sk)
    ref, ref_lse = oracle.attention_rows(q, k, v, eff.astype(np.int64), 128 ** -0.5)
    got, got_lse = to_np64(o), lse.cpu().numpy()
    live = eff > 0
    assert np.all(got[~live] == 0) and np.all(got_lse.transpose(0, 2, 1)[~live] == -np.inf)
    e, r = assert_attention_close(got[live], ref[live], got_lse.transpose(0, 2, 1)[live],
                                  ref_lse.transpose(0, 2, 1)[live], what="limited")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")


def test_merge_vs_oracle():
    """Seeded partials (bf16 O, fp32 LSE with -inf entries on either or both
    sides) merged on the GPU, in place and out of place, against the oracle's
    merge."""
    B, S, H, D = 2, 77, 4, 128
    rng = np.random.default_rng(901)
    oa = synth.normal_bf16(902, (B, S, H, D))
    ob = synth.normal_bf16(903, (B, S, H, D))
    la = rng.normal(0, 4, size=(B, H, S)).astype(np.float32)
    lb = rng.normal(0, 4, size=(B, H, S)).astype(np.float32)
    la[:, :, :5] = -np.inf
    lb[:, :, 3:8] = -np.inf
    ref, ref_l = oracle.merge_normalized([(synth.bf16_bits_to_f32(oa), la),
                                          (synth.bf16_bits_to_f32(ob), lb)])
    o, l = lcat.attn_merge(to_dev(oa), to_dev(la), to_dev(ob), to_dev(lb))
    oad, lad = to_dev(oa), to_dev(la)
    lcat.attn_merge(oad, lad, to_dev(ob), to_dev(lb), o=oad, lse=lad)
    torch.cuda.synchronize()
    for got_o, got_l in ((o, l), (oad, lad)):
        g = to_np64(got_o)
        assert np.all(np.abs(g - ref) <= 2 ** -8 * np.abs(ref) + 1e-6)
        gl = got_l.cpu().numpy()
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(gl), fin)
        assert np.all(np.abs(gl[fin] - ref_l[fin]) <= 1e-5 + 1e-6 * np.abs(ref_l[fin]))
    assert np.all(to_np64(o)[:, 3:5] == 0)            # both sides empty


@pytest.mark.parametrize("mode", ["contiguous", "striped", "zigzag"])
def test_cp_ring_attention_on_one_gpu(mode):
    """One rank's ring attention, all on one GPU: shard Q/K/V, attend the
    rank's queries to every rank's key shard with the position-derived
    limits, merge the partials; the result is the causal attention of the
    rank's tokens (oracle, full sequence).  Every partial is also checked
    against the oracle's position-masked attention (rows that see no key of
    that shard: O = 0, LSE = -inf)."""
    S, N, Hq, Hkv = 1536, 4, 16, 2
    log(f"cp ring {mode} S={S} N={N}")
    d = synth.dense_bf16(seed=910, B=1, S=S, Hq=Hq, Hkv=Hkv)
    q, k, v = (to_dev(d[n][0]) for n in ("q", "k", "v"))
    shards = [(lcat.cp_shard(k, N, s_, mode)[0], lcat.cp_shard(v, N, s_, mode)[0],
               lcat.cp_shard(k, N, s_, mode)[1]) for s_ in range(N)]
    for r in (0, N - 1):
        qr, qpos = lcat.cp_shard(q, N, r, mode)
        o = lse = None
        for s_, (ks, vs, kpos) in enumerate(shards):
            lim = lcat.attn_key_limits(qpos, kpos)
            op, lp = lcat.attn_prefill_limited(qr[None], ks[None], vs[None], lim)
            torch.cuda.synchronize()
            tq, tk = oracle.cp_tokens(S, N, mode, r), oracle.cp_tokens(S, N, mode, s_)
            pr, pl = oracle.attention_positions(d["q"][:, tq], d["k"][:, tk], d["v"][:, tk], tq, tk,
                                                d["scale"])
            live = np.isfinite(pl[0, 0])
            assert np.all(to_np64(op)[:, ~live] == 0)
            assert np.all(lp.cpu().numpy()[..., ~live] == -np.inf)
            if live.any():
                assert_attention_close(to_np64(op)[:, live], pr[:, live], lp.cpu().numpy()[..., live],
                                       pl[..., live], what="cp partial")
            if o is None:
                o, lse = op, lp
            else:
                lcat.attn_merge(o, lse, op, lp, o=o, lse=lse)
        # the same ring with the merge folded into each partial's epilogue
        oa = torch.empty_like(o)
        la = torch.empty_like(lse)
        for s_, (ks, vs, kpos) in enumerate(shards):
            lim = lcat.attn_key_limits(qpos, kpos)
            lcat.attn_prefill_limited(qr[None], ks[None], vs[None], lim, o=oa, lse=la,
                                      accumulate=s_ > 0)
        torch.cuda.synchronize()
        rows = oracle.cp_tokens(S, N, mode, r)
        ref, ref_lse = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True, rows=rows)
        e, rl = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="cp ring")
        log(f"  rank {r}: max abs {e:.3g} rel-L2 {rl:.3g}")
        e, rl = assert_attention_close(to_np64(oa), ref, la.cpu().numpy(), ref_lse,
                                       what="cp ring, merged in the epilogue")
        log(f"  rank {r} (accumulate): max abs {e:.3g} rel-L2 {rl:.3g}")


# ---------------------------------------------------------------------------
# FP8 KV cache
# ---------------------------------------------------------------------------
from oracle import fp8 as ofp8  # noqa: E402


def _fp8_pools_from_oracle(c):
    """Oracle-quantised pools of a decode cache; slots past ctx_len (and spare
    blocks) get the NaN code and NaN scales, so reading them is caught."""
    kb, vb = c["k_pool"].copy(), c["v_pool"].copy()
    kb[np.isnan(synth.bf16_bits_to_f32(kb))] = 0
    vb[np.isnan(synth.bf16_bits_to_f32(vb))] = 0
    k8, v8, ks, vs = ofp8.quantize_kv_pool(kb, vb)
    valid = np.zeros((c["n_blocks"], 64), dtype=bool)
    table = c["block_table"]
    for b, ctx in enumerate(c["ctx_len"]):
        for g in range(table.shape[1]):
            for j in range((int(ctx) + 63) // 64):
                valid[table[b, g, j], : min(64, int(ctx) - 64 * j)] = True
    k8[~valid] = 0x7F
    v8.transpose(0, 2, 1)[~valid] = 0x7F
    ks[~valid] = np.nan
    vs[~valid] = np.nan
    return k8, v8, ks, vs


def test_kv_quantize_fp8_bit_exact():
    """GPU quantisation of bf16 pools equals the oracle's codes and scales bit
    for bit (token groups spanning a wide range of magnitudes, an all-zero
    token, values that round to subnormal codes)."""
    n = 9
    kf = synth.bf16_bits_to_f32(synth.normal_bf16(950, (n, 64, 128)))
    vf = synth.bf16_bits_to_f32(synth.normal_bf16(951, (n, 128, 64)))
    mag = np.exp(np.random.default_rng(952).uniform(-30, 30, size=(n, 64))).astype(np.float32)
    kf = kf * mag[:, :, None]
    vf = vf * mag[:, None, :]
    kf[0, 5] = 0.0
    vf[1, :, 7] = 0.0
    kf[2, 9, :64] *= 1e-4                   # small entries next to a large one: subnormal codes
    kb, vb = synth.f32_to_bf16_bits(kf), synth.f32_to_bf16_bits(vf)
    k8, v8, ks, vs = lcat.attn_kv_quantize_fp8(to_dev(kb), to_dev(vb))
    torch.cuda.synchronize()
    rk8, rv8, rks, rvs = ofp8.quantize_kv_pool(kb, vb)
    assert np.array_equal(ks.cpu().numpy(), rks) and np.array_equal(vs.cpu().numpy(), rvs)
    assert np.array_equal(k8.cpu().numpy(), rk8)
    assert np.array_equal(v8.cpu().numpy(), rv8)


def test_kv_append_fp8_bit_exact():
    """Appending tokens into fp8 pools writes each token's oracle codes and
    scales at its slot (partial first and last blocks, several requests and
    heads) and leaves every other slot of the pools untouched."""
    B, Hkv, T = 3, 2, 100
    starts = np.array([0, 70, 130], dtype=np.int32)
    max_blocks = 5
    rng = np.random.default_rng(970)
    n = B * Hkv * max_blocks + 4
    ids = rng.permutation(n)[: B * Hkv * max_blocks].reshape(B, Hkv, max_blocks).astype(np.int32)
    tags = np.full((n,), -1, dtype=np.int32)
    for g in range(Hkv):
        tags[ids[:, g]] = 3 + g
    k8 = rng.integers(0, 256, size=(n, 64, 128), dtype=np.uint8)
    v8 = rng.integers(0, 256, size=(n, 128, 64), dtype=np.uint8)
    ks = rng.uniform(0.1, 1, size=(n, 64)).astype(np.float32)
    vs = rng.uniform(0.1, 1, size=(n, 64)).astype(np.float32)
    kn = synth.normal_bf16(971, (B, T, Hkv, 128))
    vn = synth.normal_bf16(972, (B, T, Hkv, 128))
    kn_f = synth.bf16_bits_to_f32(kn) * np.exp(rng.uniform(-5, 5, (B, T, Hkv, 1))).astype(np.float32)
    kn = synth.f32_to_bf16_bits(kn_f)
    d8 = [torch.from_numpy(a.copy()).cuda() for a in (k8, v8)]
    dsc = [to_dev(a.copy()) for a in (ks, vs)]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    lcat.attn_kv_append_fp8(to_dev(kn), to_dev(vn), d8[0], d8[1], dsc[0], dsc[1], to_dev(tags),
                            to_dev(ids), to_dev(starts), kv_head_base=3, dev_status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    ck, sk = ofp8.quantize_groups(synth.bf16_bits_to_f32(kn))     # [B][T][Hkv][128], [B][T][Hkv]
    cv, sv = ofp8.quantize_groups(synth.bf16_bits_to_f32(vn))
    for b in range(B):
        for t in range(T):
            pos = starts[b] + t
            for g in range(Hkv):
                blk, sl = ids[b, g, pos // 64], pos % 64
                k8[blk, sl], ks[blk, sl] = ck[b, t, g], sk[b, t, g]
                v8[blk, :, sl], vs[blk, sl] = cv[b, t, g], sv[b, t, g]
    assert np.array_equal(d8[0].cpu().numpy(), k8) and np.array_equal(d8[1].cpu().numpy(), v8)
    assert np.array_equal(dsc[0].cpu().numpy(), ks) and np.array_equal(dsc[1].cpu().numpy(), vs)


@pytest.mark.parametrize("split", [64, 256, 0])
def test_decode_fp8_vs_oracle(split):
    ctx = [1, 2, 63, 64, 65, 127, 128, 1000, 3001]
    log(f"decode fp8 ctx={ctx} split={split}")
    c = synth.decode_cache(seed=960, B=len(ctx), ctx_lens=ctx, Hq=16, Hkv=2, kv_head_base=2,
                           extra_blocks=5)
    k8, v8, ks, vs = _fp8_pools_from_oracle(c)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, lse = lcat.attn_decode_fp8(to_dev(c["q"]), torch.from_numpy(k8).cuda(),
                                  torch.from_numpy(v8).cuda(), to_dev(ks), to_dev(vs),
                                  to_dev(c["block_head"]), to_dev(c["block_table"]),
                                  to_dev(c["ctx_len"]), kv_head_base=2, split_tokens=split,
                                  dev_status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    kq, vq = ofp8.gather_dequantized(k8, v8, ks, vs, c["block_table"], c["ctx_len"])
    ref, ref_lse = oracle.decode_attention(c["q"], kq, vq, c["ctx_len"], c["scale"])
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="decode fp8")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")


@pytest.mark.parametrize("group", [1, 4, 16])
def test_decode_fp8_group_sizes(group):
    Hkv = 2
    c = synth.decode_cache(seed=961 + group, B=3, ctx_lens=[700, 64, 129], Hq=group * Hkv, Hkv=Hkv)
    k8, v8, ks, vs = _fp8_pools_from_oracle(c)
    o, lse = lcat.attn_decode_fp8(to_dev(c["q"]), torch.from_numpy(k8).cuda(),
                                  torch.from_numpy(v8).cuda(), to_dev(ks), to_dev(vs),
                                  to_dev(c["block_head"]), to_dev(c["block_table"]),
                                  to_dev(c["ctx_len"]))
    torch.cuda.synchronize()
    kq, vq = ofp8.gather_dequantized(k8, v8, ks, vs, c["block_table"], c["ctx_len"])
    ref, ref_lse = oracle.decode_attention(c["q"], kq, vq, c["ctx_len"], c["scale"])
    assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="decode fp8")


# ---------------------------------------------------------------------------
# chunked prefill against the paged cache
# ---------------------------------------------------------------------------
def _run_chunked(d, C, kv_head_base=0):
    B, S, Hq, _ = d["q"].shape
    Hkv = d["k"].shape[2]
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    n_blocks = d["n_blocks"]
    k_pool = torch.full((n_blocks, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.full((n_blocks, 128, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    tags = to_dev(d["block_head"])
    table = to_dev(d["block_table"])
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    for c0 in range(0, S, C):
        c1 = min(S, c0 + C)
        ctx_before = torch.full((B,), c0, dtype=torch.int32, device="cuda")
        oc, lc = lcat.attn_chunked_prefill(q[:, c0:c1].contiguous(), k[:, c0:c1].contiguous(),
                                           v[:, c0:c1].contiguous(), k_pool, v_pool, tags, table,
                                           ctx_before, kv_head_base=kv_head_base, dev_status=st)
        o[:, c0:c1] = oc
        lse[:, :, c0:c1] = lc
    torch.cuda.synchronize()
    return o, lse, k_pool, v_pool, st


@pytest.mark.parametrize("S,C", [(700, 256), (512, 64), (300, 300), (200, 90)])
def test_chunked_prefill_all_rows(S, C):
    log(f"chunked S={S} C={C}")
    d = synth.chunked_prefill(seed=700 + S, B=2, S=S, C=C, Hq=16, Hkv=2, kv_head_base=4)
    o, lse, k_pool, v_pool, st = _run_chunked(d, C, kv_head_base=4)
    assert st.item() == 0
    ref, ref_lse = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True)
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="chunked")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")
    # cache read back bit for bit
    kg, vg = oracle.paged_gather(bits(k_pool), bits(v_pool), d["block_table"], [S, S])
    np.testing.assert_array_equal(kg, d["k"])
    np.testing.assert_array_equal(vg, d["v"])



@pytest.mark.parametrize("S,C,stepped", [(1500, 512, False), (1500, 1024, True)])
def test_chunked_prefill_long_rows(S, C, stepped):
    """Chunks deep enough for the interleaved key loop over cached blocks;
    the stepped inputs make that loop take its exact-maximum recovery path."""
    log(f"chunked long S={S} C={C} stepped={stepped}")
    d = synth.chunked_prefill(seed=720 + S, B=2, S=S, C=C, Hq=16, Hkv=2, kv_head_base=2)
    if stepped:
        d.update(_stepped_scores(730 + S, 2, S, 16, 2, step_keys=128))
    o, lse, k_pool, v_pool, st = _run_chunked(d, C, kv_head_base=2)
    assert st.item() == 0
    ref, ref_lse = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True)
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="chunked")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")

def test_chunked_equals_dense_prefill():
    """Chunked prefill of a sequence agrees with one dense causal prefill of
    the same sequence (both against the same oracle rows)."""
    d = synth.chunked_prefill(seed=710, B=1, S=384, C=128, Hq=16, Hkv=2)
    o, lse, *_ = _run_chunked(d, 128)
    od, lsed = lcat.attn_prefill(to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"]), causal=True)
    torch.cuda.synchronize()
    assert (o.float() - od.float()).abs().max().item() <= BF16_ATOL
    assert (lse - lsed).abs().max().item() <= 2e-3


# ---------------------------------------------------------------------------
# sustained-MFMA yardstick (measurement helper, not part of the path)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("a_from_lds", [False, True])
def test_measure_mfma_rate_runs(a_from_lds):
    log(f"measure_mfma_rate n_wg=16 iters=64 a_from_lds={a_from_lds}")
    a = lcat.measure_mfma_rate(n_wg=16, iters=64, seed=5, a_from_lds=a_from_lds)
    b = lcat.measure_mfma_rate(n_wg=16, iters=64, seed=5, a_from_lds=a_from_lds)
    c = lcat.measure_mfma_rate(n_wg=16, iters=64, seed=6, a_from_lds=a_from_lds)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert torch.equal(a, b)          # the operands depend only on the seed
    assert not torch.equal(a, c)
    assert lcat.mfma_rate_flops(16, 64) == 16 * 8 * 64 * 4 * 32768


def test_measure_hbm_read_and_copy():
    log("measure_hbm_read 16 waves x 1000 units, measure_hbm_copy 1 MiB + 48 B")
    rng = np.random.default_rng(77)
    words = rng.integers(0, 2**32, size=(16 * 1000 + 7) * 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    out, nread = lcat.measure_hbm_read(buf, waves=16)
    torch.cuda.synchronize()
    assert nread == 16 * 1000 * 16
    # lane l of wave w folds units w*1000 + l + 64k (k >= 0) of its share
    units = words[: 16 * 1000 * 4].reshape(16, 1000, 4)
    fold = np.bitwise_xor.reduce(units, axis=2)              # the 4 words of a unit
    want = np.zeros((16, 64), dtype=np.uint32)
    for lane in range(64):
        want[:, lane] = np.bitwise_xor.reduce(fold[:, lane::64], axis=1)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32).reshape(16, 64), want)
    src = torch.from_numpy(rng.integers(0, 255, size=(1 << 20) + 48, dtype=np.uint8)).cuda()
    dst = torch.zeros_like(src)
    assert lcat.measure_hbm_copy(src, dst) == (1 << 20) + 48
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    keep = src.clone()
    lcat.measure_hbm_copy(src, src)     # in place: the data is unchanged
    torch.cuda.synchronize()
    assert torch.equal(src, keep)
