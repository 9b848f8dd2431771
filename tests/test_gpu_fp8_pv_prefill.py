"""GPU parity of the prefill with both products on FP8 (FA3's FP8 path with
block quantisation, "Flash Attention and distributed inference" §18.5; the
format and scale rule are the reading stated in oracle/fp8.py, with V's
blocks running along keys).

The V quantiser must reproduce the oracle's codes and scales bit for bit, in
the tile layout attn.h states.  The prefill is compared element by element
with exact attention over the dequantised Q, K and V (oracle.fp8.
attention_fp8_pv).  What that leaves is the kernel's rounding of the weights
P' to e4m3 before P V, which the oracle does not model (it depends on the
kernel's running reference), bounded per element here from the format alone:

* P' = 2^(s - m + 3) = C w_j, w the exact softmax weights and m an observed
  score of the row (m <= s_max), so the largest weight C w_max lies in
  [8, 2^8.75] and C >= 8 / w_max;
* a weight in e4m3's normal range is off by at most 2^-4 of itself; one
  below it (possible only where w_j < 2^-9 w_max) by at most
  min(2^-10, C w_j);
* both sums use the same rounded weights, so O - O'' = sum d_j (v_j - O'') /
  sum P^_j with sum P^_j >= (15/16) C W, W the total weight of the keys with
  w_j >= 2^-9 w_max, which gives
      |O - O''| <= (16/15) / W * (2^-4 a + b),
  a = sum_j w_j |v_j - O''| and b = sum over the small weights of
  min(2^-13 w_max, w_j) |v_j - O''| (both with |v_j - O''| <= |v_j| + |O''|),
plus the bf16 rounding of O and fp32 slack.  The LSE moves by
-ln(1 - 2^-4 - r) at most, r = sum over the small weights of
min(2^-13 w_max, w_j).  A per-row relative L2 bar
(0.08) and a whole-tensor one (0.045) sit above the statistical size of
that rounding (about 0.025-0.036 per row on N(0,1) data: e4m3's relative
spacing 2^-3 .. 2^-4) and far below what a wrong key order or a wrong
denominator produces (order 1).  All calls go through the C ABI.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import fp8 as ofp8
from tests.gpu_helpers import log, to_dev, to_np64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lcat = pytest.importorskip("long_context_attention_tiled_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lcat.load_library()


def _expected_v_layout(v_bits):
    """Oracle codes / exponents of V (blocks of 32 keys per dim) arranged as
    attn_quantize_fp8_v stores them."""
    v = synth.bf16_bits_to_f32(v_bits)
    B, S, H, D = v.shape
    s64 = -(-S // 64) * 64
    vt = np.zeros((B, H, D, s64), np.float32)
    vt[..., :S] = np.transpose(v, (0, 2, 3, 1))
    codes, e = ofp8.quantize_blocks(vt)                 # e [B][H][D][s64 / 32]
    eb = ofp8.e8m0_bytes(e).reshape(B, H, 4, 32, s64 // 64, 2)   # [b][g][db][r][t][h]
    scales = np.transpose(eb, (0, 1, 4, 5, 3, 2)).reshape(B, H, s64 // 64, 256)
    return codes, scales


def _run(d, causal, signs=None):
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    k8, ks = lcat.attn_quantize_fp8_blocks(k, signs=signs)
    v8t, vs = lcat.attn_quantize_fp8_v(v)
    return lcat.attn_prefill_fp8_pv(q, k8, ks, v8t, vs, causal=causal, scale=d["scale"], signs=signs)


def _bounds(d, causal, ref, rows, signs=None):
    """Per-element bound on |O - O''| and per-row bound on |dLSE| from the
    rounding of P' to e4m3 (module docstring)."""
    qd, kd = ofp8.prefill_fp8_operands(np.ascontiguousarray(d["q"][:, rows]), d["k"], d["scale"],
                                       signs)
    vabs = np.abs(ofp8.dequantized_v_keys(d["v"]))
    B, R, Hq, D = qd.shape
    S, Hkv = kd.shape[1], kd.shape[2]
    G = Hq // Hkv
    bo = np.zeros(ref.shape)
    bl = np.zeros((B, Hq, R))
    valid = (np.arange(S)[None, :] <= rows[:, None]) if causal else np.ones((R, S), bool)
    for b in range(B):
        for h in range(Hq):
            s = qd[b, :, h, :] @ kd[b, :, h // G, :].T
            s = np.where(valid, s, -np.inf)
            w = np.exp2(s - s.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            wmax = w.max(axis=1, keepdims=True)
            small = valid & (w < 2.0 ** -9 * wmax)
            W = 1.0 - np.where(small, w, 0.0).sum(axis=1, keepdims=True)
            msub = np.where(small, np.minimum(2.0 ** -13 * wmax, w), 0.0)
            rsub = msub.sum(axis=1, keepdims=True)
            oabs = np.abs(ref[b, :, h, :])
            a = w @ vabs[b, :, h // G, :] + oabs
            bs = msub @ vabs[b, :, h // G, :] + rsub * oabs
            bo[b, :, h, :] = (16 / 15) / W * (2.0 ** -4 * a + bs)
            bl[b, h, :] = -np.log(1 - 2.0 ** -4 - rsub[:, 0])
    return bo, bl


def _assert_close(got, ref, got_lse, ref_lse, d, causal, rows, what, signs=None):
    bo, bl = _bounds(d, causal, ref, rows, signs)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    lim = bo + 2.0 ** -8 * np.abs(ref) + 1e-3
    bad = err > lim
    assert not bad.any(), f"{what}: {bad.sum()} elements above the P-rounding bound, max err {err.max():.3g}"
    num = np.linalg.norm((got - ref).reshape(-1, ref.shape[-1]), axis=-1)
    den = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=-1)
    rl2 = num / np.maximum(den, 1e-30)
    assert rl2.max() <= 0.08, f"{what}: per-row relative L2 error {rl2.max():.3g}"
    tot = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert tot <= 0.045, f"{what}: relative L2 error {tot:.3g}"
    dl = np.abs(np.asarray(got_lse, np.float64) - ref_lse)
    assert (dl <= bl + 1e-3).all(), f"{what}: LSE error {dl.max():.3g}"
    return err.max(), rl2.max(), tot, (err / lim).max()


@pytest.mark.parametrize("S,B,Hkv", [(1, 1, 2), (63, 2, 2), (64, 1, 1), (100, 2, 2), (257, 1, 3),
                                     (4096, 1, 2)])
def test_quantize_fp8_v_bit_exact(S, B, Hkv):
    """Magnitudes spread over 2^-40 .. 2^40 per key, an all-zero block, a block
    of bf16 subnormals, a block whose maximum sits exactly on 448 * 2^e; the
    ragged last tile's missing keys must come back as code 0."""
    rng = np.random.default_rng(400 + S)
    v = rng.standard_normal((B, S, Hkv, 128)) * np.exp2(rng.uniform(-40, 40, (B, S, Hkv, 1)))
    if S >= 64:
        v[0, 32:64, 0, 5] = 0.0
        v[0, :32, 0, 6] = rng.uniform(-1, 1, 32) * 2.0 ** -130
        v[0, :32, 0, 7] = rng.uniform(-1, 1, 32) * 100.0
        v[0, 3, 0, 7] = 448.0 * 2.0 ** -3
    bits = synth.f32_to_bf16_bits(v.astype(np.float32))
    log(f"quantize_fp8_v S={S} B={B} Hkv={Hkv}")
    v8t, vs = lcat.attn_quantize_fp8_v(to_dev(bits))
    torch.cuda.synchronize()
    want_c, want_s = _expected_v_layout(bits)
    np.testing.assert_array_equal(v8t.cpu().numpy(), want_c)
    np.testing.assert_array_equal(vs.cpu().numpy(), want_s)


@pytest.mark.parametrize("S,B,Hq,Hkv,causal", [
    (1, 1, 16, 2, True), (63, 1, 16, 2, True), (64, 2, 16, 2, True), (65, 1, 16, 2, False),
    (300, 2, 16, 2, True), (640, 1, 16, 2, True), (640, 1, 16, 2, False), (200, 1, 8, 8, True),
    (130, 2, 4, 1, True), (257, 1, 32, 2, False),
])
def test_prefill_fp8_pv_vs_oracle(S, B, Hq, Hkv, causal):
    log(f"prefill fp8 pv S={S} B={B} Hq={Hq} Hkv={Hkv} causal={causal}")
    d = synth.dense_bf16(seed=510 + S + Hq, B=B, S=S, Hq=Hq, Hkv=Hkv)
    o, lse = _run(d, causal)
    torch.cuda.synchronize()
    ref, ref_lse = ofp8.attention_fp8_pv(d["q"], d["k"], d["v"], d["scale"], causal=causal)
    e, r, t, f = _assert_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, d, causal,
                               np.arange(S), "prefill fp8 pv")
    log(f"  max abs {e:.3g} row rel-L2 {r:.3g} rel-L2 {t:.3g} (bound used {f:.2f})")


def test_prefill_fp8_pv_uniform_v():
    """Closed form: V equal along keys gives O = V'' (the one dequantised
    value per dim) for every row, whatever the weights, because numerator and
    denominator use the same rounded weights; rows of 1 .. 2048 keys."""
    S = 2048
    d = synth.dense_bf16(seed=530, B=1, S=S, Hq=16, Hkv=2)
    vrow = np.random.default_rng(531).standard_normal((1, 1, 2, 128)) * 3
    d["v"] = np.ascontiguousarray(
        np.broadcast_to(synth.f32_to_bf16_bits(vrow.astype(np.float32)), (1, S, 2, 128)))
    log("prefill fp8 pv uniform V, S=2048 causal")
    o, _ = _run(d, True)
    torch.cuda.synchronize()
    want = ofp8.dequantized_v_keys(d["v"])[0, 0]          # [Hkv][128]
    got = to_np64(o)[0].reshape(S, 2, 8, 128)
    err = np.abs(got - want[None, :, None, :])
    assert (err <= 2.0 ** -8 * np.abs(want[None, :, None, :]) + 1e-6).all(), err.max()


@pytest.mark.parametrize("S,B,Hq,Hkv,causal,outliers", [
    (300, 2, 16, 2, True, True), (640, 1, 16, 2, False, True), (130, 2, 4, 1, True, False),
    (1100, 1, 16, 2, True, True), (1300, 1, 4, 4, True, True), (257, 1, 32, 2, False, True),
])
def test_prefill_fp8_pv_rotated_vs_oracle(S, B, Hq, Hkv, causal, outliers):
    """Incoherent processing: Q and K rotated by diag(s) H before they are
    quantised (the K quantiser and the prefill get the same signs); every
    row against the oracle over the rotated, dequantised operands, on
    N(0, 1) inputs and on inputs with outlier channels."""
    log(f"prefill fp8 pv rotated S={S} B={B} Hq={Hq} Hkv={Hkv} causal={causal} outliers={outliers}")
    gen = synth.dense_bf16_outliers if outliers else synth.dense_bf16
    d = gen(seed=560 + S, B=B, S=S, Hq=Hq, Hkv=Hkv)
    signs = synth.hadamard_signs(561 + S)
    o, lse = _run(d, causal, signs)
    torch.cuda.synchronize()
    ref, ref_lse = ofp8.attention_fp8_pv(d["q"], d["k"], d["v"], d["scale"], causal=causal,
                                         signs=signs)
    e, r, t, f = _assert_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, d, causal,
                               np.arange(S), "prefill fp8 pv rotated", signs)
    log(f"  max abs {e:.3g} row rel-L2 {r:.3g} rel-L2 {t:.3g} (bound used {f:.2f})")


def _stepped_scores(seed, B, S, Hq, Hkv, step_keys=128, step=13.0, D=128):
    """Scores that climb about 13 (natural-log units) every `step_keys` keys:
    inside the interleaved loop every step pushes the weights past 2^8.75, so
    the exact-maximum recovery runs again and again."""
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
    (1100, 2, 16, 2, False, True), (1500, 1, 8, 2, True, False), (1300, 1, 4, 4, True, False),
    (1300, 1, 4, 4, True, True),
])
def test_prefill_fp8_pv_long_rows(S, B, Hq, Hkv, causal, stepped):
    """Long enough for the interleaved key loop; every row against the oracle.
    With a GQA group below 8 a workgroup holds several 32-row blocks whose
    causal rows end in different key tiles, so its waves leave the
    interleaved loop at different iterations while sharing its barriers."""
    log(f"prefill fp8 pv long S={S} B={B} Hq={Hq} Hkv={Hkv} causal={causal} stepped={stepped}")
    d = (_stepped_scores(840 + S, B, S, Hq, Hkv) if stepped
         else synth.dense_bf16(seed=840 + S, B=B, S=S, Hq=Hq, Hkv=Hkv))
    o, lse = _run(d, causal)
    torch.cuda.synchronize()
    ref, ref_lse = ofp8.attention_fp8_pv(d["q"], d["k"], d["v"], d["scale"], causal=causal)
    e, r, t, f = _assert_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, d, causal,
                               np.arange(S), "prefill fp8 pv long")
    log(f"  max abs {e:.3g} row rel-L2 {r:.3g} rel-L2 {t:.3g} (bound used {f:.2f})")


@pytest.mark.parametrize("rotated", [False, True])
def test_prefill_fp8_pv_32k_causal_sampled(rotated):
    """The 32K causal GQA shape (16 Q / 2 KV heads) on the seeded N(0,1)
    inputs themselves, plain and with Q and K rotated (the signs the bench
    uses): 512 seeded rows plus the forced rows against the oracle over the
    dequantised operands; the error against exact attention is logged for
    the record."""
    S = 32768
    log(f"fp8 pv 32K rotated={rotated}: generating inputs")
    d = synth.causal_gqa(seed=2, S=S)
    signs = synth.hadamard_signs(93) if rotated else None
    o, lse = _run(d, True, signs)
    torch.cuda.synchronize()
    rows = synth.sample_rows(23, S, 512, [0, 1, 31, 32, 63, 64, 65, 127, 128, S // 2, S - 2, S - 1])
    log(f"fp8 pv 32K: oracle on {rows.size} rows x 16 heads")
    ref, ref_lse = ofp8.attention_fp8_pv(d["q"], d["k"], d["v"], d["scale"], causal=True, rows=rows,
                                         signs=signs)
    idx = torch.from_numpy(rows).cuda()
    got = to_np64(o[:, idx])
    e, r, t, f = _assert_close(got, ref, lse[:, :, idx].cpu().numpy(), ref_lse, d, True, rows,
                               "fp8 pv 32K", signs)
    log(f"fp8 pv 32K: max abs {e:.3g} row rel-L2 {r:.3g} rel-L2 {t:.3g} (bound used {f:.2f})")
    exact, _ = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True, rows=rows)
    dev = np.abs(got - exact)
    log(f"fp8 pv 32K: against exact attention: max abs {dev.max():.3g}, "
        f"rel-L2 {np.linalg.norm(dev) / np.linalg.norm(exact):.3g}")
