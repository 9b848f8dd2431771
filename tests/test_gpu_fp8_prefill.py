"""GPU parity of the FP8-score prefill (FA3's FP8 path with block
quantisation, "Flash Attention and distributed inference" §18.5; the format
and scale rule are the reading stated in oracle/fp8.py).

The block quantiser must reproduce the oracle's codes and scales bit for bit.
The prefill is compared element by element with the oracle's attention over
the dequantised operands (oracle.fp8.attention_fp8), with the bf16 bar: the
quantisation is modelled exactly there, so what remains is fp32 accumulation
and the bf16 rounding of P and O, as in the bf16 prefill.  All calls go
through the C ABI.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import fp8 as ofp8
from tests.gpu_helpers import assert_attention_close, log, to_dev, to_np64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lcat = pytest.importorskip("long_context_attention_tiled_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lcat.load_library()


def _quantize_k(k_bits):
    k = to_dev(k_bits)
    codes, scales = lcat.attn_quantize_fp8_blocks(k)
    return k, codes, scales


def test_quantize_fp8_blocks_bit_exact():
    """Rows with magnitudes spread over 2^-40 .. 2^40, an all-zero block, a
    block of bf16 subnormals and blocks whose maximum sits exactly on 448 * 2^e
    and just above it."""
    rng = np.random.default_rng(300)
    x = rng.standard_normal((257, 128)) * np.exp2(rng.uniform(-40, 40, (257, 1)))
    x[3, 32:64] = 0.0
    x[4, :32] = rng.uniform(-1, 1, 32) * 2.0 ** -130
    x[5, :32] = rng.uniform(-1, 1, 32) * 100.0
    x[5, 7] = 448.0 * 2.0 ** -3
    x[6, 64:96] = rng.uniform(-1, 1, 32)
    x[6, 70] = 448.0 * 2.0 ** 2 * (1 + 2.0 ** -7)
    bits = synth.f32_to_bf16_bits(x.astype(np.float32))
    log("quantize_fp8_blocks 257 x 128")
    codes, scales = lcat.attn_quantize_fp8_blocks(to_dev(bits))
    torch.cuda.synchronize()
    want_c, want_e = ofp8.quantize_blocks(synth.bf16_bits_to_f32(bits))
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)
    np.testing.assert_array_equal(scales.cpu().numpy(), ofp8.e8m0_bytes(want_e))


@pytest.mark.parametrize("S,B,Hq,Hkv,causal", [
    (1, 1, 16, 2, True), (63, 1, 16, 2, True), (64, 2, 16, 2, True), (65, 1, 16, 2, False),
    (300, 2, 16, 2, True), (640, 1, 16, 2, True), (640, 1, 16, 2, False), (200, 1, 8, 8, True),
    (130, 2, 4, 1, True), (257, 1, 32, 2, False),
])
def test_prefill_fp8_vs_oracle(S, B, Hq, Hkv, causal):
    log(f"prefill fp8 S={S} B={B} Hq={Hq} Hkv={Hkv} causal={causal}")
    d = synth.dense_bf16(seed=310 + S + Hq, B=B, S=S, Hq=Hq, Hkv=Hkv)
    k, k8, ks = _quantize_k(d["k"])
    o, lse = lcat.attn_prefill_fp8(to_dev(d["q"]), k8, ks, to_dev(d["v"]), causal=causal)
    torch.cuda.synchronize()
    ref, ref_lse = ofp8.attention_fp8(d["q"], d["k"], d["v"], d["scale"], causal=causal)
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="prefill fp8")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")


def _stepped_scores(seed, B, S, Hq, Hkv, step_keys=128, step=13.0, D=128):
    """Scores that climb about 13 (natural-log units) every `step_keys` keys,
    so the running maximum jumps far past any lazy-rescale bound inside the
    interleaved loop (the exact-maximum recovery path runs)."""
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
def test_prefill_fp8_long_rows(S, B, Hq, Hkv, causal, stepped):
    """Long enough for the interleaved key loop; every row against the oracle."""
    log(f"prefill fp8 long S={S} B={B} Hq={Hq} Hkv={Hkv} causal={causal} stepped={stepped}")
    d = (_stepped_scores(820 + S, B, S, Hq, Hkv) if stepped
         else synth.dense_bf16(seed=820 + S, B=B, S=S, Hq=Hq, Hkv=Hkv))
    k, k8, ks = _quantize_k(d["k"])
    o, lse = lcat.attn_prefill_fp8(to_dev(d["q"]), k8, ks, to_dev(d["v"]), causal=causal,
                                   scale=d["scale"])
    torch.cuda.synchronize()
    ref, ref_lse = ofp8.attention_fp8(d["q"], d["k"], d["v"], d["scale"], causal=causal)
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse,
                                  what="prefill fp8 long")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")


@pytest.mark.parametrize("rows,outliers", [(1, True), (37, False), (4096, True), (65536, True)])
def test_quantize_fp8_rotated_bit_exact(rows, outliers):
    """K rows rotated by diag(s) H (fp32 butterflies in the stated order) and
    block-quantised: codes and scale bytes equal to the oracle's."""
    gen = synth.dense_bf16_outliers if outliers else synth.dense_bf16
    d = gen(seed=570 + rows, B=1, S=rows, Hq=1, Hkv=1)
    signs = synth.hadamard_signs(571 + rows)
    log(f"quantize fp8 rotated rows={rows} outliers={outliers}")
    codes, scales = lcat.attn_quantize_fp8_blocks(to_dev(d["k"]), signs=signs)
    torch.cuda.synchronize()
    want_c, want_e = ofp8.quantize_rotated_rows(d["k"], signs)
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)
    np.testing.assert_array_equal(scales.cpu().numpy(), ofp8.e8m0_bytes(want_e))


@pytest.mark.parametrize("S,B,Hq,Hkv,causal,outliers", [
    (300, 2, 16, 2, True, True), (640, 1, 16, 2, False, True), (200, 1, 8, 8, True, False),
    (1100, 1, 16, 2, True, True), (1300, 1, 4, 4, True, True), (257, 1, 32, 2, False, True),
])
def test_prefill_fp8_rotated_vs_oracle(S, B, Hq, Hkv, causal, outliers):
    """FP8 scores with incoherent processing: every row against the oracle
    over the rotated, dequantised Q and K."""
    log(f"prefill fp8 rotated S={S} B={B} Hq={Hq} Hkv={Hkv} causal={causal} outliers={outliers}")
    gen = synth.dense_bf16_outliers if outliers else synth.dense_bf16
    d = gen(seed=580 + S, B=B, S=S, Hq=Hq, Hkv=Hkv)
    signs = synth.hadamard_signs(581 + S)
    k8, ks = lcat.attn_quantize_fp8_blocks(to_dev(d["k"]), signs=signs)
    o, lse = lcat.attn_prefill_fp8(to_dev(d["q"]), k8, ks, to_dev(d["v"]), causal=causal,
                                   scale=d["scale"], signs=signs)
    torch.cuda.synchronize()
    ref, ref_lse = ofp8.attention_fp8(d["q"], d["k"], d["v"], d["scale"], causal=causal, signs=signs)
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse,
                                  what="prefill fp8 rotated")
    log(f"  max abs {e:.3g} rel-L2 {r:.3g}")


def test_rotation_lowers_gpu_fp8_error_on_outlier_channels():
    """Both FP8 prefills on inputs with outlier channels in Q and K: with the
    rotation their outputs are at least 1.6 times closer (relative L2) to
    exact attention of the bf16 inputs than without it."""
    S = 2048
    d = synth.dense_bf16_outliers(seed=590, B=1, S=S, Hq=16, Hkv=2)
    signs = synth.hadamard_signs(591)
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    rows = synth.sample_rows(592, S, 256, [0, S - 1])
    ref, _ = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    v8t, vs = lcat.attn_quantize_fp8_v(v)
    errs = {}
    for sg in (None, signs):
        k8, ks = lcat.attn_quantize_fp8_blocks(k, signs=sg)
        o8, _ = lcat.attn_prefill_fp8(q, k8, ks, v, causal=True, scale=d["scale"], signs=sg)
        opv, _ = lcat.attn_prefill_fp8_pv(q, k8, ks, v8t, vs, causal=True, scale=d["scale"],
                                          signs=sg)
        torch.cuda.synchronize()
        for name, o in (("fp8", o8), ("fp8_pv", opv)):
            got = to_np64(o[:, sel])
            errs[name, sg is not None] = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    for name in ("fp8", "fp8_pv"):
        log(f"  {name}: rel-L2 against exact {errs[name, False]:.4f} plain, "
            f"{errs[name, True]:.4f} rotated")
        assert errs[name, False] > 1.6 * errs[name, True], (name, errs)


def test_prefill_fp8_32k_causal_sampled():
    """The 32K causal GQA shape (16 Q / 2 KV heads) on the seeded N(0,1)
    inputs themselves (RoPE has its own tests; the FP8 codes depend on the
    exact bf16 bits, so both sides take the same ones): 512 seeded rows per
    head plus the forced rows against the oracle over the dequantised
    operands; the error of the FP8 scores against exact attention is logged
    for the record."""
    S = 32768
    log("fp8 32K: generating inputs")
    d = synth.causal_gqa(seed=2, S=S)
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    k8, ks = lcat.attn_quantize_fp8_blocks(k)
    o, lse = lcat.attn_prefill_fp8(q, k8, ks, v, causal=True)
    torch.cuda.synchronize()
    rows = synth.sample_rows(23, S, 512, [0, 1, 31, 32, 63, 64, 65, 127, 128, S // 2, S - 2, S - 1])
    log(f"fp8 32K: oracle on {rows.size} rows x 16 heads")
    ref, ref_lse = ofp8.attention_fp8(d["q"], d["k"], d["v"], d["scale"], causal=True, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    got = to_np64(o[:, idx])
    e, r = assert_attention_close(got, ref, lse[:, :, idx].cpu().numpy(), ref_lse, what="fp8 32K")
    log(f"fp8 32K: max abs {e:.3g} rel-L2 {r:.3g} against the FP8 oracle")
    exact, _ = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True, rows=rows)
    dev = np.abs(got - exact)
    log(f"fp8 32K: against exact attention: max abs {dev.max():.3g}, "
        f"rel-L2 {np.linalg.norm(dev) / np.linalg.norm(exact):.3g}")
