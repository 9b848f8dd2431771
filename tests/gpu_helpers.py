"""Helpers shared by the GPU parity tests (marshalling and comparisons only)."""
import sys

import numpy as np

BF16_ATOL = 2e-2
BF16_RTOL = 2e-2
# LSE: |got - ref| <= 2e-2 + 2^-9 |ref|.  The bf16 prefill kernels multiply
# each query row by scale * log2(e) and round it to bf16 once, as they load
# it, so that the matrix cores produce the softmax exponents directly.  Every
# score q.k then carries a relative error of at most 2^-9 per product term,
# the size of the bf16 rounding the inputs themselves carry, and the LSE
# (a weighted mean of scores plus log l) moves by at most 2^-9 times the
# magnitude of the scores that hold the weight: about 1e-3 for N(0,1) data,
# about 0.2 for rows whose scores reach 200.  O is unaffected to first order
# (only score differences matter there).  The bar stays inside the allclose
# form of the bf16 tolerance, 2e-2 + 2e-2 |ref|.
BF16_LSE_ATOL = 2e-2
BF16_LSE_RTOL = 2.0 ** -9


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def to_np64(t):
    """GPU tensor -> float64 numpy (bf16 widened exactly)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def bits(t):
    """bf16 tensor -> uint16 numpy of its bit patterns."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_attention_close(got, ref, got_lse=None, ref_lse=None, atol=BF16_ATOL, rtol=BF16_RTOL,
                           rel_l2=2e-2, lse_tol=BF16_LSE_ATOL, lse_rtol=BF16_LSE_RTOL, what=""):
    """Elementwise |got-ref| <= atol + rtol|ref|, per-row relative L2 error and
    LSE error bounds (|dLSE| <= lse_tol + lse_rtol |LSE|).  Rows are the last
    axis (head dim)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {err.max():.3g}"
    num = np.linalg.norm((got - ref).reshape(-1, ref.shape[-1]), axis=-1)
    den = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=-1)
    rl2 = num / np.maximum(den, 1e-30)
    assert rl2.max() <= rel_l2, f"{what}: per-row relative L2 error {rl2.max():.3g}"
    if got_lse is not None:
        r_lse = np.asarray(ref_lse, np.float64)
        d = np.abs(np.asarray(got_lse, np.float64) - r_lse)
        ok = d <= lse_tol + lse_rtol * np.abs(np.where(np.isfinite(r_lse), r_lse, 0.0))
        assert ok.all(), f"{what}: LSE error {d.max():.3g} (at |LSE| {np.abs(r_lse).max():.3g})"
    return err.max(), rl2.max()
