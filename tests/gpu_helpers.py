"""Helpers shared by the GPU parity tests (marshalling and comparisons only)."""
import sys

import numpy as np

BF16_ATOL = 2e-2
BF16_RTOL = 2e-2


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
                           rel_l2=2e-2, lse_tol=2e-2, what=""):
    """Elementwise |got-ref| <= atol + rtol|ref|, per-row relative L2 error and
    LSE error bounds.  Rows are the last axis (head dim)."""
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
        d = np.abs(np.asarray(got_lse, np.float64) - np.asarray(ref_lse, np.float64))
        assert d.max() <= lse_tol, f"{what}: LSE error {d.max():.3g}"
    return err.max(), rl2.max()
