"""Entry points captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library issues only kernel launches on the caller's stream (no
allocation, no memset, no synchronisation), so a serving loop can capture a
decode step, or a prefill step, once and replay it.  Each test replays its
graph several times with new inputs copied into the captured buffers and
eager work and synchronisations between the replays, and checks every
replay bit for bit against the same calls made eagerly on the same inputs
(same kernels, same inputs: identical bits), and the last replay against the
fp64 oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_attention_close, bits, log, to_dev, to_np64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lcat = pytest.importorskip("long_context_attention_tiled_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lcat.load_library()


def _capture(fn):
    """fn once on a side stream (warm-up, as torch's recipe asks), then captured."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _same_f32(a, b):
    return np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


def test_decode_graph_replays_match_eager():
    """Three decode calls in one graph (three layers of a decode step): the
    bf16 cache with a workspace, its FP8 copy, and the bf16 cache again
    through attn_decode_noalloc (the entry point for callers that capture
    graphs and cannot allocate), replayed with a new query each time."""
    ctx = [1, 65, 1000, 4097, 20000]
    c = synth.decode_cache(seed=710, B=len(ctx), ctx_lens=ctx, Hq=16, Hkv=2, extra_blocks=2)
    q, k_pool, v_pool, head, table, ctx_len = (
        to_dev(c[k]) for k in ("q", "k_pool", "v_pool", "block_head", "block_table", "ctx_len"))
    k8, v8, ks, vs = lcat.attn_kv_quantize_fp8(k_pool, v_pool)
    B, Hq = c["q"].shape[:2]
    ws = torch.empty(lcat.attn_decode_workspace_bytes(B, Hq, c["max_blocks"]), dtype=torch.uint8,
                     device="cuda")
    ws8 = torch.empty_like(ws)
    o, o8, on = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    lse8, lsen = torch.empty_like(lse), torch.empty_like(lse)

    def step():
        lcat.attn_decode(q, k_pool, v_pool, head, table, ctx_len, workspace=ws, o=o, lse=lse)
        lcat.attn_decode_fp8(q, k8, v8, ks, vs, head, table, ctx_len, workspace=ws8, o=o8,
                             lse=lse8)
        lcat.attn_decode_noalloc(q, k_pool, v_pool, head, table, ctx_len, o=on, lse=lsen)

    g = _capture(step)
    for rep in range(4):
        log(f"decode graph replay {rep}: ctx={ctx}")
        qn = synth.normal_bf16(720 + rep, tuple(q.shape))
        q.copy_(to_dev(qn))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, o8, lse8, on, lsen)]
        eo, el = lcat.attn_decode(q, k_pool, v_pool, head, table, ctx_len)
        eo8, el8 = lcat.attn_decode_fp8(q, k8, v8, ks, vs, head, table, ctx_len)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got[0]), bits(eo)) and _same_f32(got[1], el)
        assert np.array_equal(bits(got[2]), bits(eo8)) and _same_f32(got[3], el8)
        assert np.array_equal(bits(got[4]), bits(eo)) and _same_f32(got[5], el)
    ref, ref_lse = oracle.decode_attention(qn, c["k_seq"], c["v_seq"], c["ctx_len"],
                                           c["scale"])
    assert_attention_close(to_np64(got[0]), ref, got[1].cpu().numpy(), ref_lse)


def test_prefill_step_graph_replays_match_eager():
    """The prefill step (fresh Q and K copied in, RoPE of Q and K in one
    launch, causal GQA prefill) captured once and replayed on new inputs."""
    S, Hq, Hkv = 700, 16, 2
    d = synth.dense_bf16(seed=730, B=1, S=S, Hq=Hq, Hkv=Hkv)
    q0, k0, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    pos = to_dev(d["positions"])
    q, k = torch.empty_like(q0), torch.empty_like(k0)
    o = torch.empty_like(q0)
    lse = torch.empty((1, Hq, S), dtype=torch.float32, device="cuda")

    def step():
        q.copy_(q0)
        k.copy_(k0)
        lcat.rope_apply_qk(q[0], k[0], pos)
        lcat.attn_prefill(q, k, v, causal=True, o=o, lse=lse)

    g = _capture(step)
    for rep in range(3):
        log(f"prefill graph replay {rep}: S={S}")
        dn = synth.dense_bf16(seed=740 + rep, B=1, S=S, Hq=Hq, Hkv=Hkv)
        q0.copy_(to_dev(dn["q"]))
        k0.copy_(to_dev(dn["k"]))
        v.copy_(to_dev(dn["v"]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = o.clone(), lse.clone()
        qe, ke = q0.clone(), k0.clone()
        lcat.rope_apply_qk(qe[0], ke[0], pos)
        eo, el = lcat.attn_prefill(qe, ke, v, causal=True)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got_o), bits(eo)) and _same_f32(got_l, el)
    qr = oracle.rope(dn["q"][0], dn["positions"])[None]
    kr = oracle.rope(dn["k"][0], dn["positions"])[None]
    ref, ref_lse = oracle.attention(qr, kr, oracle.widen(dn["v"]), dn["scale"], causal=True)
    assert_attention_close(to_np64(got_o), ref, got_l.cpu().numpy(), ref_lse)
