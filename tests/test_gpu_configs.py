"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.

* causal GQA prefill with RoPE, 1 x 32768 tokens, 16 Q / 2 KV heads, D=128;
* sequence-shard input [4][16384][64 heads][128] relayed out to one rank's
  [65536][16][128] (bit-exact against the oracle relayout), RoPE at global
  positions 0..65535, causal prefill; the same relayout with RoPE fused in,
  and the reverse relayout of the output;
* split-K decode of 32 requests with contexts uniform in [8192, 131072] over
  a shuffled, NaN-poisoned paged cache (every output row checked);
* chunked prefill of 4 x 131072 tokens in 8192-token chunks against the
  growing paged cache;
* one rank of zigzag context parallelism (4 ranks) over 65536 tokens: its
  queries against every rank's key shard, merged by LSE.

Large outputs are compared on a seeded sample of >= 512 query rows per head
plus forced rows (first/last, tile edges, shard and chunk boundaries); the
fp64 oracle evaluates exactly those rows.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_attention_close, bits, log, to_dev, to_np64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")
lcat = pytest.importorskip("long_context_attention_tiled_amd")

N_SAMPLE = 512


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lcat.load_library()


def prefill_reference(q, k, v, positions, rows, scale, base=10000.0):
    """Oracle rows of causal attention after fp64 RoPE of the raw bf16 inputs."""
    qr = oracle.rope(q[0, rows], positions[rows], base)[None]      # [1][R][Hq][D]
    kr = oracle.rope(k[0], positions, base)[None]                    # [1][S][Hkv][D]
    lim = (rows + 1)[None, :]
    return oracle.attention_rows(qr, kr, oracle.widen(v), lim, scale)


def forced_rows(S, extra=()):
    base = [0, 1, 31, 32, 63, 64, 65, 127, 128, 255, 256, S // 2, S - 2, S - 1]
    return [r for r in list(base) + list(extra) if 0 <= r < S]


def test_causal_gqa_prefill_32k():
    S = 32768
    log("C2: generating inputs")
    d = synth.causal_gqa(seed=2, S=S)
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    pos = to_dev(d["positions"])
    log("C2: rope + prefill")
    lcat.rope_apply(q[0], pos)
    lcat.rope_apply(k[0], pos)
    o, lse = lcat.attn_prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    rows = synth.sample_rows(22, S, N_SAMPLE, forced_rows(S))
    log(f"C2: oracle on {rows.size} rows x 16 heads")
    ref, ref_lse = prefill_reference(d["q"], d["k"], d["v"], d["positions"].astype(np.int64),
                                     rows, d["scale"])
    got = to_np64(o[:, torch.from_numpy(rows).cuda()])
    got_lse = lse[:, :, torch.from_numpy(rows).cuda()].cpu().numpy()
    e, r = assert_attention_close(got, ref, got_lse, ref_lse, what="C2")
    log(f"C2: max abs {e:.3g} rel-L2 {r:.3g}")


def test_causal_prefill_131072_sampled():
    """The longest sequence the bench runs (a 131072-token request, as in the
    chunked workload) as one dense causal prefill with RoPE of Q and K in one
    launch: sampled rows against the oracle, including the first and last
    rows and rows at tile edges."""
    S = 131072
    log("S=131072: generating inputs")
    d = synth.causal_gqa(seed=8, S=S)
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    pos = to_dev(d["positions"])
    log("S=131072: rope + prefill")
    lcat.rope_apply_qk(q[0], k[0], pos)
    o, lse = lcat.attn_prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    rows = synth.sample_rows(23, S, 32, forced_rows(S, (S - 64, S - 65)))
    log(f"S=131072: oracle on {rows.size} rows x 16 heads")
    ref, ref_lse = prefill_reference(d["q"], d["k"], d["v"], d["positions"].astype(np.int64),
                                     rows, d["scale"])
    got = to_np64(o[:, torch.from_numpy(rows).cuda()])
    got_lse = lse[:, :, torch.from_numpy(rows).cuda()].cpu().numpy()
    e, r = assert_attention_close(got, ref, got_lse, ref_lse, what="S=131072")
    log(f"S=131072: max abs {e:.3g} rel-L2 {r:.3g}")


def test_ulysses_relayout_rope_prefill_64k():
    SP, S_loc = 4, 16384
    S = SP * S_loc
    log("C3: generating shard inputs")
    d = synth.ulysses_shards(seed=3, SP=SP, S_loc=S_loc)
    rank = 0
    qd = lcat.seq_to_head_permute(to_dev(d["q"]), rank)
    kd = lcat.seq_to_head_permute(to_dev(d["k"]), rank)
    vd = lcat.seq_to_head_permute(to_dev(d["v"]), rank)
    torch.cuda.synchronize()
    log("C3: relayout bit-exact check")
    q_p = oracle.permute(d["q"], rank)
    k_p = oracle.permute(d["k"], rank)
    v_p = oracle.permute(d["v"], rank)
    assert np.array_equal(bits(qd), q_p)
    assert np.array_equal(bits(kd), k_p)
    assert np.array_equal(bits(vd), v_p)
    gpos = d["shard_positions"].reshape(-1)          # global position of relayed token t
    assert np.array_equal(gpos, np.arange(S))
    log("C3: rope + prefill")
    posd = to_dev(gpos.astype(np.int32))
    lcat.rope_apply(qd, posd)
    lcat.rope_apply(kd, posd)
    o, lse = lcat.attn_prefill(qd[None], kd[None], vd[None], causal=True)
    torch.cuda.synchronize()
    boundaries = [S_loc * i + j for i in range(1, SP) for j in (-1, 0, 1)]
    rows = synth.sample_rows(33, S, N_SAMPLE, forced_rows(S, boundaries))
    log(f"C3: oracle on {rows.size} rows x 16 heads")
    ref, ref_lse = prefill_reference(q_p[None], k_p[None], v_p[None], gpos.astype(np.int64), rows,
                                     d["scale"])
    idx = torch.from_numpy(rows).cuda()
    e, r = assert_attention_close(to_np64(o[:, idx]), ref, lse[:, :, idx].cpu().numpy(), ref_lse,
                                  what="C3")
    log(f"C3: max abs {e:.3g} rel-L2 {r:.3g}")


def test_ulysses_all_ranks_equal_full_head_attention():
    """The one-GPU emulation of the sequence-parallel step: every rank r of
    SP=4 relays out its heads from the four sequence shards, applies RoPE at
    global positions and runs causal attention; the ranks' head slices, put
    side by side, must equal attention over the full 64-query-head /
    8-KV-head problem (oracle on sampled rows).  Ranks 0 and 2 take the
    separate relayout and RoPE kernels, ranks 1 and 3 the fused one."""
    SP, S_loc, Hq_tot, Hkv_tot = 4, 1024, 64, 8
    S = SP * S_loc
    d = synth.ulysses_shards(seed=930, SP=SP, S_loc=S_loc, Hq_tot=Hq_tot, Hkv_tot=Hkv_tot)
    gpos = d["shard_positions"].reshape(-1)
    posd = to_dev(gpos.astype(np.int32))
    qs, ks, vs = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    o_full = torch.empty((1, S, Hq_tot, 128), dtype=torch.bfloat16, device="cuda")
    lse_full = torch.empty((1, Hq_tot, S), dtype=torch.float32, device="cuda")
    hq, hk = Hq_tot // SP, Hkv_tot // SP
    for r in range(SP):
        log(f"ulysses emulation: rank {r}")
        if r % 2 == 0:
            qd, kd, vd = lcat.seq_to_head_permute_qkv(qs, ks, vs, r)
            lcat.rope_apply(qd, posd)
            lcat.rope_apply(kd, posd)
        else:
            qd, kd, vd = lcat.seq_to_head_permute_qkv_rope(qs, ks, vs, r, posd)
        o, lse = lcat.attn_prefill(qd[None], kd[None], vd[None], causal=True)
        o_full[:, :, hq * r:hq * (r + 1)] = o
        lse_full[:, hq * r:hq * (r + 1)] = lse
    torch.cuda.synchronize()
    boundaries = [S_loc * i + j for i in range(1, SP) for j in (-1, 0, 1)]
    rows = synth.sample_rows(931, S, 128, forced_rows(S, boundaries))
    full = lambda x: x.reshape(1, S, x.shape[2], x.shape[3])     # shards in order = global order
    log(f"ulysses emulation: oracle on {rows.size} rows x {Hq_tot} heads")
    ref, ref_lse = prefill_reference(full(d["q"]), full(d["k"]), full(d["v"]),
                                     gpos.astype(np.int64), rows, d["scale"])
    idx = torch.from_numpy(rows).cuda()
    e, r_ = assert_attention_close(to_np64(o_full[:, idx]), ref, lse_full[:, :, idx].cpu().numpy(),
                                   ref_lse, what="Ulysses emulation")
    log(f"ulysses emulation: max abs {e:.3g} rel-L2 {r_:.3g}")


def test_ulysses_relayout_with_rope_64k():
    """The fused relayout + RoPE at the 64K shape the benchmark times: V bit
    for bit over the whole tensor, Q and K on sampled tokens (shard
    boundaries included) against the oracle's rotation of the oracle's
    relayout, and the whole output bit for bit equal to relayout followed by
    rope_apply."""
    SP, S_loc = 4, 16384
    S = SP * S_loc
    log("C3 fused: generating shard inputs")
    d = synth.ulysses_shards(seed=3, SP=SP, S_loc=S_loc)
    gpos = d["shard_positions"].reshape(-1)
    posd = to_dev(gpos.astype(np.int32))
    qin, kin, vin = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    qo, ko, vo = lcat.seq_to_head_permute_qkv_rope(qin, kin, vin, 0, posd)
    q2, k2, v2 = lcat.seq_to_head_permute_qkv(qin, kin, vin, 0)
    lcat.rope_apply(q2, posd)
    lcat.rope_apply(k2, posd)
    torch.cuda.synchronize()
    for a, b2 in ((qo, q2), (ko, k2), (vo, v2)):
        assert torch.equal(a.view(torch.int16), b2.view(torch.int16))
    assert np.array_equal(bits(vo), oracle.permute(d["v"], 0))
    toks = synth.sample_rows(34, S, N_SAMPLE, [S_loc * i + j for i in range(1, SP) for j in (-1, 0, 1)])
    log(f"C3 fused: oracle RoPE on {toks.size} tokens")
    for got, x in ((qo, d["q"]), (ko, d["k"])):
        ref = oracle.rope(oracle.permute(x, 0)[toks], gpos[toks])
        g = synth.bf16_bits_to_f32(bits(got)[toks]).astype(np.float64)
        assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-6)


def test_ulysses_output_relayout_64k():
    """The reverse exchange at the 64K shape: rank 0's output [65536][16][128]
    back to its head slice of [4][16384][64][128], bit for bit, on a seeded
    bf16 tensor of that shape; the other slices keep their prior contents."""
    SP, S_loc, H_tot = 4, 16384, 64
    x = synth.normal_bf16(36, (SP * S_loc, H_tot // SP, 128))
    prior = synth.normal_bf16(37, (SP, S_loc, H_tot, 128))
    out = to_dev(prior)
    log("C3 output relayout: rank 0")
    lcat.head_to_seq_permute(to_dev(x), SP, H_tot, 0, out=out)
    torch.cuda.synchronize()
    ref = prior.copy()
    oracle.unpermute(x, SP, H_tot, 0, out=ref)
    assert np.array_equal(bits(out), ref)


def run_cp_rank(q, k, v, S, N, rank, mode, accumulate):
    """One rank's ring attention on one GPU: shard, key limits from the
    positions, prefix-limited partials against every key shard, combined by
    the LSE merge kernel or merged in each partial's epilogue."""
    qr, qpos = lcat.cp_shard(q, N, rank, mode)
    o = lse = None
    for s_ in range(N):
        ks, kpos = lcat.cp_shard(k, N, s_, mode)
        vs, _ = lcat.cp_shard(v, N, s_, mode)
        lim = lcat.attn_key_limits(qpos, kpos)
        if accumulate:
            o, lse = lcat.attn_prefill_limited(qr[None], ks[None], vs[None], lim, o=o, lse=lse,
                                               accumulate=s_ > 0)
            continue
        op, lp = lcat.attn_prefill_limited(qr[None], ks[None], vs[None], lim)
        if o is None:
            o, lse = op, lp
        else:
            lcat.attn_merge(o, lse, op, lp, o=o, lse=lse)
    return o, lse


@pytest.mark.parametrize("rank,accumulate", [(0, False), (0, True), (3, True)])
def test_cp_zigzag_64k(rank, accumulate):
    S, N = 65536, 4
    log(f"CP zigzag 64K rank {rank}: generating")
    d = synth.dense_bf16(seed=920, B=1, S=S, Hq=16, Hkv=2)
    q, k, v = (to_dev(d[n][0]) for n in ("q", "k", "v"))
    o, lse = run_cp_rank(q, k, v, S, N, rank, "zigzag", accumulate)
    torch.cuda.synchronize()
    toks = oracle.cp_tokens(S, N, "zigzag", rank)
    L = toks.size // 2
    local = synth.sample_rows(921 + rank, toks.size, N_SAMPLE, [0, 1, L - 1, L, L + 1, 2 * L - 1])
    log(f"CP zigzag 64K rank {rank}: oracle on {local.size} rows x 16 heads")
    ref, ref_lse = oracle.attention(d["q"], d["k"], d["v"], d["scale"], causal=True, rows=toks[local])
    idx = torch.from_numpy(local).cuda()
    e, r = assert_attention_close(to_np64(o[:, idx]), ref, lse[:, :, idx].cpu().numpy(), ref_lse,
                                  what="CP zigzag")
    log(f"CP zigzag 64K rank {rank}: max abs {e:.3g} rel-L2 {r:.3g}")


def test_decode_paged_32_requests():
    log("C4: generating cache")
    c = synth.decode_cache(seed=4, B=32)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = [to_dev(c[k_]) for k_ in ("q", "k_pool", "v_pool", "block_head", "block_table", "ctx_len")]
    log(f"C4: decode, total context {int(c['ctx_len'].sum())} tokens")
    o, lse = lcat.attn_decode(*args, dev_status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    ref, ref_lse = oracle.decode_attention(c["q"], c["k_seq"], c["v_seq"], c["ctx_len"], c["scale"])
    e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse, what="C4")
    log(f"C4: max abs {e:.3g} rel-L2 {r:.3g}")


def test_decode_fp8_32_requests():
    """FP8-cache decode at the 32-request shape, in the launch configuration
    the benchmark times (equal-share split): seeded e4m3 codes (exponent
    fields 3..10, random signs) and per-token scales for every cached token,
    the NaN code and NaN scales in unused slots; every request (all 16
    heads, whole contexts) against the oracle over the dequantised cache."""
    from oracle import fp8 as ofp8
    log("C4 fp8: generating cache")
    c = synth.decode_cache(seed=4, B=32, with_content=False)
    n = c["n_blocks"]
    rng = np.random.default_rng(930)

    def codes(shape):
        e = rng.integers(3, 11, size=shape, dtype=np.uint8)
        m = rng.integers(0, 8, size=shape, dtype=np.uint8)
        sgn = rng.integers(0, 2, size=shape, dtype=np.uint8)
        return (sgn << 7) | (e << 3) | m

    k8, v8 = codes((n, 64, 128)), codes((n, 128, 64))
    ks = rng.uniform(0.02, 0.1, size=(n, 64)).astype(np.float32)
    vs = rng.uniform(0.02, 0.1, size=(n, 64)).astype(np.float32)
    valid = np.zeros((n, 64), dtype=bool)
    table = c["block_table"]
    for b, ctx in enumerate(c["ctx_len"]):
        nb = (int(ctx) + 63) // 64
        for g in range(table.shape[1]):
            valid[table[b, g, :nb - 1]] = True
            valid[table[b, g, nb - 1], : int(ctx) - 64 * (nb - 1)] = True
    k8[~valid] = 0x7F
    v8.transpose(0, 2, 1)[~valid] = 0x7F
    ks[~valid] = np.nan
    vs[~valid] = np.nan
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    log(f"C4 fp8: decode, total context {int(c['ctx_len'].sum())} tokens")
    o, lse = lcat.attn_decode_fp8(to_dev(c["q"]), torch.from_numpy(k8).cuda(),
                                  torch.from_numpy(v8).cuda(), to_dev(ks), to_dev(vs),
                                  to_dev(c["block_head"]), to_dev(table), to_dev(c["ctx_len"]),
                                  dev_status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    got, got_lse = to_np64(o), lse.cpu().numpy()
    log("C4 fp8: oracle on all 32 requests, one at a time")
    worst = (0.0, 0.0)
    for b in range(32):
        kq, vq = ofp8.gather_dequantized(k8, v8, ks, vs, table, c["ctx_len"], requests=[b])
        ref, ref_lse = oracle.decode_attention(c["q"][b:b + 1], kq, vq, c["ctx_len"][b:b + 1],
                                               c["scale"])
        e, r = assert_attention_close(got[b:b + 1], ref, got_lse[b:b + 1], ref_lse,
                                      what=f"C4 fp8 request {b}")
        worst = (max(worst[0], e), max(worst[1], r))
    log(f"C4 fp8: max abs {worst[0]:.3g} rel-L2 {worst[1]:.3g}")


def test_chunked_prefill_4x131072():
    B, S, C = 4, 131072, 8192
    log("C5: generating inputs")
    d = synth.chunked_prefill(seed=5, B=B, S=S, C=C)
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    n_blocks = d["n_blocks"]
    k_pool = torch.full((n_blocks, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.full((n_blocks, 128, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    tags, table = to_dev(d["block_head"]), to_dev(d["block_table"])
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, 16, S), dtype=torch.float32, device="cuda")
    log("C5: 16 chunk steps")
    for c0 in range(0, S, C):
        cb = torch.full((B,), c0, dtype=torch.int32, device="cuda")
        oc, lc = lcat.attn_chunked_prefill(q[:, c0:c0 + C].contiguous(), k[:, c0:c0 + C].contiguous(),
                                           v[:, c0:c0 + C].contiguous(), k_pool, v_pool, tags, table,
                                           cb, dev_status=st)
        o[:, c0:c0 + C] = oc
        lse[:, :, c0:c0 + C] = lc
    torch.cuda.synchronize()
    assert st.item() == 0
    # 512 seeded rows per request and head, plus every chunk boundary
    # 8192c-1 / 8192c in every request
    boundaries = [C * i + j for i in range(1, S // C) for j in (-1, 0)]
    for b in range(B):
        rows = synth.sample_rows(55 + b, S, N_SAMPLE, forced_rows(S, boundaries))
        idx = torch.from_numpy(rows).cuda()
        log(f"C5: oracle request {b}: {rows.size} rows x 16 heads")
        ref, ref_lse = oracle.attention(d["q"][b:b + 1], d["k"][b:b + 1], d["v"][b:b + 1],
                                        d["scale"], causal=True, rows=rows)
        e, r = assert_attention_close(to_np64(o[b:b + 1, idx]), ref,
                                      lse[b:b + 1, :, idx].cpu().numpy(), ref_lse, what=f"C5[{b}]")
        log(f"C5[{b}]: max abs {e:.3g} rel-L2 {r:.3g}")
    log("C5: cache read-back for request 0")
    kg, vg = oracle.paged_gather(bits(k_pool), bits(v_pool), d["block_table"][:1], [S])
    assert np.array_equal(kg[0], d["k"][0]) and np.array_equal(vg[0], d["v"][0])
