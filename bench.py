"""Throughput of the exact-attention hot path on one MI355X.

Step (the timed unit): one pass of the causal GQA prefill workload —
RoPE at absolute positions on Q and K, then causal attention — for batch 1,
sequence 32768, 16 query heads / 2 KV heads, head_dim 128, bf16 inputs.
``value`` is the algorithmic attention FLOP rate of that step (QK^T and PV
over the unmasked causal pairs only: 4*D*Hq*S*(S+1)/2 FLOP).

The same JSON line also carries, each measured in this run:
  roofline        the prefill kernel's average duration from HIP events on
                  its stream, against the bf16 dense MFMA peak;
  mfma_sustained  the bf16 MFMA rate this device sustains on random operands
                  held in registers (no memory or LDS traffic), the most any
                  bf16 matrix kernel reaches here, and (a_from_lds) the rate
                  when each MFMA's A operand is read from LDS, as the
                  attention kernels read K and V; the prefill kernel's rate
                  is also given as a fraction of both (frac_of_sustained,
                  frac_of_sustained_lds);
  decode          paged decode with the key blocks of all requests shared out
                  equally over the GPU's waves, 32 requests with contexts
                  uniform in [8192, 131072], KV bytes per second against 8 TB/s
                  and against a plain streaming read of as many bytes
                  (read_sustained); and (fp8_cache) the same decode over the
                  FP8 copy of the cache, against a streaming read of its own
                  (smaller) byte count;
  relayout        sequence-shard -> head-shard relayout of one rank's share of
                  [4][16384][64|8][128] bf16 Q/K/V (one launch), bytes per second,
                  also against a plain streaming copy of as many bytes
                  (copy_sustained), and (fused_rope) the same relayout with
                  RoPE on Q and K;
  relayout_back   the reverse exchange: that rank's attention output
                  [65536][16][128] back to its head slice of the shards;
  rope            rope_apply on the step's Q and K with cold buffers, against
                  an in-place copy of the same bytes;
  prefill_fp8     the step with FP8 scores (K block-quantised, QK^T on the
                  scaled FP8 matrix cores, P V in bf16), against the fp8 peak
                  and next to the bf16 kernel on the same inputs, and
                  (fp8_pv) with P V on FP8 as well (V block-quantised along
                  keys);
  prefill_64k     the relayout + RoPE + causal prefill pipeline at 65536,
                  with separate and with fused relayout + RoPE;
  chunked_prefill 4 requests x 131072 tokens in 8192-token chunks;
  cp_zigzag_64k   one rank of zigzag context parallelism (4 ranks, 65536
                  tokens): partials against every key shard, merged by LSE;
  cpu_baseline    the fp64 CPU oracle timed on a bounded sample of query rows
                  of the step workload, on this host's cores.
The decode and relayout times are means over calls enqueued back to back;
the relayouts cycle through 4 separate buffer sets so that no call reads data
an earlier call left in the last-level cache (the decode reads 2.35 GB per
call, far more than that cache holds).

Inputs are seeded synthetic N(0,1) data resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn prefill TFLOP/s (% MFMA peak) + decode KV GB/s (% HBM peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
D = 128

# Seeds of every synthetic input (numpy SeedSequence for synth's generators,
# torch.Generator for tensors drawn on the GPU).
SEEDS = {
    "tiny_fp32": 1,                       # synth.tiny_exact
    "causal_gqa_32k": 2,                  # synth.causal_gqa
    "decode_32req": 4,                    # synth.decode_cache (lengths, tables, q)
    "decode_pools": [41, 42],             # torch: K pool, V pool
    "relayout_64k": [31, 32, 33],         # torch: Q, K, V of buffer set r (+10 r)
    "chunked_4x131072": [51, 52, 53],     # torch: Q, K, V
    "cp_zigzag_64k": [61, 62, 63],        # torch: Q, K, V
    "cpu_sample_rows": 77,                # synth.sample_rows
    "hadamard_signs": 93,                 # synth.hadamard_signs (FP8 incoherent processing)
    "fp8_outliers": 94,                   # synth.dense_bf16_outliers
    "decode_graph": 95,                   # synth.decode_cache (q); torch pools 200 + 2 l, 201 + 2 l
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def causal_flops(B, S, Hq, D=D, ctx_before=0):
    """QK^T + PV FLOPs over visible pairs: row i sees ctx_before + i + 1 keys."""
    pairs = S * ctx_before + S * (S + 1) // 2
    return 4.0 * D * Hq * B * pairs


# The source file that defines each kernel whose traffic is recorded.
KERNEL_SOURCES = {
    "prefill_kernel": "prefill_bf16.hip",
    "permute16_kernel": "permute.hip",
    "permute_rope_kernel": "relayout_rope.hip",
    "rope_kernel": "rope.hip",
    "decode_stream_kernel": "decode.hip",
}


def kernel_source_hash(kernel):
    """sha256 (first 16 hex digits) over the source file that defines
    `kernel`, every local header it includes (transitively) and the compile
    flags: a change anywhere else leaves the kernel's recorded traffic valid."""
    import re
    from long_context_attention_tiled_amd import _build
    csrc = os.path.join(ROOT, "long_context_attention_tiled_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    seen, todo = set(), [os.path.join(csrc, KERNEL_SOURCES[kernel])]
    while todo:
        path = os.path.normpath(todo.pop())
        if path in seen:
            continue
        seen.add(path)
        with open(path) as f:
            for name in re.findall(r'^#include "([^"]+)"', f.read(), re.M):
                for d in (os.path.dirname(path), csrc, inc):
                    cand = os.path.normpath(os.path.join(d, name))
                    if os.path.exists(cand):
                        todo.append(cand)
                        break
    h = hashlib.sha256()
    for path in sorted(seen):
        with open(path, "rb") as f:
            h.update(os.path.relpath(path, ROOT).encode() + b"\0" + f.read() + b"\0")
    h.update(" ".join(_build.HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """Measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled
    by a copy-kernel calibration) if recorded for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel, {}).get(workload)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


class EventTimer:
    """Average duration of one launch site, from HIP events on the stream the
    kernels are enqueued on (the current torch stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        self.s = self.torch.cuda.Event(enable_timing=True)
        self.e = self.torch.cuda.Event(enable_timing=True)
        self.s.record()
        return self

    def __exit__(self, *a):
        self.e.record()
        self.pairs.append((self.s, self.e))

    def times_ms(self):
        return [s.elapsed_time(e) for s, e in self.pairs]

    def mean_ms(self):
        return float(np.mean(self.times_ms()))


def back_to_back_ms(torch, fn, iters):
    """Mean GPU time of ``fn`` over ``iters`` calls enqueued back to back
    between one pair of events (one untimed call first keeps the stream busy,
    so host-side launch latency does not enter the measurement)."""
    fn()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def dev_tensor(torch, a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def seeded_normal_bf16(torch, shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


# ---------------------------------------------------------------------------
def bench_step(torch, lcat, synth, steps, warmup):
    """The timed step.  RoPE rotates Q and K in place, so every step (warm-up
    included) runs on its own copy of the unrotated inputs, staged in HBM
    before timing starts (144 MB per step): each timed step is the
    configured workload, not a re-rotation of the previous step's output."""
    S, Hq, Hkv = 32768, 16, 2
    d = synth.causal_gqa(seed=SEEDS["causal_gqa_32k"], S=S, Hq=Hq, Hkv=Hkv)
    q0, k0, v = dev_tensor(torch, d["q"]), dev_tensor(torch, d["k"]), dev_tensor(torch, d["v"])
    pos = dev_tensor(torch, d["positions"])
    n = warmup + steps
    qs = [q0.clone() for _ in range(n)]
    ks = [k0.clone() for _ in range(n)]
    del q0, k0
    o = torch.empty_like(qs[0])
    lse = torch.empty((1, Hq, S), dtype=torch.float32, device="cuda")
    timer = EventTimer(torch)

    def step(i, time_kernel):
        q, k = qs[i], ks[i]
        lcat.rope_apply_qk(q[0], k[0], pos)
        if time_kernel:
            with timer:
                lcat.attn_prefill(q, k, v, causal=True, o=o, lse=lse)
        else:
            lcat.attn_prefill(q, k, v, causal=True, o=o, lse=lse)

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, n):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del qs, ks
    flops = causal_flops(1, S, Hq)
    ms_step = wall * 1e3 / steps
    k_ms = timer.mean_ms()
    achieved = flops / (k_ms * 1e-3) / 1e12
    traffic = load_traffic("prefill_kernel", "causal_gqa_32k")
    check = dict(d=d, o=o, lse=lse)
    return check, dict(
        value=flops / (wall / steps) / 1e12, ms_per_step=ms_step,
        roofline=dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4),
                      traffic=traffic, kernel="prefill_kernel<dense,causal>",
                      kernel_ms=round(k_ms, 4), kernel_ms_median=round(float(np.median(timer.times_ms())), 4),
                      kernel_ms_min=round(float(np.min(timer.times_ms())), 4), flop_per_launch=flops,
                      timed_launches=f"prefill launches {warmup + 1}..{n} of this process "
                                     f"(the first {warmup} are warm-up)"))


def bench_mfma_rate(torch, lcat, reps=3, n_wg=1024, iters=65536):
    out = torch.empty(n_wg * 512, dtype=torch.float32, device="cuda")
    res = {}
    for lds in (False, True):
        lcat.measure_mfma_rate(n_wg, iters, a_from_lds=lds, out=out)   # warm-up: clocks settle
        torch.cuda.synchronize()
        timer = EventTimer(torch)
        for r in range(reps):
            with timer:
                lcat.measure_mfma_rate(n_wg, iters, seed=r + 2, a_from_lds=lds, out=out)
        torch.cuda.synchronize()
        ms = timer.mean_ms()
        tflops = lcat.mfma_rate_flops(n_wg, iters) / (ms * 1e-3) / 1e12
        res[lds] = dict(tflops=round(tflops, 1), frac_of_peak=round(tflops / PEAK_BF16_TFLOPS, 4),
                        ms_per_launch=round(ms, 3))
    out_d = dict(res[False],
                 kernel="mfma_rate_kernel: v_mfma_f32_32x32x16_bf16, 4 chains x 2 waves per SIMD, "
                        "uniform random bf16 operands in [-1, 1) from registers",
                 launch=f"{n_wg} workgroups x 8 waves, {4 * iters} MFMA per wave")
    out_d["a_from_lds"] = dict(res[True],
                               kernel="mfma_lds_rate_kernel: the same, with each MFMA's A "
                                      "operand read from LDS (16 B per lane) just before it")
    return out_d


def bench_decode(torch, lcat, synth, iters=20):
    c = synth.decode_cache(seed=SEEDS["decode_32req"], B=32, with_content=False)
    n_blocks = c["n_blocks"]
    k_pool = seeded_normal_bf16(torch, (n_blocks, 64, D), SEEDS["decode_pools"][0])
    v_pool = seeded_normal_bf16(torch, (n_blocks, D, 64), SEEDS["decode_pools"][1])
    args = [dev_tensor(torch, c["q"]), k_pool, v_pool, dev_tensor(torch, c["block_head"]),
            dev_tensor(torch, c["block_table"]), dev_tensor(torch, c["ctx_len"])]
    B, Hq = c["q"].shape[:2]
    ws = torch.empty(lcat.attn_decode_workspace_bytes(B, Hq, c["max_blocks"]), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    for _ in range(3):
        lcat.attn_decode(*args, workspace=ws, o=o, lse=lse)
    torch.cuda.synchronize()
    ms = back_to_back_ms(torch, lambda: lcat.attn_decode(*args, workspace=ws, o=o, lse=lse), iters)
    ctx_total = int(c["ctx_len"].sum())
    nbytes = ctx_total * c["Hkv"] * D * 2 * 2 + 2 * B * Hq * D * 2 + B * Hq * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = dict(ms=round(ms, 4), GBps=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4),
               bytes=nbytes, context_tokens=ctx_total, requests=B,
               traffic=load_traffic("decode_stream_kernel", "decode_32req_bf16"),
               workload="32 requests, ctx U[8192,131072], 16 Q / 2 KV heads, paged 64-token blocks")

    # yardstick: a plain streaming read of the same number of bytes
    buf = torch.empty(nbytes // 16 * 16, dtype=torch.uint8, device="cuda")
    rd_out, rd_bytes = lcat.measure_hbm_read(buf)
    torch.cuda.synchronize()
    ms_rd = back_to_back_ms(torch, lambda: lcat.measure_hbm_read(buf, out=rd_out), iters)
    del buf
    rd_gbs = rd_bytes / (ms_rd * 1e-3) / 1e9
    res["read_sustained"] = dict(GBps=round(rd_gbs, 1), frac_hbm=round(rd_gbs / PEAK_HBM_GBS, 4),
                                 bytes=rd_bytes,
                                 kernel="hbm_read_kernel: 4096 waves, contiguous shares, "
                                        "32 x 16-byte loads per lane in flight")
    res["frac_of_sustained_read"] = round(gbs / rd_gbs, 4)

    # the same cache in FP8 (e4m3 + one fp32 scale per token for K and for V)
    k8, v8, ks, vs = lcat.attn_kv_quantize_fp8(k_pool, v_pool)
    args8 = [args[0], k8, v8, ks, vs] + args[3:]
    o8, lse8 = torch.empty_like(o), torch.empty_like(lse)
    for _ in range(3):
        lcat.attn_decode_fp8(*args8, workspace=ws, o=o8, lse=lse8)
    torch.cuda.synchronize()
    ms8 = back_to_back_ms(torch, lambda: lcat.attn_decode_fp8(*args8, workspace=ws, o=o8, lse=lse8),
                          iters)
    nbytes8 = ctx_total * c["Hkv"] * (2 * D + 8) + 2 * B * Hq * D * 2 + B * Hq * 4
    gbs8 = nbytes8 / (ms8 * 1e-3) / 1e9
    del k8, v8, ks, vs
    # its own yardstick: a streaming read of the FP8 decode's byte count
    buf = torch.empty(nbytes8 // 16 * 16, dtype=torch.uint8, device="cuda")
    rd8_out, rd8_bytes = lcat.measure_hbm_read(buf)
    torch.cuda.synchronize()
    ms_rd8 = back_to_back_ms(torch, lambda: lcat.measure_hbm_read(buf, out=rd8_out), iters)
    del buf
    rd8_gbs = rd8_bytes / (ms_rd8 * 1e-3) / 1e9
    res["fp8_cache"] = dict(ms=round(ms8, 4), GBps=round(gbs8, 1),
                            frac_hbm=round(gbs8 / PEAK_HBM_GBS, 4), bytes=nbytes8,
                            traffic=load_traffic("decode_stream_kernel", "decode_32req_fp8"),
                            read_sustained=dict(GBps=round(rd8_gbs, 1),
                                                frac_hbm=round(rd8_gbs / PEAK_HBM_GBS, 4),
                                                bytes=rd8_bytes),
                            frac_of_sustained_read=round(gbs8 / rd8_gbs, 4),
                            frac_of_bf16_bytes_read=round(gbs8 / rd_gbs, 4),
                            speedup_vs_bf16=round(ms / ms8, 3))
    check = dict(c=c, q=args[0], k_pool=k_pool, v_pool=v_pool, o=o, lse=lse)
    return check, res


def rotating(fns):
    """One call per invocation, cycling through ``fns``."""
    it = [0]

    def call():
        fns[it[0] % len(fns)]()
        it[0] += 1
    return call


def bench_relayout_and_prefill_64k(torch, lcat, iters=20, n_sets=4):
    """The relayouts and the copy yardstick cycle through ``n_sets`` separate
    input/output sets (1.25 GiB of inputs each), so no call finds its data in
    the 256 MB last-level cache from an earlier call: the rates are HBM rates."""
    SP, S_loc, Hq_tot, Hkv_tot = 4, 16384, 64, 8
    S = SP * S_loc
    sets = []
    for r in range(n_sets):
        sq, sk, sv = (x + 10 * r for x in SEEDS["relayout_64k"])
        qin = seeded_normal_bf16(torch, (SP, S_loc, Hq_tot, D), sq)
        kin = seeded_normal_bf16(torch, (SP, S_loc, Hkv_tot, D), sk)
        vin = seeded_normal_bf16(torch, (SP, S_loc, Hkv_tot, D), sv)
        qo = torch.empty((S, Hq_tot // SP, D), dtype=torch.bfloat16, device="cuda")
        ko = torch.empty((S, Hkv_tot // SP, D), dtype=torch.bfloat16, device="cuda")
        vo = torch.empty_like(ko)
        back = torch.zeros((SP, S_loc, Hq_tot, D), dtype=torch.bfloat16, device="cuda")
        sets.append((qin, kin, vin, qo, ko, vo, back))
    qin, kin, vin, qo, ko, vo, _ = sets[0]

    def relayout(st=sets[0]):   # Q, K and V of rank 0 in one launch
        lcat.seq_to_head_permute_qkv(st[0], st[1], st[2], 0, outs=(st[3], st[4], st[5]))

    relayout_all = rotating([lambda st=st: relayout(st) for st in sets])
    for _ in range(n_sets):
        relayout_all()
    torch.cuda.synchronize()
    ms = back_to_back_ms(torch, relayout_all, iters)
    nbytes = 2 * (qo.numel() + ko.numel() + vo.numel()) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    relay = dict(ms=round(ms, 4), GBps=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4),
                 bytes=nbytes, traffic=load_traffic("permute16_kernel", "relayout_qkv_64k"),
                 workload="rank 0 of [4][16384][64|8][128] bf16 Q/K/V",
                 buffer_sets=n_sets)

    # yardstick: a plain streaming copy moving the same bytes (half read, half written)
    pairs = [(st[0].view(-1)[: nbytes // 4], st[6].view(-1)[: nbytes // 4]) for st in sets]
    copy_all = rotating([lambda pr=pr: lcat.measure_hbm_copy(pr[0], pr[1]) for pr in pairs])
    for _ in range(n_sets):
        copy_all()
    torch.cuda.synchronize()
    ms_c = back_to_back_ms(torch, copy_all, iters)
    cp_gbs = nbytes / (ms_c * 1e-3) / 1e9
    relay["copy_sustained"] = dict(GBps=round(cp_gbs, 1), frac_hbm=round(cp_gbs / PEAK_HBM_GBS, 4),
                                   bytes=nbytes,
                                   kernel="hbm_copy_kernel: contiguous, 4 x 16 B per thread, "
                                          "non-temporal stores")
    relay["frac_of_sustained_copy"] = round(gbs / cp_gbs, 4)

    pos = torch.arange(S, dtype=torch.int32, device="cuda")

    def relayout_rope(st=sets[0]):   # the same relayout with RoPE on Q and K in the same pass
        lcat.seq_to_head_permute_qkv_rope(st[0], st[1], st[2], 0, pos, outs=(st[3], st[4], st[5]))

    rope_all = rotating([lambda st=st: relayout_rope(st) for st in sets])
    for _ in range(n_sets):
        rope_all()
    torch.cuda.synchronize()
    ms_r = back_to_back_ms(torch, rope_all, iters)
    gbs_r = nbytes / (ms_r * 1e-3) / 1e9
    relay["fused_rope"] = dict(ms=round(ms_r, 4), GBps=round(gbs_r, 1),
                               frac_hbm=round(gbs_r / PEAK_HBM_GBS, 4),
                               frac_of_sustained_copy=round(gbs_r / cp_gbs, 4))

    o = torch.empty((1, S, Hq_tot // SP, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, Hq_tot // SP, S), dtype=torch.float32, device="cuda")
    ptimer, ftimer, ktimer = EventTimer(torch), EventTimer(torch), EventTimer(torch)
    for it in range(4):
        with ptimer:   # relayout, then RoPE in place, then prefill
            relayout()
            lcat.rope_apply_qk(qo, ko, pos)
            with ktimer:
                lcat.attn_prefill(qo[None], ko[None], vo[None], causal=True, o=o, lse=lse)
        with ftimer:   # fused relayout + RoPE, then prefill
            relayout_rope()
            lcat.attn_prefill(qo[None], ko[None], vo[None], causal=True, o=o, lse=lse)
        if it == 0:
            torch.cuda.synchronize()
            for t in (ptimer, ftimer, ktimer):
                t.pairs.clear()
    torch.cuda.synchronize()
    flops = causal_flops(1, S, Hq_tot // SP)
    kms = ktimer.mean_ms()
    pre = dict(pipeline_ms=round(ptimer.mean_ms(), 3), pipeline_fused_ms=round(ftimer.mean_ms(), 3),
               kernel_ms=round(kms, 3), TFLOPs=round(flops / (kms * 1e-3) / 1e12, 1),
               frac_mfma=round(flops / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               workload="relayout + RoPE + causal prefill, seq 65536, 16 Q / 2 KV heads")

    # the reverse exchange: rank 0's output [S][16][D] back to its head slice
    # of the shards (set 0's input is the prefill output, the others stand in
    # with the same shape)
    outs = [o[0]] + [st[3] for st in sets[1:]]
    back_all = rotating([lambda x=x, st=st: lcat.head_to_seq_permute(x, SP, Hq_tot, 0, out=st[6])
                         for x, st in zip(outs, sets)])
    for _ in range(n_sets):
        back_all()
    torch.cuda.synchronize()
    ms_b = back_to_back_ms(torch, back_all, iters)
    nb = 2 * o[0].numel() * 2
    gbs_b = nb / (ms_b * 1e-3) / 1e9
    relay_back = dict(ms=round(ms_b, 4), GBps=round(gbs_b, 1), frac_hbm=round(gbs_b / PEAK_HBM_GBS, 4),
                      frac_of_sustained_copy=round(gbs_b / cp_gbs, 4), buffer_sets=n_sets,
                      bytes=nb, workload="rank 0's O [65536][16][128] bf16 -> [4][16384][64][128]")
    # o and lse are the prefill of set 0 after the fused relayout + RoPE of rank 0
    check = dict(qin=sets[0][0], kin=sets[0][1], vin=sets[0][2], o=o, lse=lse, SP=SP)
    return check, (relay, pre, relay_back)


PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 (e4m3) MFMA


def bench_fp8_prefill(torch, lcat, synth, reps=10, warmup=5):
    """The step workload with FP8 scores: RoPE on Q and K, block quantisation
    of K (attn_quantize_fp8_blocks), then attn_prefill_fp8 (Q quantised in the
    kernel, S = QK^T on the scaled FP8 matrix cores, P V in bf16).  The kernel
    is also timed next to the bf16 prefill on the same inputs, and the two
    outputs are compared (rel-L2 of the FP8 result against the bf16 one).
    ``fp8_pv``: the same rotated inputs with V block-quantised along keys
    (attn_quantize_fp8_v) through attn_prefill_fp8_pv (both products on FP8).
    ``incoherent``: attn_prefill_fp8_pv with Q and K rotated by the
    random-sign Hadamard matrix before quantisation, timed on the same
    inputs; and, on a 4096-token input with outlier channels in Q and K,
    each FP8 prefill's distance to the bf16 prefill with and without the
    rotation."""
    S, Hq, Hkv = 32768, 16, 2
    d = synth.causal_gqa(seed=SEEDS["causal_gqa_32k"], S=S, Hq=Hq, Hkv=Hkv)
    q0, k0, v = dev_tensor(torch, d["q"]), dev_tensor(torch, d["k"]), dev_tensor(torch, d["v"])
    pos = dev_tensor(torch, d["positions"])
    n = warmup + reps
    qs = [q0.clone() for _ in range(n)]
    ks = [k0.clone() for _ in range(n)]
    k8 = torch.empty(k0.shape, dtype=torch.uint8, device="cuda")
    ksc = torch.empty((*k0.shape[:-1], D // 32), dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(q0), torch.empty((1, Hq, S), dtype=torch.float32, device="cuda")
    step_t, kern_t, quant_t = EventTimer(torch), EventTimer(torch), EventTimer(torch)
    for i in range(n):   # the first `warmup` steps let the clock settle
        with step_t:
            lcat.rope_apply_qk(qs[i][0], ks[i][0], pos)
            with quant_t:
                lcat.attn_quantize_fp8_blocks(ks[i], k8, ksc)
            with kern_t:
                lcat.attn_prefill_fp8(qs[i], k8, ksc, v, causal=True, o=o, lse=lse)
        if i == warmup - 1:
            torch.cuda.synchronize()
            for t in (step_t, kern_t, quant_t):
                t.pairs.clear()
    torch.cuda.synchronize()
    flops = causal_flops(1, S, Hq)
    kms = kern_t.mean_ms()
    tf = flops / (kms * 1e-3) / 1e12
    # the same rotated inputs through the bf16 prefill, timed the same way
    ob = torch.empty_like(o)
    bf_t = EventTimer(torch)
    for i in range(n):
        with bf_t:
            lcat.attn_prefill(qs[-1], ks[-1], v, causal=True, o=ob)
        if i == warmup - 1:
            torch.cuda.synchronize()
            bf_t.pairs.clear()
    torch.cuda.synchronize()
    bms = bf_t.mean_ms()
    diff = (o.float() - ob.float()).norm().item() / ob.float().norm().item()
    # both products on FP8: V quantised along keys, then attn_prefill_fp8_pv
    s64 = (S + 63) // 64 * 64
    v8t = torch.empty((1, Hkv, D, s64), dtype=torch.uint8, device="cuda")
    vsc = torch.empty((1, Hkv, s64 // 64, 256), dtype=torch.uint8, device="cuda")
    op = torch.empty_like(o)
    pv_t, vq_t = EventTimer(torch), EventTimer(torch)
    # this kernel draws less power than the others and the clock keeps rising
    # over its first ~12 launches: three times the warm-up before timing
    for i in range(3 * warmup + reps):
        with vq_t:
            lcat.attn_quantize_fp8_v(v, v8t, vsc)
        with pv_t:
            lcat.attn_prefill_fp8_pv(qs[-1], k8, ksc, v8t, vsc, causal=True, o=op, lse=lse)
        if i == 3 * warmup - 1:
            torch.cuda.synchronize()
            pv_t.pairs.clear()
            vq_t.pairs.clear()
    torch.cuda.synchronize()
    pms = pv_t.mean_ms()
    ptf = flops / (pms * 1e-3) / 1e12
    pdiff = (op.float() - ob.float()).norm().item() / ob.float().norm().item()
    fp8_pv = dict(kernel_ms=round(pms, 4), TFLOPs=round(ptf, 1),
                  frac_fp8_peak=round(ptf / PEAK_FP8_TFLOPS, 4),
                  quantize_v_us=round(vq_t.mean_ms() * 1e3, 2),
                  speedup_vs_bf16_kernel=round(bms / pms, 3),
                  speedup_vs_fp8_scores_kernel=round(kms / pms, 3),
                  rel_l2_vs_bf16_kernel=round(pdiff, 5),
                  workload="the same inputs, V block-quantised along keys, both products on FP8")
    # incoherent processing: the same inputs with Q and K rotated
    signs = synth.hadamard_signs(SEEDS["hadamard_signs"])
    k8r, kscr = torch.empty_like(k8), torch.empty_like(ksc)
    lcat.attn_quantize_fp8_blocks(ks[-1], k8r, kscr, signs=signs)
    rot_t = EventTimer(torch)
    for i in range(3 * warmup + reps):
        with rot_t:
            lcat.attn_prefill_fp8_pv(qs[-1], k8r, kscr, v8t, vsc, causal=True, o=op, lse=lse,
                                     signs=signs)
        if i == 3 * warmup - 1:
            torch.cuda.synchronize()
            rot_t.pairs.clear()
    torch.cuda.synchronize()
    rms = rot_t.mean_ms()
    rdiff = (op.float() - ob.float()).norm().item() / ob.float().norm().item()
    # accuracy on outlier channels, against the bf16 prefill of the same input
    do = synth.dense_bf16_outliers(seed=SEEDS["fp8_outliers"], B=1, S=4096, Hq=Hq, Hkv=Hkv)
    qo, ko, vo = (dev_tensor(torch, do[x]) for x in ("q", "k", "v"))
    ref, _ = lcat.attn_prefill(qo, ko, vo, causal=True)
    vo8, vosc = lcat.attn_quantize_fp8_v(vo)
    acc = {}
    for tag, sg in (("plain", None), ("rotated", signs)):
        ko8, kosc = lcat.attn_quantize_fp8_blocks(ko, signs=sg)
        o8, _ = lcat.attn_prefill_fp8(qo, ko8, kosc, vo, causal=True, scale=do["scale"], signs=sg)
        opv, _ = lcat.attn_prefill_fp8_pv(qo, ko8, kosc, vo8, vosc, causal=True, scale=do["scale"],
                                          signs=sg)
        for name, out in (("fp8", o8), ("fp8_pv", opv)):
            acc[f"{name}_{tag}"] = round((out.float() - ref.float()).norm().item()
                                         / ref.float().norm().item(), 5)
    incoherent = dict(fp8_pv_kernel_ms=round(rms, 4),
                      fp8_pv_TFLOPs=round(flops / (rms * 1e-3) / 1e12, 1),
                      slowdown_vs_plain=round(rms / pms, 4),
                      fp8_pv_rel_l2_vs_bf16_kernel=round(rdiff, 5),
                      outliers_rel_l2_vs_bf16_kernel=acc,
                      outliers_workload="4096 tokens causal, 16 Q / 2 KV heads, 4 seeded head "
                                        "dims of Q x8 and of K x2 (synth.dense_bf16_outliers)")
    # QK^T at the fp8 peak plus P V at the bf16 peak
    mixed_peak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
    return dict(fp8_pv=fp8_pv, incoherent=incoherent, kernel_ms=round(kms, 4), TFLOPs=round(tf, 1),
                frac_fp8_peak=round(tf / PEAK_FP8_TFLOPS, 4),
                frac_mixed_peak=round(tf / mixed_peak, 4), mixed_peak_TFLOPs=round(mixed_peak, 1),
                step_ms=round(step_t.mean_ms(), 4), quantize_k_us=round(quant_t.mean_ms() * 1e3, 2),
                bf16_kernel_ms=round(bms, 4), speedup_vs_bf16_kernel=round(bms / kms, 3),
                rel_l2_vs_bf16_kernel=round(diff, 5),
                workload="causal GQA prefill, seq 32768, 16 Q / 2 KV heads: RoPE, K block "
                         "quantisation, FP8 scores with bf16 P V")


def bench_decode_graph(torch, lcat, synth, layers=32, iters=20):
    """A launch-bound decode step: 4 requests of 8192 cached tokens (16 Q /
    2 KV heads) through ``layers`` layers, each with its own paged cache
    (33.5 MB per layer), as ``layers`` attn_decode calls made from Python
    one after the other, against the same calls captured once in a HIP graph
    and replayed.  Wall time per step between synchronisations."""
    c = synth.decode_cache(seed=SEEDS["decode_graph"], B=4, ctx_lens=[8192] * 4,
                           with_content=False)
    n_blocks, B, Hq = c["n_blocks"], 4, 16
    q = dev_tensor(torch, c["q"])
    meta = [dev_tensor(torch, c[k]) for k in ("block_head", "block_table", "ctx_len")]
    pools = [(seeded_normal_bf16(torch, (n_blocks, 64, D), 200 + 2 * l_),
              seeded_normal_bf16(torch, (n_blocks, D, 64), 201 + 2 * l_)) for l_ in range(layers)]
    wsb = lcat.attn_decode_workspace_bytes(B, Hq, c["max_blocks"])
    ws = [torch.empty(wsb, dtype=torch.uint8, device="cuda") for _ in range(layers)]
    outs = [(torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda"),
             torch.empty((B, Hq), dtype=torch.float32, device="cuda")) for _ in range(layers)]

    def step():
        for l_, (kp, vp) in enumerate(pools):
            lcat.attn_decode(q, kp, vp, *meta, workspace=ws[l_], o=outs[l_][0], lse=outs[l_][1])

    def wall_us(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(iters):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / iters

    for _ in range(3):
        step()
    eager_us = wall_us(step)
    eager_last = [o.clone() for o, _ in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    graph_us = wall_us(g.replay)
    same = all(torch.equal(o.view(torch.int16), e.view(torch.int16))
               for (o, _), e in zip(outs, eager_last))
    nbytes = layers * (int(c["ctx_len"].sum()) * 2 * D * 2 * 2 + 2 * B * Hq * D * 2 + B * Hq * 4)
    del pools, ws
    return dict(layers=layers, eager_us_per_step=round(eager_us, 1),
                graph_us_per_step=round(graph_us, 1), speedup=round(eager_us / graph_us, 2),
                graph_us_per_layer=round(graph_us / layers, 2),
                graph_GBps=round(nbytes / (graph_us * 1e-6) / 1e9, 1),
                graph_equals_eager=bool(same),
                workload=f"{layers} layers x 4 requests x 8192 cached tokens, 16 Q / 2 KV heads")


def bench_rope(torch, lcat, iters=30, n_sets=6):
    """rope_apply on the 32K step's Q [32768][16][128] and K [32768][2][128]
    bf16, in place, each alone and both in one rope_apply_qk launch, cycling
    through ``n_sets`` buffers (768 MB of Q, so no
    call finds its data in the last-level cache); against an in-place copy of
    the same bytes (the yardstick for a pass that rewrites its input) and a
    copy into a separate buffer."""
    S = 32768
    pos = torch.arange(S, dtype=torch.int32, device="cuda")
    res = {}
    for name, H in (("q", 16), ("k", 2)):
        xs = [seeded_normal_bf16(torch, (S, H, D), 81 + i) for i in range(n_sets)]
        run = rotating([lambda x=x: lcat.rope_apply(x, pos) for x in xs])
        for _ in range(n_sets):
            run()
        torch.cuda.synchronize()
        ms = back_to_back_ms(torch, run, iters)
        nb = 2 * S * H * D * 2
        gbs = nb / (ms * 1e-3) / 1e9
        res[name] = dict(us=round(ms * 1e3, 2), GBps=round(gbs, 1),
                         frac_hbm=round(gbs / PEAK_HBM_GBS, 4), bytes=nb,
                         shape=f"[{S}][{H}][{D}] bf16, positions 0..{S - 1}")
        if name == "q":
            flat = [x.view(-1) for x in xs]
            cp_in = rotating([lambda f=f: lcat.measure_hbm_copy(f, f) for f in flat])
            for _ in range(n_sets):
                cp_in()
            torch.cuda.synchronize()
            ms_in = back_to_back_ms(torch, cp_in, iters)
            dst = torch.empty_like(flat[0])
            cp_out = rotating([lambda f=f: lcat.measure_hbm_copy(f, dst) for f in flat])
            ms_out = back_to_back_ms(torch, cp_out, iters)
            in_gbs, out_gbs = nb / (ms_in * 1e-3) / 1e9, nb / (ms_out * 1e-3) / 1e9
            res["copy_in_place"] = dict(GBps=round(in_gbs, 1),
                                        frac_hbm=round(in_gbs / PEAK_HBM_GBS, 4),
                                        kernel="hbm_copy_kernel with dst == src")
            res["copy_separate"] = dict(GBps=round(out_gbs, 1),
                                        frac_hbm=round(out_gbs / PEAK_HBM_GBS, 4))
            res["q"]["frac_of_in_place_copy"] = round(gbs / in_gbs, 4)
        del xs
    # Q and K of one step in a single launch (rope_apply_qk), the form the
    # step uses: 144 MB moved per call.
    qs = [seeded_normal_bf16(torch, (S, 16, D), 81 + i) for i in range(n_sets)]
    ks = [seeded_normal_bf16(torch, (S, 2, D), 91 + i) for i in range(n_sets)]
    run = rotating([lambda a=a, b=b: lcat.rope_apply_qk(a, b, pos) for a, b in zip(qs, ks)])
    for _ in range(n_sets):
        run()
    torch.cuda.synchronize()
    ms = back_to_back_ms(torch, run, iters)
    nb = 2 * S * (16 + 2) * D * 2
    gbs = nb / (ms * 1e-3) / 1e9
    res["qk"] = dict(us=round(ms * 1e3, 2), GBps=round(gbs, 1),
                     frac_hbm=round(gbs / PEAK_HBM_GBS, 4), bytes=nb,
                     two_calls_us=round(res["q"]["us"] + res["k"]["us"], 2),
                     shape=f"Q [{S}][16][{D}] and K [{S}][2][{D}] bf16, one launch")
    del qs, ks
    res["buffer_sets"] = n_sets
    return res


def bench_chunked(torch, lcat, synth):
    B, S, C, Hq, Hkv = 4, 131072, 8192, 16, 2
    table, tags, n_blocks = synth.chunked_block_table(B, S, C, Hkv)
    q = seeded_normal_bf16(torch, (B, S, Hq, D), SEEDS["chunked_4x131072"][0])
    k = seeded_normal_bf16(torch, (B, S, Hkv, D), SEEDS["chunked_4x131072"][1])
    v = seeded_normal_bf16(torch, (B, S, Hkv, D), SEEDS["chunked_4x131072"][2])
    k_pool = torch.empty((n_blocks, 64, D), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.empty((n_blocks, D, 64), dtype=torch.bfloat16, device="cuda")
    tags_d, table_d = dev_tensor(torch, tags), dev_tensor(torch, table)
    qs = [q[:, c0:c0 + C].contiguous() for c0 in range(0, S, C)]
    ks = [k[:, c0:c0 + C].contiguous() for c0 in range(0, S, C)]
    vs = [v[:, c0:c0 + C].contiguous() for c0 in range(0, S, C)]
    cbs = [torch.full((B,), c0, dtype=torch.int32, device="cuda") for c0 in range(0, S, C)]
    # each chunk writes its own output, as a serving engine would
    os_ = [torch.empty((B, C, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in qs]
    lses = [torch.empty((B, Hq, C), dtype=torch.float32, device="cuda") for _ in qs]
    timer = EventTimer(torch)
    for rep in range(2):
        with timer:
            for i in range(len(qs)):
                lcat.attn_chunked_prefill(qs[i], ks[i], vs[i], k_pool, v_pool, tags_d, table_d,
                                          cbs[i], o=os_[i], lse=lses[i])
        if rep == 0:
            torch.cuda.synchronize()
            timer.pairs.clear()
    torch.cuda.synchronize()
    ms = timer.mean_ms()
    flops = causal_flops(B, S, Hq)
    tf = flops / (ms * 1e-3) / 1e12
    del qs, ks, vs, k_pool, v_pool
    check = dict(q=q, k=k, v=v, outs=os_, lses=lses, C=C)
    return check, dict(ms_per_pass=round(ms, 2), TFLOPs=round(tf, 1),
                       frac_mfma=round(tf / PEAK_BF16_TFLOPS, 4), chunks=S // C,
                       workload="4 requests x 131072 tokens, 8192-token chunks, 16 Q / 2 KV heads")


def bench_cp(torch, lcat, iters=3):
    """Zigzag context parallelism, 4 ranks over 65536 tokens, 16 Q / 2 KV heads:
    the work of one rank (its queries against every rank's key shard with
    position-derived limits, the partials combined by the LSE rescale), all
    shards resident."""
    S, N, Hq, Hkv, mode = 65536, 4, 16, 2, "zigzag"
    q, k, v = (seeded_normal_bf16(torch, shape, sd) for shape, sd in
               zip(((S, Hq, D), (S, Hkv, D), (S, Hkv, D)), SEEDS["cp_zigzag_64k"]))
    shards = [(lcat.cp_shard(k, N, s_, mode), lcat.cp_shard(v, N, s_, mode)[0]) for s_ in range(N)]
    res = {}
    for rank in (0, N - 1):
        qr, qpos = lcat.cp_shard(q, N, rank, mode)
        n = qr.shape[0]
        lims = [torch.empty((1, n), dtype=torch.int32, device="cuda") for _ in range(N)]
        parts = [(torch.empty((1, n, Hq, D), dtype=torch.bfloat16, device="cuda"),
                  torch.empty((1, Hq, n), dtype=torch.float32, device="cuda")) for _ in range(N)]

        def rank_step_merge():   # partials, then the LSE merge kernel
            for s_, ((ks, kpos), vs) in enumerate(shards):
                lcat.attn_key_limits(qpos, kpos, out=lims[s_])
                lcat.attn_prefill_limited(qr[None], ks[None], vs[None], lims[s_], o=parts[s_][0],
                                          lse=parts[s_][1])
            for s_ in range(1, N):
                lcat.attn_merge(parts[0][0], parts[0][1], parts[s_][0], parts[s_][1],
                                o=parts[0][0], lse=parts[0][1])

        def rank_step():   # each partial merged into the running result in its epilogue
            for s_, ((ks, kpos), vs) in enumerate(shards):
                lcat.attn_key_limits(qpos, kpos, out=lims[s_])
                lcat.attn_prefill_limited(qr[None], ks[None], vs[None], lims[s_], o=parts[0][0],
                                          lse=parts[0][1], accumulate=s_ > 0)

        times = {}
        for name, fn in (("merge_kernels", rank_step_merge), ("accumulate", rank_step)):
            fn()
            torch.cuda.synchronize()
            timer = EventTimer(torch)
            for _ in range(iters):
                with timer:
                    fn()
            torch.cuda.synchronize()
            times[name] = timer.mean_ms()
        ms = times["accumulate"]
        pairs = float((qpos.long() + 1).sum().item())      # causal: keys at positions <= p
        flops = 4.0 * D * Hq * pairs
        tf = flops / (ms * 1e-3) / 1e12
        res[f"rank{rank}"] = dict(ms=round(ms, 3), TFLOPs=round(tf, 1),
                                  frac_mfma=round(tf / PEAK_BF16_TFLOPS, 4), flop=flops,
                                  ms_with_merge_kernels=round(times["merge_kernels"], 3))
    res["workload"] = ("zigzag context parallelism, 4 ranks over 65536 tokens, 16 Q / 2 KV heads: "
                       "one rank's 4 partials (key limits + prefix-limited prefill), each merged "
                       "into the running (O, LSE) in its epilogue; ms_with_merge_kernels: the same "
                       "with separate LSE merge launches")
    return res


def bench_fixed_cost(torch, lcat, reps=10):
    """Per-workgroup fixed cost of the dense prefill kernel: non-causal launches
    of 4096 workgroups (B x S/32 x Hkv at 16 Q / 2 KV heads) that see 8, 16, 32
    or 64 key tiles each, and a least-squares fit of launch time against
    tiles per workgroup (16 rounds of 256 workgroups per launch)."""
    Hq, Hkv = 16, 2
    pts = []
    for S, B in ((512, 128), (1024, 64), (2048, 32), (4096, 16)):
        q = seeded_normal_bf16(torch, (B, S, Hq, D), 71)
        k = seeded_normal_bf16(torch, (B, S, Hkv, D), 72)
        v = seeded_normal_bf16(torch, (B, S, Hkv, D), 73)
        o, lse = torch.empty_like(q), torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        run = lambda: lcat.attn_prefill(q, k, v, causal=False, o=o, lse=lse)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        ms = back_to_back_ms(torch, run, reps)
        flops = 4.0 * D * Hq * B * S * S
        pts.append(dict(tiles_per_wg=S // 64, workgroups=B * (S // 32) * Hkv, ms=round(ms, 4),
                        TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1)))
    t = np.array([p_["tiles_per_wg"] for p_ in pts], float)
    m = np.array([p_["ms"] for p_ in pts]) * 1e3 / (4096 / 256)   # us per round of 256
    (fixed, per_tile), *_ = np.linalg.lstsq(np.stack([np.ones_like(t), t], 1), m, rcond=None)
    return dict(points=pts, fixed_us_per_workgroup=round(float(fixed), 2),
                us_per_key_tile=round(float(per_tile), 3),
                workload="non-causal prefill, 16 Q / 2 KV heads, 4096 workgroups per launch")


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on every configuration, on this host's cores
# ---------------------------------------------------------------------------
BF16_TOL = 2e-2   # |gpu - oracle| <= 2e-2 + 2e-2 |oracle| on every sampled row


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def pick(t, rows, dim=1):
    """Rows ``rows`` (numpy indices) of a GPU tensor along ``dim``."""
    import torch
    return t.index_select(dim, torch.as_tensor(rows, dtype=torch.long, device=t.device))


def host(t):
    """torch tensor -> numpy (bf16 as uint16 bit patterns)."""
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def widen_bf16(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def compare(got, ref, got_lse=None, ref_lse=None):
    """Largest error of the GPU rows against the oracle rows, and whether every
    element is within the bf16 bar (fp32 rows: max |err| <= 1e-3)."""
    err = np.abs(got - ref)
    out = dict(max_abs_err=float(err.max()),
               within_tol=bool(np.all(err <= BF16_TOL + BF16_TOL * np.abs(ref))))
    if got_lse is not None:
        out["max_lse_err"] = float(np.max(np.abs(got_lse - ref_lse)))
    return out


def timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0


def rate(flops, sec, full_pairs, sample_pairs):
    return dict(seconds=round(sec, 3), TFLOPs=round(flops / sec / 1e12, 6),
                full_config_seconds_extrapolated=round(sec * full_pairs / sample_pairs, 1))


def cpu_tiny(lcat, torch):
    """Tiny fp32 case in full: 256 queries and keys, one head, non-causal."""
    import oracle
    import synth
    d = synth.tiny_exact(seed=SEEDS["tiny_fp32"])
    (ref, ref_lse), sec = timed(lambda: oracle.attention(d["q"], d["k"], d["v"], d["scale"]))
    o, lse = lcat.attn_prefill(dev_tensor(torch, d["q"]), dev_tensor(torch, d["k"]),
                               dev_tensor(torch, d["v"]), causal=False, scale=d["scale"])
    got = o.cpu().numpy().astype(np.float64)
    pairs = 256 * 256
    r = rate(4.0 * 64 * pairs, sec, pairs, pairs)
    err = float(np.abs(got - ref).max())
    r.update(rows="all 256", max_abs_err=err, within_tol=err <= 1e-3,
             max_lse_err=float(np.abs(lse.cpu().numpy() - ref_lse).max()))
    return r


def cpu_prefill_32k(chk, rows_n=512):
    """Causal GQA prefill at 32768: RoPE of the sampled query rows and of all
    keys, then causal attention of those rows."""
    import oracle
    import synth
    d = chk["d"]
    S, Hq = d["q"].shape[1], d["q"].shape[2]
    rows = synth.sample_rows(SEEDS["cpu_sample_rows"], S, rows_n, forced=(0, 1, 255, 256, S - 1))
    pos = d["positions"].astype(np.int64)

    def run():
        qr = oracle.rope(d["q"][0, rows], pos[rows])[None]
        kr = oracle.rope(d["k"][0], pos)[None]
        return oracle.attention_rows(qr, kr, oracle.widen(d["v"]), (rows + 1)[None], d["scale"])
    (ref, ref_lse), sec = timed(run)
    sample_pairs = float(np.sum(rows + 1))
    r = rate(4.0 * D * Hq * sample_pairs, sec, S * (S + 1) / 2, sample_pairs)
    r.update(rows=f"{rows.size} of the {S} query rows x {Hq} heads")
    r.update(compare(widen_bf16(host(pick(chk["o"], rows))), ref,
                     host(pick(chk["lse"], rows, 2)), ref_lse))
    return r


def cpu_pipeline_64k(chk, rows_n=512):
    """64K pipeline, rank 0: relayout of the [4][16384][64|8][128] inputs,
    RoPE at positions 0..65535, causal attention of the sampled rows."""
    import oracle
    import synth
    qin, kin, vin = host(chk["qin"]), host(chk["kin"]), host(chk["vin"])
    S = qin.shape[0] * qin.shape[1]
    rows = synth.sample_rows(SEEDS["cpu_sample_rows"] + 1, S, rows_n,
                             forced=(0, 1, 16383, 16384, 32767, 32768, 49151, 49152, S - 1))
    pos = np.arange(S, dtype=np.int64)

    def run():
        q, k, v = (oracle.permute(x, 0) for x in (qin, kin, vin))
        qr = oracle.rope(q[rows], pos[rows])[None]
        kr = oracle.rope(k, pos)[None]
        return oracle.attention_rows(qr, kr, v[None], (rows + 1)[None], 1.0 / np.sqrt(D))
    (ref, ref_lse), sec = timed(run)
    Hq = ref.shape[2]
    sample_pairs = float(np.sum(rows + 1))
    r = rate(4.0 * D * Hq * sample_pairs, sec, S * (S + 1) / 2, sample_pairs)
    r.update(rows=f"{rows.size} of the {S} query rows x {Hq} heads")
    r.update(compare(widen_bf16(host(pick(chk["o"], rows))), ref,
                     host(pick(chk["lse"], rows, 2)), ref_lse))
    return r


def cpu_decode(chk):
    """Paged decode, all 32 requests x 16 heads: gather of each request's
    cache, then attention of its one query over all ctx_len keys."""
    import oracle
    c = chk["c"]
    kp, vp, q = host(chk["k_pool"]), host(chk["v_pool"]), host(chk["q"])
    ctx = c["ctx_len"]

    def run():
        ks, vs = oracle.paged_gather(kp, vp, c["block_table"], ctx)
        return oracle.decode_attention(q, [ks[b] for b in range(len(ctx))],
                                       [vs[b] for b in range(len(ctx))], ctx, c["scale"])
    (ref, ref_lse), sec = timed(run)
    pairs = float(np.sum(ctx))
    Hq = q.shape[1]
    r = rate(4.0 * D * Hq * pairs, sec, pairs, pairs)
    r.update(rows=f"all {len(ctx)} requests x {Hq} heads")
    r.update(compare(widen_bf16(host(chk["o"])), ref, host(chk["lse"]), ref_lse))
    return r


def cpu_chunked(chk, rows_per_req=64):
    """Chunked prefill, 4 x 131072: causal attention of sampled rows of every
    request over the full sequence (what the chunks compute, by definition)."""
    import oracle
    import synth
    C = chk["C"]
    B, S, Hq = chk["q"].shape[:3]
    forced = [r for c0 in range(C, S, C) for r in (c0 - 1, c0)] + [0, S - 1]
    rows = synth.sample_rows(SEEDS["cpu_sample_rows"] + 2, S, rows_per_req, forced=forced)
    k, v = host(chk["k"]), host(chk["v"])
    qs = host(pick(chk["q"], rows))

    def run():
        return oracle.attention_rows(qs, k, v, np.broadcast_to(rows + 1, (B, rows.size)),
                                     1.0 / np.sqrt(D))
    (ref, ref_lse), sec = timed(run)
    got = np.stack([widen_bf16(host(chk["outs"][r // C][:, r % C])) for r in rows], axis=1)
    got_lse = np.stack([host(chk["lses"][r // C][:, :, r % C]) for r in rows], axis=2)
    sample_pairs = float(B * np.sum(rows + 1))
    r = rate(4.0 * D * Hq * sample_pairs, sec, B * S * (S + 1) / 2, sample_pairs)
    r.update(rows=f"{rows.size} of {S} per request x {B} requests x {Hq} heads, "
                  f"incl. every chunk boundary")
    r.update(compare(got, ref, got_lse, ref_lse))
    return r


def cpu_baseline(lcat, torch, checks):
    """The fp64 oracle timed on a bounded sample of each configuration, on all
    host cores in this process's affinity mask; each sample's GPU rows from
    the legs above are checked against it."""
    import oracle
    cfg = {}
    t0 = time.perf_counter()
    cfg["tiny_fp32"] = cpu_tiny(lcat, torch)
    if "step" in checks:
        cfg["causal_gqa_32k"] = cpu_prefill_32k(checks["step"])
    if "relayout" in checks:
        cfg["pipeline_64k"] = cpu_pipeline_64k(checks["relayout"])
    if "decode" in checks:
        cfg["decode_32req"] = cpu_decode(checks["decode"])
    if "chunked" in checks:
        cfg["chunked_4x131072"] = cpu_chunked(checks["chunked"])
    total = time.perf_counter() - t0
    head = cfg.get("causal_gqa_32k", cfg["tiny_fp32"])
    return dict(value=head["TFLOPs"], unit="TFLOP/s", cores=oracle.num_threads(), kind="oracle",
                cpu_model=cpu_model(), seconds_total=round(total, 1),
                sample=(f"{head['rows']} of the seq-32768 causal GQA step workload, "
                        "fp64, incl. RoPE of those rows and all keys; per-configuration samples, "
                        "extrapolated full-configuration times and GPU-vs-oracle errors on the "
                        "same rows under 'configs'"),
                all_within_tol=all(c.get("within_tol", True) for c in cfg.values()),
                configs=cfg)


def git_sha():
    """Commit of the working tree, when it is a git checkout (None otherwise)."""
    import subprocess
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                           timeout=10)
    except (OSError, subprocess.SubprocessError):
        return None
    return (r.stdout.strip() or None) if r.returncode == 0 else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="time only the step workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["step", "decode", "relayout", "chunked", "cp", "mfma",
                                       "fixed_cost", "rope", "fp8", "decode_graph"],
                    help="run a single leg (for profiling); prints its own JSON object")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this library runs on exactly one GPU; --gpus {args.gpus} is not "
              "supported (the sequence-parallel exchange across GPUs is not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_attention_tiled_amd as lcat
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    lib = lcat.load_library()
    build_id = lib.attn_build_id().decode()
    if args.only and args.only != "step":
        log(f"bench: only {args.only}")
        if args.only == "decode":
            res = bench_decode(torch, lcat, synth)[1]
        elif args.only == "relayout":
            res = bench_relayout_and_prefill_64k(torch, lcat)[1]
        elif args.only == "cp":
            res = bench_cp(torch, lcat)
        elif args.only == "mfma":
            res = bench_mfma_rate(torch, lcat)
        elif args.only == "fixed_cost":
            res = bench_fixed_cost(torch, lcat)
        elif args.only == "rope":
            res = bench_rope(torch, lcat)
        elif args.only == "fp8":
            res = bench_fp8_prefill(torch, lcat, synth)
        elif args.only == "decode_graph":
            res = bench_decode_graph(torch, lcat, synth)
        else:
            res = bench_chunked(torch, lcat, synth)[1]
        print(json.dumps({args.only: res, "build_id": build_id}), flush=True)
        return
    log("bench: causal GQA prefill step (seq 32768)")
    checks = {}
    checks["step"], step = bench_step(torch, lcat, synth, args.steps, args.warmup)
    out = {
        "metric": METRIC, "value": round(step["value"], 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16, resident in HBM",
        "config": {"workload": "causal GQA prefill with RoPE at absolute positions: batch 1, "
                               "seq 32768, 16 Q / 2 KV heads, head_dim 128",
                   "global_batch": 1, "seq_len": 32768, "parallelism": "single GPU"},
        "roofline": step["roofline"],
        "seeds": SEEDS, "build_id": build_id, "git_sha": git_sha(),
    }
    if not args.no_extra and not args.only:
        log("bench: sustained MFMA rate")
        out["mfma_sustained"] = bench_mfma_rate(torch, lcat)
        out["roofline"]["frac_of_sustained"] = round(
            out["roofline"]["achieved"] / out["mfma_sustained"]["tflops"], 4)
        out["roofline"]["frac_of_sustained_lds"] = round(
            out["roofline"]["achieved"] / out["mfma_sustained"]["a_from_lds"]["tflops"], 4)
        log("bench: rope_apply")
        out["rope"] = bench_rope(torch, lcat)
        log("bench: prefill with FP8 scores")
        out["prefill_fp8"] = bench_fp8_prefill(torch, lcat, synth)
        log("bench: decode")
        checks["decode"], out["decode"] = bench_decode(torch, lcat, synth)
        log("bench: decode step in a HIP graph")
        out["decode_graph"] = bench_decode_graph(torch, lcat, synth)
        log("bench: relayout + prefill 64k")
        checks["relayout"], (out["relayout"], out["prefill_64k"], out["relayout_back"]) = \
            bench_relayout_and_prefill_64k(torch, lcat)
        log("bench: chunked prefill")
        checks["chunked"], out["chunked_prefill"] = bench_chunked(torch, lcat, synth)
        log("bench: context parallelism (zigzag, 4 ranks, 64k)")
        out["cp_zigzag_64k"] = bench_cp(torch, lcat)
    if not args.no_cpu_baseline and not args.only:
        log("bench: cpu baseline (oracle) and GPU-vs-oracle check of the sampled rows")
        out["cpu_baseline"] = cpu_baseline(lcat, torch, checks)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
