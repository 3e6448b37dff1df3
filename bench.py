#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm SECONDS] [--no-secondary] [--no-cpu-baseline]
                    [--no-cpu-configs] [--workloads LIST]

Primary line: causal GQA prefill, bf16, B=2 Hq=32 Hkv=8 S=8192 D=128 (workload gqa_prefill_s8192). One step is the
hot path over one batch: the RoPE cos/sin table, RoPE on K, then attn_prefill_rope (attention with the rotation of
Q fused into the kernel's load of Q). `value` is the algorithmic attention flops
(QK^T and PV over the unmasked pairs, 2 flop per multiply-add) per second of wall time over K timed steps,
with the inputs already resident in HBM. Secondary objects on the same line (same method, HIP events on the
launch stream): paged GQA decode (bf16, FP8 E4M3 and int8 caches) and MLA absorbed decode in GB/s of algorithmic
bytes, the 131072-token prefill and the chunked prefill from a paged cache (four 2048-token chunks on 0 / 4096 /
8192 / 14336 cached tokens; one step = append with RoPE on K, RoPE on Q, attend) and the 131072-token prefill with a
sliding window of 4096 plus anchors every 32 tokens in TFLOP/s of visible pairs, and DeepSeek Sparse
Attention decode (lightning indexer over 32768 cached tokens, top-2048 selection, sparse MLA) in GB/s of
algorithmic bytes.

`roofline` describes the dominant kernel of each workload: achieved = algorithmic work per launch / average
launch duration (HIP events on the stream the kernel runs on), against MI355X's published peaks (bf16 dense MFMA
2.5 PFLOP/s, HBM 8 TB/s). `traffic` is the counter-measured HBM bytes per launch from the committed rocprofv3
summary (profiles/traffic.json) when it was taken on the current kernel source, else null.

Before its `warmup` steps the primary workload runs untimed steps for `--prewarm` seconds (0.5 by default) so the
GPU clock has settled; the timed region is the same K steps (reported as `prewarm`).

`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the primary workload (seeded query rows, every
head): a reported baseline, not a target. `cpu_baseline_configs` times the oracle on every configuration the parity
tests run in full (fp32 MHA, paged decode, MLA decode) and on the 131072-token prefill's 256 sampled rows, with the
CPU model and BLAS thread count.
"""
import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import (WORKLOADS, prefill_inputs, paged_decode_inputs, mla_inputs, sampled_rows,  # noqa: E402
                   chunked_prefill_inputs, dsa_inputs)

METRIC = "prefill attention TFLOP/s (% bf16 MFMA peak); decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = {
    "prefill_bf16_kernel": "prefill.hip",
    "decode_paged_q8_kernel": "decode.hip",
    "decode_paged_lds_kernel": "decode.hip",
    "mla_split_kernel": "mla.hip",
    "mla_split_fp8mma_kernel": "mla.hip",
    "dsa_indexer_kernel": "dsa.hip",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(fname):
    """Digest of a kernel source and device.h with comments and blank space removed: the counters stay valid for
    an edit that only touches comments, and any change to the code itself invalidates them."""
    p = os.path.join(ROOT, "transformer_attention_causal_amd", "csrc", fname)
    h = hashlib.sha256()
    for f in (p, os.path.join(ROOT, "transformer_attention_causal_amd", "csrc", "device.h")):
        with open(f, encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from profiles/traffic.json (rocprofv3 FETCH_SIZE and WRITE_SIZE,
    scaled by a plain-copy calibration), if measured on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f).get(f"{kernel}@{workload}")
    if not t or t.get("source_sha") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return t.get("hbm_bytes_per_launch")


def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class EventTimer:
    """Average duration of one kernel launch, recorded with events on the launch stream."""

    def __init__(self, torch):
        self.torch, self.pairs = torch, []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append([e, None])

    def stop(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))


def roofline_compute(flops, ms, kernel, workload):
    achieved = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic_for(kernel, workload), "kernel": kernel,
            "kernel_ms": round(ms, 4)}


def roofline_hbm(nbytes, ms, kernel, workload, timed=None):
    """`ms` times one library call; `timed` names the kernels it launches when there is more than `kernel`."""
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_for(kernel, workload), "kernel": kernel,
            "timed": timed or kernel, "kernel_ms": round(ms, 4)}


# --------------------------------------------------------------------------------------------------- prefill --
def bench_prefill(torch, ta, w, steps, warmup, seed=0, local_global=False, prewarm_s=0.0):
    log(f"[bench] {w.name}: generating inputs")
    inp = prefill_inputs(w, seed=seed)
    q, k, v = (dev_bf16(torch, inp[n]) for n in ("q", "k", "v"))
    pos = torch.from_numpy(inp["positions"]).cuda()
    o = torch.empty_like(q)
    timer = EventTimer(torch)

    table = torch.empty((w.seqlen, w.head_dim // 2, 2), dtype=torch.float32, device="cuda")

    def step(timed):
        if local_global:
            ta.attn_rope_apply(q, pos, w.theta)
            ta.attn_rope_apply(k, pos, w.theta)
            if timed:
                timer.start()
            ta.attn_prefill_local_global(q, k, v, w.window, w.n_lead, w.anchor_stride, softmax_scale=w.scale, o=o)
        else:
            # RoPE(Q) fused into the prefill's load of Q: the step builds the cos/sin table, rotates K in place,
            # and attends with q unrotated
            ta.attn_rope_table(w.seqlen, w.head_dim, w.theta, table=table)
            ta.attn_rope_apply(k, pos, w.theta)
            if timed:
                timer.start()
            ta.attn_prefill_rope(q, k, v, table, softmax_scale=w.scale, o=o)
        if timed:
            timer.stop()

    # Clock-settle pre-warm, independent of `warmup`: untimed steps until prewarm_s seconds of wall time have
    # passed (the GPU clock takes about 0.1 s of load to settle; shorter warm-ups under-report by 5-25%).
    pw_steps, t_pw = 0, time.perf_counter()
    while time.perf_counter() - t_pw < prewarm_s:
        for _ in range(8):
            step(False)
        pw_steps += 8
        torch.cuda.synchronize()
    prewarm = {"seconds": round(time.perf_counter() - t_pw, 3), "steps": pw_steps}
    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    kern_ms = timer.mean_ms()
    del q, k, v, o
    torch.cuda.empty_cache()
    return wall_ms, kern_ms, prewarm


# ---------------------------------------------------------------------------------------------- paged decode --
def decode_bytes(w, inp):
    """Algorithmic bytes of one decode step: every cached K and V row of every sequence once (2 bytes per element,
    or 1 for an 8-bit cache, plus its scales), q, o, the used block table entries and the lengths."""
    tokens = int(inp["seq_lens"].astype(np.int64).sum())
    pages = int(((inp["seq_lens"].astype(np.int64) + w.page_size - 1) // w.page_size).sum())
    qo = 2 * inp["q"].size * 2
    elem = 1 if inp.get("kv", "bf16") != "bf16" else 2
    scales = 2 * w.hkv * w.head_dim * 4 if elem == 1 else 0
    return tokens * w.hkv * w.head_dim * 2 * elem + qo + pages * 4 + inp["seq_lens"].size * 4 + scales


def bench_decode(torch, ta, w, steps, warmup, seed=0, kv="bf16"):
    log(f"[bench] {w.name} ({kv} cache): generating inputs")
    inp = paged_decode_inputs(w, seed=seed, kv=kv)
    q = dev_bf16(torch, inp["q"])
    if kv == "bf16":
        kc, vc = dev_bf16(torch, inp["k_cache"]), dev_bf16(torch, inp["v_cache"])
    else:
        kc, vc = torch.from_numpy(inp["k_cache"]).cuda(), torch.from_numpy(inp["v_cache"]).cuda()
        ksc, vsc = torch.from_numpy(inp["k_scale"]).cuda(), torch.from_numpy(inp["v_scale"]).cuda()
    table = torch.from_numpy(inp["block_table"]).cuda()
    lens = torch.from_numpy(inp["seq_lens"]).cuda()
    pos = torch.from_numpy(inp["positions"]).cuda()
    ta.attn_rope_apply(q, pos, w.theta)
    o = torch.empty_like(q)
    ws = torch.empty(ta.attn_decode_paged_workspace_size(w.batch, w.hq, w.head_dim, inp["max_len"]),
                     dtype=torch.uint8, device="cuda")
    timer = EventTimer(torch)
    for i in range(warmup + steps):
        if i >= warmup:
            timer.start()
        if kv == "bf16":
            ta.attn_decode_paged(q, kc, vc, table, lens, inp["max_len"], softmax_scale=w.scale, o=o, workspace=ws)
        else:
            ta.attn_decode_paged_q8(q, kc, vc, ksc, vsc, kv, table, lens, inp["max_len"], softmax_scale=w.scale, o=o,
                                    workspace=ws)
        if i >= warmup:
            timer.stop()
    torch.cuda.synchronize()
    ms = timer.mean_ms()
    nbytes = decode_bytes(w, inp)
    del q, kc, vc, o, ws
    torch.cuda.empty_cache()
    return ms, nbytes, int(inp["seq_lens"].sum())


def mla_bytes(w, elem=2):
    """Algorithmic bytes of one MLA decode: every cached latent and rope element once (2 bytes, or 1 for an 8-bit
    cache plus its per-channel scales), the queries, the output and the lengths."""
    scales = (w.latent + w.rope) * 4 if elem == 1 else 0
    return (w.batch * w.seqlen * (w.latent + w.rope) * elem + w.batch * w.heads * (w.latent + w.rope) * 2
            + w.batch * w.heads * w.latent * 2 + w.batch * 4 + scales)


def mla_flops(w):
    return w.batch * w.heads * w.seqlen * (2 * (w.latent + w.rope) + 2 * w.latent)


def bench_mla(torch, ta, w, steps, warmup, seed=0, kv="bf16"):
    log(f"[bench] {w.name} ({kv} cache): generating inputs")
    inp = mla_inputs(w, seed=seed, kv=kv)
    ql, qp = (dev_bf16(torch, inp[n]) for n in ("q_lat", "q_pe"))
    if kv == "bf16":
        ckv, kpe = (dev_bf16(torch, inp[n]) for n in ("c_kv", "k_pe"))
    else:
        ckv, kpe, cs, ps = (torch.from_numpy(inp[n]).cuda() for n in ("c_kv", "k_pe", "c_scale", "pe_scale"))
    lens = torch.from_numpy(inp["seq_lens"]).cuda()
    o = torch.empty_like(ql)
    ws = torch.empty(ta.attn_mla_decode_workspace_size(w.batch, w.heads, w.latent, w.seqlen), dtype=torch.uint8,
                     device="cuda")
    timer = EventTimer(torch)
    for i in range(warmup + steps):
        if i >= warmup:
            timer.start()
        if kv == "bf16":
            ta.attn_mla_decode(ql, qp, ckv, kpe, lens, w.scale, o=o, workspace=ws)
        else:
            ta.attn_mla_decode_q8(ql, qp, ckv, kpe, cs, ps, kv, lens, w.scale, o=o, workspace=ws)
        if i >= warmup:
            timer.stop()
    torch.cuda.synchronize()
    ms = timer.mean_ms()
    del ql, qp, ckv, kpe, o, ws
    torch.cuda.empty_cache()
    return ms


# ------------------------------------------------------------------------------------------- chunked prefill --
def bench_chunked(torch, ta, w, steps, warmup, seed=0):
    log(f"[bench] {w.name}: generating inputs")
    inp = chunked_prefill_inputs(w, seed=seed)
    q, kn, vn = (dev_bf16(torch, inp[n]) for n in ("q", "k_new", "v_new"))
    kc, vc = dev_bf16(torch, inp["k_cache"]), dev_bf16(torch, inp["v_cache"])
    table, cu, ctx, pos = (torch.from_numpy(inp[n]).cuda() for n in ("block_table", "cu_new", "ctx_lens",
                                                                     "positions"))
    o = torch.empty_like(q)
    n_pos = int(inp["positions"].max()) + 1
    rope_tab = torch.empty((n_pos, q.shape[-1] // 2, 2), dtype=torch.float32, device="cuda")
    timer = EventTimer(torch)

    def step(timed):
        ta.attn_rope_table(n_pos, q.shape[-1], w.theta, table=rope_tab)
        ta.attn_kv_append_paged(kn, vn, cu, ctx, kc, vc, table, w.theta)
        if timed:
            timer.start()
        ta.attn_prefill_paged_rope(q, kc, vc, table, cu, ctx, inp["max_new"], rope_tab, softmax_scale=w.scale, o=o)
        if timed:
            timer.stop()

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    kern_ms = timer.mean_ms()
    del q, kn, vn, kc, vc, o, rope_tab
    torch.cuda.empty_cache()
    return wall_ms, kern_ms


# ---------------------------------------------------------------------------------------- sparse attention --
def dsa_bytes(w):
    """Algorithmic bytes of each DSA kernel: the indexer reads every indexer key, its queries and weights, and
    writes one fp32 score per token; top-k reads the scores and writes the indices; sparse MLA reads the selected
    [c_kv ; k_pe] rows, the queries, and writes the latent output."""
    b, t = w.batch, w.seqlen
    idx = b * t * w.idx_dim * 2 + b * w.idx_heads * (w.idx_dim * 2 + 4) + b * t * 4
    topk = b * t * 4 + b * w.topk * 4 + b * 4
    sparse = (b * w.topk * (w.latent + w.rope) * 2 + b * w.heads * (w.latent + w.rope) * 2 + b * w.heads * w.latent * 2
              + b * w.topk * 4)
    return {"indexer": idx, "topk": topk, "sparse_mla": sparse}


def bench_dsa(torch, ta, w, steps, warmup, seed=0):
    log(f"[bench] {w.name}: generating inputs")
    inp = dsa_inputs(w, seed=seed)
    qi, ki = dev_bf16(torch, inp["q_idx"]), dev_bf16(torch, inp["k_idx"])
    wi = torch.from_numpy(inp["w_idx"]).cuda()
    ql, qp, ckv, kpe = (dev_bf16(torch, inp[n]) for n in ("q_lat", "q_pe", "c_kv", "k_pe"))
    lens = torch.from_numpy(inp["seq_lens"]).cuda()
    scores = torch.empty((w.batch, w.seqlen), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.batch, w.topk), dtype=torch.int32, device="cuda")
    o = torch.empty_like(ql)
    ws = torch.empty(ta.attn_mla_sparse_decode_workspace_size(w.batch, w.heads, w.latent, w.topk), dtype=torch.uint8,
                     device="cuda")
    timers = {k: EventTimer(torch) for k in ("indexer", "topk", "sparse_mla")}

    def step(timed):
        for name, fn in (("indexer", lambda: ta.attn_dsa_indexer(qi, wi, ki, lens, scores=scores)),
                         ("topk", lambda: ta.attn_topk(scores, lens, w.topk, indices=idx)),
                         ("sparse_mla", lambda: ta.attn_mla_sparse_decode(ql, qp, ckv, kpe, lens, idx, w.scale, o=o,
                                                                         workspace=ws))):
            if timed:
                timers[name].start()
            fn()
            if timed:
                timers[name].stop()

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = {k: t.mean_ms() for k, t in timers.items()}
    eager = [t.clone() for t in (scores, idx, o)]
    # The same step captured once as a HIP graph and replayed, as a serving loop runs a launch-bound decode step:
    # no host work between the three kernels. The replay must reproduce the eager outputs bit for bit.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(False)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(False)
    for t in (scores, idx, o):
        t.zero_()
    graph.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip((scores, idx, o), eager)):
        raise RuntimeError("dsa step: graph replay differs from the eager step")
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / steps
    del graph, qi, ki, wi, ql, qp, ckv, kpe, scores, idx, o, ws, eager
    torch.cuda.empty_cache()
    return graph_ms, wall_ms, ms


# ------------------------------------------------------------------------------------------------ cpu oracle --
def cpu_baseline(w, n_rows=4096, seed=0):
    """Time the fp64 oracle on `n_rows` seeded query rows (all heads, all batches) of the prefill workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        threads = 1
    inp = prefill_inputs(w, seed=seed)
    rows = sampled_rows(w.seqlen, n_rows, seed=seed)

    def f32(b):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    t0 = time.perf_counter()
    pos = np.broadcast_to(np.arange(w.seqlen), (w.batch, w.seqlen))
    k = oracle.rope(f32(inp["k"]), pos, w.theta)
    v = f32(inp["v"]).astype(np.float64)
    q = np.zeros((w.batch, w.seqlen, w.hq, w.head_dim))
    q[:, rows] = oracle.rope(f32(inp["q"][:, rows]), np.broadcast_to(rows, (w.batch, rows.size)), w.theta)
    oracle.attention_prefill_rows(q, k, v, rows, True, w.scale)
    dt = time.perf_counter() - t0
    flops = 4 * w.batch * w.hq * w.head_dim * int((rows + 1).sum())
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows.size} seeded query rows x {w.hq} heads x {w.batch} sequences of {w.name} "
                      f"(fp64 numpy, scores materialised, {dt:.1f} s)",
            "wall_s": round(dt, 3), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_info()["model"]}


def cpu_info():
    """CPU model, cores the process may run on, and numpy's BLAS thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        threads = 1
    return {"model": model, "affinity_cpus": len(os.sched_getaffinity(0)), "blas_threads": int(threads)}


def cpu_oracle_configs():
    """The fp64 oracle timed on each configuration as the parity tests run it: the fp32 MHA workload, the paged
    decode and the MLA decode in full, and the 131072-token prefill on its 256 seeded rows (every head). Input
    generation is not timed. Reports wall time, implied fp64 GFLOP/s of the algorithmic flops, and GB/s of the
    algorithmic bytes for the decode workloads. A reported baseline, not a target."""
    import oracle

    def f32(b):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)

    out = {"cpu": cpu_info()}
    # fp32 MHA, full
    w = WORKLOADS["mha_fp32_s256"]
    inp = prefill_inputs(w, seed=0)
    t0 = time.perf_counter()
    pos = inp["positions"].reshape(w.batch, w.seqlen)
    oracle.attention_prefill(oracle.rope(inp["q"], pos, w.theta), oracle.rope(inp["k"], pos, w.theta),
                             inp["v"].astype(np.float64), True, w.scale)
    dt = time.perf_counter() - t0
    out[w.name] = {"sample": "full", "wall_s": round(dt, 3), "gflops": round(w.flops / dt / 1e9, 2)}
    # paged decode, full
    wd = WORKLOADS["paged_decode_b64"]
    inp = paged_decode_inputs(wd, seed=0)
    kc, vc = f32(inp["k_cache"]), f32(inp["v_cache"])
    t0 = time.perf_counter()
    qr = oracle.rope(f32(inp["q"])[:, None], inp["positions"][:, None], wd.theta)[:, 0]
    oracle.decode_paged(qr, kc, vc, inp["block_table"], inp["seq_lens"], wd.scale)
    dt = time.perf_counter() - t0
    tokens = int(inp["seq_lens"].astype(np.int64).sum())
    out[wd.name] = {"sample": "full", "wall_s": round(dt, 3),
                    "gflops": round(4 * wd.hq * wd.head_dim * tokens / dt / 1e9, 2),
                    "GB/s": round(decode_bytes(wd, inp) / dt / 1e9, 3)}
    del inp, kc, vc
    # MLA decode, full
    wm = WORKLOADS["mla_decode_b32"]
    m = mla_inputs(wm, seed=0)
    ql, qp, ckv, kpe = (f32(m[n]) for n in ("q_lat", "q_pe", "c_kv", "k_pe"))
    t0 = time.perf_counter()
    oracle.mla_decode(ql, qp, ckv, kpe, m["seq_lens"], wm.scale)
    dt = time.perf_counter() - t0
    out[wm.name] = {"sample": "full", "wall_s": round(dt, 3), "gflops": round(mla_flops(wm) / dt / 1e9, 2),
                    "GB/s": round(mla_bytes(wm) / dt / 1e9, 3)}
    del m, ql, qp, ckv, kpe
    # 131072-token prefill on its 256 sampled rows
    wl = WORKLOADS["gqa_prefill_s131072"]
    inp = prefill_inputs(wl, seed=0)
    rows = sampled_rows(wl.seqlen, wl.sampled_rows, seed=0)
    t0 = time.perf_counter()
    pos = np.broadcast_to(np.arange(wl.seqlen), (wl.batch, wl.seqlen))
    k = oracle.rope(f32(inp["k"]), pos, wl.theta)
    v = f32(inp["v"]).astype(np.float64)
    q = np.zeros((wl.batch, wl.seqlen, wl.hq, wl.head_dim))
    q[:, rows] = oracle.rope(f32(inp["q"][:, rows]), np.broadcast_to(rows, (wl.batch, rows.size)), wl.theta)
    oracle.attention_prefill_rows(q, k, v, rows, True, wl.scale)
    dt = time.perf_counter() - t0
    flops = 4 * wl.batch * wl.hq * wl.head_dim * int((rows + 1).sum())
    out[wl.name] = {"sample": f"{rows.size} seeded query rows x {wl.hq} heads", "wall_s": round(dt, 3),
                    "gflops": round(flops / dt / 1e9, 2)}
    return out


# ------------------------------------------------------------------------------------------------------ main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # Warm-up long enough (about 0.1 s of work) for the GPU clock to settle before the timed steps.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-secondary", action="store_true", help="only the primary prefill workload")
    ap.add_argument("--workloads", default="prefill,decode,mla,long,chunked,dsa,decode_fp8,decode_int8,swa,mla_fp8,mla_int8",
                    help="comma list of prefill (primary), decode, mla, long, chunked, dsa, decode_fp8, decode_int8, "
                         "swa; profiling runs select one")
    ap.add_argument("--prewarm", type=float, default=0.5,
                    help="seconds of untimed primary steps before the warm-up steps (GPU clock settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cpu-configs", action="store_true",
                    help="skip the per-configuration oracle timings (keep only the bounded primary sample)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration for traffic measurements)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_attention_causal_amd as ta
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ta.load_library()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 3}))
        return

    sel = set(args.workloads.split(","))
    if sel - {"prefill", "decode", "mla", "long", "chunked", "dsa", "decode_fp8", "decode_int8", "swa", "mla_fp8",
              "mla_int8"}:
        print(f"unknown workloads {sel}", file=sys.stderr)
        sys.exit(2)
    if args.no_secondary:
        sel &= {"prefill"}
    w = WORKLOADS["gqa_prefill_s8192"]
    if "prefill" not in sel:          # profiling run of one secondary workload
        line = {}
        run_secondary(torch, ta, args, sel, line)
        print(json.dumps(line))
        return
    wall_ms, kern_ms, prewarm = bench_prefill(torch, ta, w, args.steps, args.warmup, prewarm_s=args.prewarm)
    value = w.flops / (wall_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded iid N(0,1), bf16)",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "hq": w.hq, "hkv": w.hkv,
                   "head_dim": w.head_dim, "causal": True, "rope_theta": w.theta,
                   "step": "rope_table + rope(k) + prefill_rope (rope(q) fused)", "flops_per_step": w.flops},
        "roofline": roofline_compute(w.flops, kern_ms, "prefill_bf16_kernel", w.name),
    }
    line["pct_bf16_peak_step"] = round(value / PEAK_BF16_TFLOPS, 4)
    line["prewarm"] = prewarm          # untimed clock-settle steps run before the `warmup` steps

    run_secondary(torch, ta, args, sel, line)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle sample)")
        line["cpu_baseline"] = cpu_baseline(w)
        if not args.no_cpu_configs:
            line["cpu_baseline_configs"] = cpu_oracle_configs()
    print(json.dumps(line))


def run_secondary(torch, ta, args, sel, line):
    if "decode" in sel:
        wd = WORKLOADS["paged_decode_b64"]
        ms, nbytes, tokens = bench_decode(torch, ta, wd, max(20, args.steps), max(100, args.warmup))
        line["paged_decode"] = {"workload": wd.name, "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                                "ms": round(ms, 4), "bytes": nbytes, "tokens": tokens,
                                "roofline": roofline_hbm(nbytes, ms, "decode_paged_lds_kernel", wd.name,
                                                         "decode_paged_lds_kernel + decode_combine_kernel")}
    for kv in ("fp8", "int8"):
        if f"decode_{kv}" not in sel:
            continue
        wd = WORKLOADS["paged_decode_b64"]
        ms, nbytes, tokens = bench_decode(torch, ta, wd, max(20, args.steps), max(100, args.warmup), kv=kv)
        line[f"paged_decode_{kv}"] = {
            "workload": wd.name, "kv_cache": kv, "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms": round(ms, 4), "bytes": nbytes, "tokens": tokens,
            "roofline": roofline_hbm(nbytes, ms, "decode_paged_q8_kernel", f"{wd.name}_{kv}",
                                     "decode_paged_q8_kernel + decode_combine_kernel")}
    if "mla" in sel:
        wm = WORKLOADS["mla_decode_b32"]
        ms = bench_mla(torch, ta, wm, max(20, args.steps), max(300, args.warmup))
        nbytes = mla_bytes(wm)
        line["mla_decode"] = {"workload": wm.name, "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                              "ms": round(ms, 4), "bytes": nbytes,
                              "tflops": round(mla_flops(wm) / (ms * 1e-3) / 1e12, 1),
                              "roofline": roofline_hbm(nbytes, ms, "mla_split_kernel", wm.name,
                                                       "mla_split_kernel + mla_combine_kernel")}
    for kv in ("fp8", "int8"):
        if f"mla_{kv}" in sel:
            wm = WORKLOADS["mla_decode_b32"]
            ms = bench_mla(torch, ta, wm, max(20, args.steps), max(300, args.warmup), kv=kv)
            nbytes = mla_bytes(wm, elem=1)
            kern = "mla_split_fp8mma_kernel" if kv == "fp8" else "mla_split_kernel"
            line[f"mla_decode_{kv}"] = {
                "workload": f"{wm.name} ({kv} latent cache)", "value": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "unit": "GB/s", "ms": round(ms, 4), "bytes": nbytes,
                "tflops": round(mla_flops(wm) / (ms * 1e-3) / 1e12, 1),
                "roofline": roofline_hbm(nbytes, ms, kern, f"{wm.name}_{kv}", f"{kern} + mla_combine_kernel")}
    if "long" in sel:
        wl = WORKLOADS["gqa_prefill_s131072"]
        wall_l, kern_l, _ = bench_prefill(torch, ta, wl, 2, 1)
        line["long_prefill"] = {"workload": wl.name, "value": round(wl.flops / (wall_l * 1e-3) / 1e12, 2),
                                "unit": "TFLOP/s", "ms_per_step": round(wall_l, 3),
                                "roofline": roofline_compute(wl.flops, kern_l, "prefill_bf16_kernel", wl.name)}
    if "chunked" in sel:
        wc = WORKLOADS["chunked_prefill_b4"]
        wall_c, kern_c = bench_chunked(torch, ta, wc, max(20, args.steps), max(100, args.warmup))
        line["chunked_prefill"] = {"workload": wc.name, "value": round(wc.flops / (wall_c * 1e-3) / 1e12, 2),
                                   "unit": "TFLOP/s", "ms_per_step": round(wall_c, 4),
                                   "ctx_lens": list(wc.ctx_lens), "new_lens": list(wc.new_lens),
                                   "step": "rope_table + kv_append_paged (rope k) + prefill_paged_rope (rope(q) fused)",
                                   "roofline": roofline_compute(wc.flops, kern_c, "prefill_bf16_kernel", wc.name)}
    if "swa" in sel:
        wsw = WORKLOADS["swa_prefill_s131072"]
        wall_w, kern_w, _ = bench_prefill(torch, ta, wsw, 5, 2, local_global=True)
        line["local_global_prefill"] = {
            "workload": wsw.name, "value": round(wsw.flops / (wall_w * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(wall_w, 3), "window": wsw.window, "n_lead": wsw.n_lead,
            "anchor_stride": wsw.anchor_stride, "flops_per_step": wsw.flops,
            "step": "rope(q) + rope(k) + prefill_local_global",
            "roofline": roofline_compute(wsw.flops, kern_w, "prefill_bf16_kernel", wsw.name)}
    if "dsa" in sel:
        ws_ = WORKLOADS["dsa_decode_b32"]
        wall_s, eager_s, ms = bench_dsa(torch, ta, ws_, max(20, args.steps), max(100, args.warmup))
        nb = dsa_bytes(ws_)
        total = sum(nb.values())
        line["dsa_decode"] = {
            "workload": ws_.name, "value": round(total / (wall_s * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(wall_s, 4), "launch": "one HIP graph of the three kernels, replayed",
            "eager_ms_per_step": round(eager_s, 4), "bytes_per_step": total, "topk": ws_.topk,
            "seqlen": ws_.seqlen, "step": "dsa_indexer + topk + mla_sparse_decode",
            "kernels": {k: {"ms": round(v, 4), "bytes": nb[k], "GB/s": round(nb[k] / (v * 1e-3) / 1e9, 1)}
                        for k, v in ms.items()},
            "roofline": roofline_hbm(nb["indexer"], ms["indexer"], "dsa_indexer_kernel", ws_.name)}


if __name__ == "__main__":
    main()
