#!/usr/bin/env python3
"""Benchmark of the fused DSA decode step on one MI355X.

Workload: decode at 128K context -- 8 independent sequences of 131,072 cached
tokens, top-k 2048, 64 absorbed query heads over 576-wide latent rows, a
32 x 128 indexer with integer-valued keys/queries and weights in [1, 4]
(synthetic, seeded).  A step is one ``dsa_decode_step`` call over the batch:
indexer scores of every cached token, exact top-k, sparse absorbed-MLA
attention, split merge.  Inputs are resident in HBM before timing starts;
steps rotate over several device replicas of the caches so that no step
finds its inputs in the 256 MB Infinity Cache left by the previous one.

Prints ONE JSON line.  ``value`` is queries per second; ``roofline`` is the
dominant kernel (the indexer score kernel): algorithmic bytes per launch over
its average duration, measured with HIP events on the launch stream;
``cpu_baseline`` is the CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import json

import numpy as np
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_score_m128k_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "deepseek_sparse_attention_amd", "csrc", "dsa_kernels.hip")
METRIC = "DSA decode queries/sec at 128K ctx, top-k 2048; achieved HBM GB/s vs peak"
KERNELS = ["score", "filter", "select", "attend", "merge"]


def algorithmic_bytes(w):
    """Bytes the method must move per query and per score launch (inputs
    read once, output written once; intermediates excluded)."""
    g = w.geom
    D = g["d_latent"] + g["d_rope"]
    rows = w.q_nvis.astype("int64") // g["kpool"]
    # keys: each sequence's visible rows once, however many of its queries read them
    seq_rows = {}
    for s_, r in zip(w.q_seq.tolist(), rows.tolist()):
        seq_rows[s_] = max(seq_rows.get(s_, 0), r)
    keys = np.array(list(seq_rows.values()), dtype=np.int64) * g["d_idx"] * 2
    qi_w = g["n_idx_heads"] * g["d_idx"] * 2 + g["n_idx_heads"] * 4
    kp, keep = g["kpool"], g["top_k"] // g["kpool"]
    kept = [int(n) if int(n) // kp <= keep else keep * kp + int(n) % kp for n in w.q_nvis]
    sel_rows = sum(kept) * D * 2
    q = w.n_q * g["n_heads"] * D * 2
    out = w.n_q * g["n_heads"] * g["d_latent"] * 4
    step = int(keys.sum()) + w.n_q * qi_w + sel_rows + q + out
    score_launch = int(keys.sum()) + w.n_q * qi_w
    return step, score_launch


def score_kernel_hash() -> str:
    """sha256 (16 hex digits) of the decode score kernel's source text, from
    its template line to its closing brace."""
    import hashlib
    src = open(KERNEL_SRC).read()
    i = src.index("template <bool STRIDE, bool F16, int NW>\n__global__ __launch_bounds__(64 * NW) void k_score(Args a) {")
    j = src.index("\n}\n", i) + 3
    return hashlib.sha256(src[i:j].encode()).hexdigest()[:16]


def measured_traffic(w):
    """HBM bytes per k_score launch from the committed rocprofv3 counter
    readings (FETCH_SIZE and WRITE_SIZE scaled by the copy calibration), or
    None if they were taken on another workload or another kernel source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("workload") != w.name or t.get("kernel_sha") != score_kernel_hash():
        return None
    return int(round((t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024))


def prefill_score_flops(w) -> int:
    """MFMA flops of the prefill scorer: 2 x 32 heads x 128 per scored row."""
    g = w.geom
    rows = w.q_nvis.astype("int64") // g["kpool"]
    scored = rows[rows > g["top_k"] // g["kpool"]]
    return int(2 * g["n_idx_heads"] * g["d_idx"] * scored.sum())


def cpu_baseline(w, budget_s: float):
    """The oracle as it stands, on whole steps of the same workload, repeated
    until about budget_s seconds of wall time have passed (at most 64 steps),
    on every host thread; then on one thread, one whole step of the tiny
    decode (one query over 4,096 tokens) and one query of the 8 x 64K decode
    (its first sequence and query, drawn from the same seeds)."""
    from oracle import oracle as O
    from deepseek_sparse_attention_amd import inputs as I
    threads = O.max_threads()
    done, t0 = 0, time.perf_counter()
    while True:
        O.decode_step(w.geom, w.q_seq, w.q_nvis, w.idx_q, w.idx_w, w.idx_k, w.q, w.cache)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= 64:
            break
    res = {"value": round(done * w.n_q / el, 3), "unit": "queries/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} full step(s) of the same workload ({done * w.n_q} queries), "
                     f"{el:.1f} s wall on {threads} OpenMP threads of {cpu_model()}"}
    one = {}
    O.set_threads(1)
    try:
        for name, sw in (("c0", I.config("c0")),
                         ("c1_one_query", I.make_workload("c1", 1, I.GEOM_TOKEN, 1, 65536, [0], [65536]))):
            t0 = time.perf_counter()
            O.decode_step(sw.geom, sw.q_seq, sw.q_nvis, sw.idx_q, sw.idx_w, sw.idx_k, sw.q, sw.cache)
            el = time.perf_counter() - t0
            one[name] = {"queries_per_s": round(sw.n_q / el, 3), "s": round(el, 3)}
    finally:
        O.set_threads(threads)
    res["single_thread"] = one
    return res


def stream_read_rate(gib: int = 1, reps: int = 20) -> dict:
    """The plainest streaming read of HBM on this device (the library's
    non-temporal grid-stride probe over a buffer of `gib` GiB, which no cache
    holds): the practical read roof beside the published 8 TB/s."""
    import torch
    from deepseek_sparse_attention_amd import binding as B
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda").fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        B.stream_read(buf, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        B.stream_read(buf, sink)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    gbps = buf.numel() / (us * 1e-6) / 1e9
    del buf
    return {"GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes": gib << 30,
            "us": round(us, 2)}


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo, or "unknown CPU"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="m128k")
    ap.add_argument("--batch", type=int, default=8, help="sequences at the 128K decode point (m128k only)")
    ap.add_argument("--window", type=int, default=1,
                    help="query rows per sequence at the last positions (speculative verify; m128k only)")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--producer", action="store_true",
                    help="time the k-pool key producer instead: one bulk append of 2^20 - 1 tokens")
    ap.add_argument("--absorb", action="store_true",
                    help="time the absorption GEMMs instead (absorb + project, 8 and 512 queries)")
    ap.add_argument("--prepare", action="store_true",
                    help="time the indexer input preparation (rope + Hadamard + rounding, key append) instead")
    ap.add_argument("--f16", action="store_true", help="indexer queries and keys in f16 (prepare and decode)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (to scale byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(sharding over several GPUs is described, not implemented)", file=sys.stderr)
        return 2

    if args.producer:
        return run_producer(args)
    if args.prepare:
        return run_prepare(args)
    if args.absorb:
        return run_absorb(args)

    import torch
    from deepseek_sparse_attention_amd import binding as B
    from deepseek_sparse_attention_amd import inputs as I
    from deepseek_sparse_attention_amd.workload import DeviceWorkload

    torch.cuda.set_device(0)
    B.device_check()
    t0 = time.perf_counter()
    if args.config == "m128k" and args.window > 1:
        w = I.decode_window(args.batch, args.window, poison_beyond=False)
    elif args.config == "m128k":
        w = I.decode_128k(args.batch, poison_beyond=False)
    else:
        w = I.config(args.config, poison_beyond=False)
    print(f"[bench] {args.config}: generated in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    reps = [DeviceWorkload(w) for _ in range(max(1, args.replicas))]
    R = len(reps)
    torch.cuda.synchronize()
    print(f"[bench] {R} device replicas resident", file=sys.stderr, flush=True)

    for i in range(args.warmup):
        reps[i % R].decode_step()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        reps[i % R].decode_step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / args.steps
    qps = w.n_q / (ms_step * 1e-3)
    step_bytes, score_bytes = algorithmic_bytes(w)
    print(f"[bench] {ms_step * 1e3:.1f} us/step, wall {wall * 1e6 / args.steps:.1f} us/step", file=sys.stderr,
          flush=True)

    # ---- per-kernel durations: each kernel of the same fused step launched
    # with its own start and stop events, over a second pass
    n_k = 2 * len(KERNELS)
    n_rep = min(args.steps, 100)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_k)] for _ in range(n_rep)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(n_rep):
        B.set_timing_events(evs[i])
        reps[i % R].decode_step()
    B.set_timing_events(None)
    ran = B.timing_ran()                # the same kernels run at every step of one workload
    torch.cuda.synchronize()
    names = KERNELS
    per = {k: 0.0 for k in names}
    for row in evs:
        for j, k in enumerate(names):
            if (ran >> j) & 1:          # a kernel that did not run leaves its events unrecorded
                per[k] += row[2 * j].elapsed_time(row[2 * j + 1]) * 1e3 / n_rep
    score_us = per["score"]
    prefill = w.n_seq == 1 and w.n_q > 1
    if prefill:
        flops = prefill_score_flops(w)
        achieved = flops / (score_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": "k_score_prefill", "achieved": round(achieved, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": None, "flops_per_launch": flops}
    else:
        achieved = score_bytes / (score_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": "k_score", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(w),
                "bytes_per_launch": score_bytes}

    res = {
        "metric": METRIC,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": _workload_name(w), "batch": w.n_q, "context": int(w.q_nvis.max()),
                   "top_k": w.geom["top_k"], "replicas": R},
        "step_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_hbm": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernels_us": {k: round(v, 2) for k, v in per.items()},
        "roofline": roof,
    }
    if not prefill:
        res["stream_read"] = stream_read_rate()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = src.numel()
    if not args.no_cpu_baseline:
        del reps
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


def run_producer(args) -> int:
    """k-pool key producer on the k-pool buffer size: one sequence, 2^20 - 1
    tokens appended at once (262,143 pools); cells are 512 B (key | gate),
    pool keys 256 B.  Inputs resident in HBM; 4 replicas rotated."""
    import torch
    from deepseek_sparse_attention_amd import binding as B

    torch.cuda.set_device(0)
    B.device_check()
    T = (1 << 20) - 1
    P = T // 4
    g = torch.Generator(device="cpu").manual_seed(20261202)
    pos = torch.randn((4, 128), generator=g).cuda()
    reps = []
    for r in range(max(1, args.replicas)):
        cells = (torch.randn((1, T, 256), generator=g) * 2).to(torch.bfloat16).view(torch.int16).cuda()
        reps.append(cells)
    n_tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_new = torch.full((1,), T, dtype=torch.int32, device="cuda")
    roll = torch.zeros((1, 4, 256), dtype=torch.int16, device="cuda")
    keys = torch.empty((1, P, 128), dtype=torch.int16, device="cuda")
    R = len(reps)
    for i in range(args.warmup):
        B.pool_append(n_tok, n_new, T, reps[i % R], roll, keys, pos)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        B.pool_append(n_tok, n_new, T, reps[i % R], roll, keys, pos)
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / args.steps
    nbytes = T * 512 + P * 256
    gbps = nbytes / (us * 1e-6) / 1e9
    res = {
        "metric": "k-pool key producer: pool keys per second (bulk append of 2^20 - 1 tokens)",
        "value": round(P / (us * 1e-6), 1), "unit": "pool keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in, fp32 math, bf16 out", "data": "synthetic",
        "config": {"workload": f"k-pool producer: 1 sequence, {T} tokens appended, {P} pools", "replicas": R},
        "roofline": {"bound": "hbm", "kernel": "k_pool_append", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        n = 1 << 16
        cells = reps[0][:, :n].cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        O.pool_append(np.zeros(1, np.int32), np.array([n], np.int32), cells,
                      np.zeros((1, 4, 256), np.uint16), np.zeros((1, n // 4, 128), np.uint16),
                      pos.cpu().numpy())
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round((n // 4) / el, 1), "unit": "pool keys/s", "cores": 1,
                               "kind": "oracle", "sample": f"{n} tokens ({n // 4} pools) of the same buffer, "
                                                           f"{el:.2f} s, one thread (the producer oracle is serial)"}
    print(json.dumps(res), flush=True)
    return 0


def run_absorb(args) -> int:
    """Absorption GEMMs (absorb the key up-projection into the query, project
    the attention output through the value up-projection), 64 heads, bf16
    weights [64][256][512] each.  Timed for a decode batch of 8 queries (the
    32 MiB of weights dominate) and a 512-query prefill chunk; both are
    HBM-bound (the chunk does about 115 and 150 flop per byte, under the
    ~312 flop/B ridge of 2.5 PFLOP/s over 8 TB/s); 4 weight replicas rotated."""
    import torch
    from deepseek_sparse_attention_amd import binding as B

    torch.cuda.set_device(0)
    B.device_check()
    g = torch.Generator(device="cpu").manual_seed(20261202)
    R = max(1, args.replicas)
    wk = [(torch.randn((64, 256, 512), generator=g) * 0.05).to(torch.bfloat16).view(torch.int16).cuda() for _ in range(R)]
    wv = [(torch.randn((64, 256, 512), generator=g) * 0.05).to(torch.bfloat16).view(torch.int16).cuda() for _ in range(R)]

    def timed(n_q):
        qn = torch.randn((n_q, 64, 256), generator=g).to(torch.bfloat16).view(torch.int16).cuda()
        qr = torch.randn((n_q, 64, 64), generator=g).to(torch.bfloat16).view(torch.int16).cuda()
        qa = torch.empty((n_q, 64, 576), dtype=torch.int16, device="cuda")
        o = torch.randn((n_q, 64, 512), generator=g).cuda()
        ctx = torch.empty((n_q, 64, 256), device="cuda")
        for i in range(args.warmup):
            B.absorb_query(qn, qr, wk[i % R], qa)
            B.project_output(o, wv[i % R], ctx)
        torch.cuda.synchronize()
        # each kernel's `steps` launches back to back (weights rotated),
        # captured in a HIP graph so that the host's per-call cost does not
        # stretch the few-microsecond decode launches
        graphs = [torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()]
        with torch.cuda.graph(graphs[0]):
            for i in range(args.steps):
                B.absorb_query(qn, qr, wk[i % R], qa)
        with torch.cuda.graph(graphs[1]):
            for i in range(args.steps):
                B.project_output(o, wv[i % R], ctx)
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        graphs[0].replay()
        ev[1].record()
        graphs[1].replay()
        ev[2].record()
        torch.cuda.synchronize()
        ta = ev[0].elapsed_time(ev[1]) * 1e3 / args.steps
        tp = ev[1].elapsed_time(ev[2]) * 1e3 / args.steps
        wbytes = 64 * 256 * 512 * 2
        b_abs = wbytes + n_q * 64 * (256 + 64 + 576) * 2
        b_prj = wbytes + n_q * 64 * (512 + 256) * 4
        fl = 2 * n_q * 64 * 256 * 512
        return {"queries": n_q, "absorb_us": round(ta, 2), "project_us": round(tp, 2),
                "absorb_GBps": round(b_abs / (ta * 1e-6) / 1e9, 1), "project_GBps": round(b_prj / (tp * 1e-6) / 1e9, 1),
                "absorb_TFLOPs": round(fl / (ta * 1e-6) / 1e12, 1), "project_TFLOPs": round(fl / (tp * 1e-6) / 1e12, 1),
                "bytes": b_abs + b_prj, "flops": 2 * fl}

    dec, pre = timed(8), timed(512)
    us = dec["absorb_us"] + dec["project_us"]
    gbps = dec["bytes"] / (us * 1e-6) / 1e9
    res = {
        "metric": "absorption GEMMs (absorb + project), decode batch of 8 queries per second",
        "value": round(8 / (us * 1e-6), 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "absorb q_nope 256 -> 512 and project o 512 -> 256 per head, 64 heads, "
                               "bf16 weights [64][256][512] x 2", "replicas": R},
        "roofline": {"bound": "hbm", "kernel": "k_absorb + k_project", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": dec["bytes"]},
        "decode_8": dec, "prefill_512": pre,
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        rng = np.random.default_rng(1)
        qn = rng.integers(-3, 4, size=(8, 64, 256)).astype(np.uint16)
        t0 = time.perf_counter()
        O.absorb_query(qn, None, wk[0].cpu().numpy().view(np.uint16))
        O.project_output(rng.standard_normal((8, 64, 512)).astype(np.float32), wv[0].cpu().numpy().view(np.uint16))
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(8 / el, 1), "unit": "queries/s", "cores": O.max_threads(),
                               "kind": "oracle", "sample": f"one decode batch of 8 queries, {el:.2f} s"}
    print(json.dumps(res), flush=True)
    return 0


def run_prepare(args) -> int:
    """Indexer input preparation: rope on the tail 64 dimensions, the
    orthonormal Walsh-Hadamard rotation and rounding to the indexer's 16-bit
    format, for the indexer queries of a step (32 heads x 128, float32 in) and
    the keys it appends to the key cache.  Timed for a decode batch (8
    queries, 8 keys) and a 512-token prefill chunk (512 queries, 512 keys);
    the decode batch is the headline, the chunk is the bandwidth case."""
    import torch
    from deepseek_sparse_attention_amd import binding as B
    from deepseek_sparse_attention_amd import inputs as I

    torch.cuda.set_device(0)
    B.device_check()
    geom = dict(I.GEOM_TOKEN, idx_f16=int(args.f16))
    T = 131072

    def timed(n_q, n_new, n_seq):
        # decode: query i and key i belong to sequence i, at position T - 1;
        # chunk: one sequence, queries and keys at positions T - n .. T - 1
        q_in, k_in = I.indexer_projections(11, n_q, n_new)
        dev = "cuda"
        per = n_new // n_seq
        q_seq = torch.arange(n_q, dtype=torch.int32, device=dev) % n_seq
        q_nvis = (T - per + 1 + torch.arange(n_q, dtype=torch.int32, device=dev) // n_seq).to(torch.int32)
        b = B.batch(q_seq, q_nvis, T, n_seq)
        k_seq = torch.arange(n_new, dtype=torch.int32, device=dev) % n_seq
        k_pos = (T - per + torch.arange(n_new, dtype=torch.int32, device=dev) // n_seq).to(torch.int32)
        d_q, d_k = torch.from_numpy(q_in).to(dev), torch.from_numpy(k_in).to(dev)
        q_out = torch.empty((n_q, 32, 128), dtype=torch.int16, device=dev)
        cache = torch.zeros((n_seq, T, 128), dtype=torch.int16, device=dev)
        for _ in range(args.warmup):
            B.index_prepare(geom, b, d_q, q_out, k_seq, k_pos, d_k, cache, T)
        torch.cuda.synchronize()
        # the call takes less device time than its host-side launch: time it
        # replayed from a captured graph of `per_graph` calls
        per_graph = 50
        graph, side = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side), torch.cuda.graph(graph, stream=side):
            for _ in range(per_graph):
                B.index_prepare(geom, b, d_q, q_out, k_seq, k_pos, d_k, cache, T)
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // per_graph)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            graph.replay()
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) * 1e3 / (reps * per_graph)
        nbytes = n_q * (32 * 128 * (4 + 2) + 4) + n_new * (128 * (4 + 2) + 8)
        # reference at the same size: torch's float32 -> bfloat16 cast of the
        # queries (the same bytes read and written per element), same timing
        cast_out = torch.empty((n_q, 32, 128), dtype=torch.bfloat16, device=dev)
        cgraph = torch.cuda.CUDAGraph()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side), torch.cuda.graph(cgraph, stream=side):
            for _ in range(per_graph):
                cast_out.copy_(d_q)
        torch.cuda.current_stream().wait_stream(side)
        cgraph.replay()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            cgraph.replay()
        ev[1].record()
        torch.cuda.synchronize()
        cast_us = ev[0].elapsed_time(ev[1]) * 1e3 / (reps * per_graph)
        return {"queries": n_q, "keys": n_new, "us": round(us, 3), "bytes": nbytes,
                "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                "torch_cast_us": round(cast_us, 3), "torch_cast_bytes": n_q * 32 * 128 * 6}

    dec, pre = timed(8, 8, 8), timed(512, 512, 1)
    res = {
        "metric": "indexer input preparation, decode batch of 8 queries + 8 appended keys per second",
        "value": round(8 / (dec["us"] * 1e-6), 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dec["us"] * 1e-3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "indexer rope + Hadamard + rounding to " + ("f16" if args.f16 else "bf16")
                               + ", 32 heads x 128, keys appended at position 131071"},
        "roofline": {"bound": "hbm", "kernel": "k_index_prep (512-token chunk)", "achieved": pre["GBps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(pre["GBps"] / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": pre["bytes"]},
        "decode_8": dec, "prefill_512": pre,
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        q_in, k_in = I.indexer_projections(11, 8, 8)
        t0 = time.perf_counter()
        O.index_prepare(np.full(8, T, np.int32), q_in, np.arange(8, dtype=np.int32), np.full(8, T - 1, np.int32),
                        k_in, np.zeros((8, T, 128), np.uint16), 64, args.f16)
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(8 / el, 1), "unit": "queries/s", "cores": O.max_threads(),
                               "kind": "oracle", "sample": f"one decode batch of 8 queries + 8 keys, {el:.3f} s"}
    print(json.dumps(res), flush=True)
    return 0


def _workload_name(w) -> str:
    g = w.geom
    shape = (f"top-k {g['top_k']}, kpool {g['kpool']}, {g['n_heads']} heads x {g['d_latent'] + g['d_rope']} "
             f"latent rows, indexer {g['n_idx_heads']}x{g['d_idx']}")
    if w.n_seq == 1 and w.n_q > 1:
        return (f"{w.name}: prefill chunk of {w.n_q} consecutive positions ending at {int(w.q_nvis.max())} "
                f"cached tokens, {shape}")
    if w.n_q > w.n_seq:
        return (f"{w.name}: verify windows, {w.n_seq} sequences x {w.n_q // w.n_seq} rows at the last positions "
                f"of {int(w.q_nvis.max())} cached tokens, {shape}")
    return f"{w.name}: decode, {w.n_q} sequences x {int(w.q_nvis.max())} cached tokens, {shape}"


if __name__ == "__main__":
    sys.exit(main())
