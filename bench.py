#!/usr/bin/env python3
"""Prefill throughput of the decision path on one MI355X.

A step is one whole prefill-and-decide of the workload's request (embedding,
every layer, readout) through the library's resident-input plan: token ids
and metadata already sit in device memory when the timed region starts.
Prints one JSON line with the throughput (prefill tokens/s), ms per request,
the dominant kernel's roofline fraction (HIP events recorded by the library
on the launch stream), the attention and scan fractions, the boundary call
s1_prefill_decide (host arrays in and out) timed per call, the same figures
for the 16-request and branched workloads on the same weights, and the CPU
oracle's throughput on the whole request.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s and ms/request, 4B-shape hybrid bf16 on 1 MI355X"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def requests_in(batch):
    """A request is a sequence that is not a prefix of another sequence: a
    prefix and its branches form one request."""
    import numpy as np
    prefixes = set(int(p) for p in batch.prefix_of if p >= 0)
    return sum(1 for i in range(batch.n_seqs) if batch.prefix_of[i] < 0 and i not in prefixes) + len(prefixes)


def gemm_flops(shape, T):
    """Algorithmic flops of each projection GEMM family for T tokens."""
    d, F = shape.d_model, shape.ffn
    H, dk, dv = shape.la_heads, shape.la_dk, shape.la_dv
    Hq, Hkv, hd = shape.fa_q_heads, shape.fa_kv_heads, shape.fa_head_dim
    return {
        "gemm_la_in": 2 * T * d * (2 * H * dk + H * dv + H),
        "gemm_fa_qkv": 2 * T * d * (Hq + 2 * Hkv) * hd,
        # per launch averaged over the layers (K = H dv on linear layers, Hq hd on full ones)
        "gemm_o": 2 * T * d * (shape.n_linear * H * dv + shape.n_full * Hq * hd) / shape.n_layers,
        "gemm_gate_up": 2 * T * d * 2 * F,
        "gemm_down": 2 * T * F * d,
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, weights, batch, budget_s=30.0):
    """The CPU oracle as it stands (float32 mode, numpy's BLAS on the host
    cores) timed on the whole request, end to end: prefill_decide over every
    layer and the readout, the per-layer weight decode included.  One
    warm-up, then the median of three runs, or fewer runs when one takes
    more than a third of the budget."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    om = oracle.OracleModel(shape, weights.tensors, dtype=np.float32)
    times = []
    t0 = time.time()
    oracle.prefill_decide(om, batch)
    warm = time.time() - t0
    n_runs = 3 if warm * 3 <= budget_s else 1
    for _ in range(n_runs):
        t0 = time.time()
        oracle.prefill_decide(om, batch)
        times.append(time.time() - t0)
    med = float(np.median(times))
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in info if i.get("user_api") == "blas")
    return {"value": batch.n_tokens / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "ms_per_request": round(med * 1e3 / requests_in(batch), 1),
            "sample": f"float32 oracle prefill_decide of the whole {batch.n_tokens}-token request "
                      f"({batch.n_questions} questions), median of {n_runs} after one warm-up "
                      f"({', '.join(f'{t:.2f}' for t in times)} s); {len(os.sched_getaffinity(0))} host cores "
                      f"visible",
            "cpu": cpu_model(), "blas": blas or "unknown"}


def decide_leg(model, batch, warmup=2, timed=20):
    """s1_prefill_decide, host arrays in and out (the boundary call): wall
    time per call from entry to return with the results on the host, the
    copies of the request and the results included, and the device time of
    the same calls (HIP events inside the call)."""
    import numpy as np
    for _ in range(warmup):
        model.decide(batch)
    wall, dev = [], []
    for _ in range(timed):
        _, _, t = model.decide(batch)
        wall.append(t["wall_us"] / 1e3)
        dev.append(t["device_us"] / 1e3)
    wall = np.asarray(wall)
    med = float(np.median(wall))
    return {"calls": timed, "warmup": warmup, "wall_ms_median": round(med, 4),
            "wall_ms_p95": round(float(np.percentile(wall, 95)), 4), "wall_ms_mean": round(float(wall.mean()), 4),
            "wall_ms_min": round(float(wall.min()), 4), "device_ms_median": round(float(np.median(dev)), 4),
            "tokens_per_s_at_median": round(batch.n_tokens / (med / 1e3), 1)}


def attention_flops(shape, batch):
    """Algorithmic attention flops per step: 4 Hq hd per visible (query, key)
    pair (the causal half, a branch's prefix keys included), every full
    layer."""
    pre = batch.prefix_of
    pairs = 0
    for i in range(batch.n_seqs):
        L = int(batch.seq_lens[i])
        P = int(batch.seq_lens[pre[i]]) if pre[i] >= 0 else 0
        pairs += L * (L + 1) // 2 + P * L
    return 4 * shape.fa_q_heads * shape.fa_head_dim * pairs * shape.n_full


def attention_roofline(shape, batch, prof, steps_p):
    if "attention" not in prof:
        return None
    fl = attention_flops(shape, batch)
    us = prof["attention"][1] / steps_p
    tf = fl / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4), "flops_per_step": fl, "us_per_step": round(us, 1),
            "launches_per_step": prof["attention"][0] // steps_p}


def workload_leg(model, name, args, stream):
    """Another workload of the same shape on the loaded model: the plan
    replayed as a HIP graph (tokens/s, ms/request), per-kernel times, the
    attention and scan rooflines, and the boundary call's wall time."""
    import torch
    from s1_workloads import make_batch, shape_of
    shape = shape_of(name)
    batch = make_batch(name)
    plan = model.plan(batch)
    dp = torch.zeros(max(plan.n_options, 1), dtype=torch.float32, device="cuda")
    dd = torch.zeros((max(plan.n_questions, 1), 6), dtype=torch.float32, device="cuda")
    sp = stream.cuda_stream
    plan.set_graph(True)
    steps = max(3, args.steps // 2)
    for _ in range(2):
        plan.run(dp.data_ptr(), dd.data_ptr(), sp)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        plan.run(dp.data_ptr(), dd.data_ptr(), sp)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    plan.set_graph(False)
    prof = {}
    n_prof = 2
    for _ in range(n_prof):
        for k, (n, us) in plan.profile(dp.data_ptr(), dd.data_ptr(), sp).items():
            a, b = prof.get(k, (0, 0.0))
            prof[k] = (a + n, b + us)
    tokens = plan.tokens
    plan.free()
    reqs = requests_in(batch)
    gemm_us = sum(prof[k][1] for k in ("gemm_la_in", "gemm_fa_qkv", "gemm_o", "gemm_gate_up", "gemm_down")
                  if k in prof) / n_prof
    all_gemm_flops = 2 * tokens * shape.linear_params()
    return {"tokens_per_step": int(tokens), "requests_per_step": reqs, "questions_per_step": int(batch.n_questions),
            "steps": steps, "ms_per_step": round(ms, 3), "tokens_per_s": round(tokens / (ms / 1e3), 1),
            "ms_per_request": round(ms / reqs, 3),
            "kernels": {k: {"launches_per_step": n // n_prof, "us_per_step": round(us / n_prof, 1)}
                        for k, (n, us) in sorted(prof.items())},
            "all_gemms_tflops": round(all_gemm_flops / (gemm_us * 1e-6) / 1e12, 1),
            "attention": attention_roofline(shape, batch, prof, n_prof),
            "scan": scan_roofline(shape, batch, tokens, prof, n_prof),
            "prefill_decide": decide_leg(model, batch, warmup=2, timed=max(5, args.steps // 2))}


GEMM_SOURCE = os.path.join(ROOT, "prefill_only_decision_amd", "csrc", "gemm.hip")
COPY_BYTES = 1 << 30   # the calibration copy reads and writes this many bytes


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_gemm_gate_up_{workload}.json")


def source_digest():
    import hashlib
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_counters(fetch_csv, write_csv, workload):
    """HBM bytes per launch of the FFN gate/up GEMM (the epilogue-3 GEMM
    kernel) from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch), each scaled by what the same counter reads for the plain
    1 GiB copy that --calibrate-copy adds to the run."""
    import csv
    import re
    import statistics

    def per_kernel(path, counter):
        gemm, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, kib = r["Kernel_Name"], float(r["Counter_Value"])
            if re.search(r"gemm_\w+_kernel<.*, 3(, (true|false))?>\(s1::GemmArgs\)", name):
                gemm.append(kib * 1024)
            elif "elementwise" in name and kib * 1024 > COPY_BYTES / 2:
                copy.append(kib * 1024)
        if not gemm or not copy:
            raise SystemExit(f"{path}: no {counter} values for the gate/up GEMM or the calibration copy")
        return statistics.median(gemm), statistics.median(copy)

    g_f, c_f = per_kernel(fetch_csv, "FETCH_SIZE")
    g_w, c_w = per_kernel(write_csv, "WRITE_SIZE")
    rec = {"kernel": "gemm_gate_up (epilogue 3, SwiGLU)", "workload": workload,
           "fetch_bytes_per_launch": round(g_f * COPY_BYTES / c_f),
           "write_bytes_per_launch": round(g_w * COPY_BYTES / c_w),
           "raw_fetch_bytes": round(g_f), "raw_write_bytes": round(g_w),
           "copy_bytes": COPY_BYTES, "copy_fetch_bytes": round(c_f), "copy_write_bytes": round(c_w),
           "gemm_source_sha256": source_digest(),
           "commands": [f"rocprofv3 --pmc {c} -d gpurun_out/pmc_{c.lower()} -o run -f csv -- python3 bench.py "
                        f"--workload {workload} --steps 2 --warmup 1 --no-cpu-baseline --no-serve --no-peaks "
                        f"--no-readout-stress --no-other-workloads --profile-steps 1 --calibrate-copy"
                        for c in ("FETCH_SIZE", "WRITE_SIZE")]}
    rec["traffic_bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    with open(traffic_file(workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def stored_traffic(workload):
    """Counter-measured HBM bytes per gate/up launch, or None when missing or
    taken on another version of the GEMM source."""
    try:
        rec = json.load(open(traffic_file(workload)))
    except (OSError, ValueError):
        return None
    return rec["traffic_bytes_per_launch"] if rec.get("gemm_source_sha256") == source_digest() else None


def scan_roofline(shape, batch, tokens, prof, steps_p):
    """Achieved HBM bandwidth of the linear-attention scan per step: per
    token and layer it must read q, k, v (bf16) and the log decay (fp32) and
    write o (bf16); per prefix and layer it writes the fp32 final state and
    each branch reads it.  The scan is latency-bound at a few hundred tokens
    (a few (sequence, head) chains, one 64-token chunk apart)."""
    if shape.la_kind != "gla" or "la_scan" not in prof:
        return None
    H, dk, dv = shape.la_heads, shape.la_dk, shape.la_dv
    per_token = H * (2 * dk + dv) * 2 + 4 * H + H * dv * 2
    pre = batch.prefix_of
    n_states = int(len(set(int(p) for p in pre if p >= 0)) + int((pre >= 0).sum()))
    per_layer = tokens * per_token + n_states * H * dk * dv * 4
    us = prof["la_scan"][1] / steps_p
    gbs = per_layer * shape.n_linear / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_token_layer": per_token,
            "bytes_per_step": per_layer * shape.n_linear, "us_per_step": round(us, 1),
            "launches_per_step": prof["la_scan"][0] // steps_p}


def measure_peaks(stream, reps=5):
    """Achievable peaks on this GPU, in the same job: a register-resident
    bf16 matrix-instruction loop (two four-wave workgroups per CU, eight
    independent accumulators per wave) and a 1 GiB streaming copy (bytes
    read + bytes written over the time)."""
    import torch

    from prefill_only_decision_amd import binding as B

    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sp = stream.cuda_stream
    seed = torch.randint(-2 ** 15, 2 ** 15, (1024,), dtype=torch.int16, device="cuda")
    seed = torch.where((seed & 0x7F80) == 0x7F80, seed & ~0x4000, seed)   # no inf / nan patterns
    blocks, iters = 2 * n_cu, 20000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    t = timed(lambda: B.mfma_peak(seed.data_ptr(), blocks, iters, out.data_ptr(), sp))
    flops = blocks * 4 * 8 * iters * 2 * 32 * 32 * 16
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    tc = timed(lambda: B.stream_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, sp))
    sink = torch.empty(1024, dtype=torch.int32, device="cuda")
    tr = timed(lambda: B.stream_read(src.data_ptr(), COPY_BYTES, sink.data_ptr(), sp))
    del src, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(flops / t / 1e12, 1), "hbm_copy_gbs": round(2 * COPY_BYTES / tc / 1e9, 1),
            "hbm_read_gbs": round(COPY_BYTES / tr / 1e9, 1),
            "mfma_probe": f"{blocks} workgroups x 4 waves x 8 x {iters} v_mfma_f32_32x32x16_bf16 on registers",
            "copy_probe": f"{COPY_BYTES} bytes read + written, 16-byte non-temporal accesses",
            "read_probe": f"{COPY_BYTES} bytes read, same accesses", "cus": n_cu}


def add_measured_fraction(obj, peaks, key):
    """Fraction of the measured peak: the MFMA loop for MFMA-bound kernels;
    for HBM-bound kernels (mostly reads) the faster of the copy and the
    read-only stream."""
    if obj and peaks:
        peak = peaks[key] if key != "hbm" else max(peaks["hbm_copy_gbs"], peaks["hbm_read_gbs"])
        obj["frac_of_measured_peak"] = round(obj["achieved"] / peak, 4)


READOUT_STRESS_Q, READOUT_STRESS_K = 4096, 10


def readout_stress_leg(shape, stream, reps=20):
    """The decision readout at a declared stress shape (4,096 questions x 10
    options on the model's width and vocabulary), where it moves enough
    bytes to be measured against HBM bandwidth: the real readouts read under
    1 MB and are latency-bound.  Bytes: each question's fp32 row, its
    options' bf16 embedding rows and the final-norm gains."""
    import numpy as np
    import torch

    from prefill_only_decision_amd import binding as B

    Q, K, d, V = READOUT_STRESS_Q, READOUT_STRESS_K, shape.d_model, shape.vocab
    rng = np.random.default_rng(12)
    g = torch.Generator(device="cuda").manual_seed(12)
    E = (torch.randn(V, d, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    x = torch.randn(Q, d, device="cuda", generator=g)
    wf = torch.ones(d, device="cuda")
    rows = torch.arange(Q, dtype=torch.int32, device="cuda")
    offs = torch.arange(0, Q * K + 1, K, dtype=torch.int32, device="cuda")
    ids = np.concatenate([rng.choice(V, K, replace=False) for _ in range(Q)]).astype(np.int32)
    ids = torch.from_numpy(ids).cuda()
    qt = torch.zeros(Q, dtype=torch.uint8, device="cuda")
    probs = torch.empty(Q * K, dtype=torch.float32, device="cuda")
    dec = torch.empty((Q, 6), dtype=torch.float32, device="cuda")
    sp = stream.cuda_stream

    def run():
        B.readout(B.S1_BF16, x.data_ptr(), d, wf.data_ptr(), 1e-6, E.data_ptr(), Q, rows.data_ptr(),
                  offs.data_ptr(), ids.data_ptr(), qt.data_ptr(), probs.data_ptr(), dec.data_ptr(), sp)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = Q * d * 4 + Q * K * d * 2 + d * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    del E, x
    torch.cuda.empty_cache()
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "questions": Q, "options_per_question": K,
            "bytes_per_launch": nbytes, "us_per_launch": round(us, 2)}


SERVE_BUCKETS = tuple(range(256, 2049, 128))   # length buckets, 128 tokens apart


def serve_leg(model, shape, stream, n_requests=48):
    """Request replay at concurrency 1, 8 and 16 (the pages' protocol:
    warm p50 / p95 latency, requests/s and decisions/s at predeclared
    concurrency).  Requests are drawn like the packed 16-request workload:
    one sequence of L ~ U[256, 2048] tokens with 1-6 questions.  At
    concurrency 1 each request is copied into the smallest length-bucket
    plan that holds it and its captured HIP graph is replayed (a plan built
    per request is timed beside it); at concurrency c > 1, c requests arrive
    together and run as one packed request (plan built per group).  Latency
    is host wall time from arrival to the request's outputs on the host,
    after one excluded warm-up round per mode."""
    import numpy as np
    import torch
    from s1_workloads.batch import random_batch
    rng = np.random.default_rng(2024)
    reqs = [random_batch(shape.vocab, [int(rng.integers(256, 2049))], seed=[77, k],
                         questions_per_seq=[int(rng.integers(1, 7))]) for k in range(n_requests)]
    sp = stream.cuda_stream
    max_q, max_o = 6, 64
    cap = max_o + 2 * max_q
    dp = torch.zeros(16 * cap, dtype=torch.float32, device="cuda")
    dd = torch.zeros((16 * max_q, 6), dtype=torch.float32, device="cuda")

    def stats(lat, total_s, n_dec):
        lat = np.sort(np.asarray(lat) * 1e3)
        return {"p50_ms": round(float(np.percentile(lat, 50)), 3), "p95_ms": round(float(np.percentile(lat, 95)), 3),
                "requests_per_s": round(len(lat) / total_s, 1), "decisions_per_s": round(n_dec / total_s, 1)}

    buckets = {L: model.bucket_plan(L, max_q, max_o) for L in SERVE_BUCKETS}
    for b in buckets.values():
        b.set_graph(True)

    def one_bucket(r):
        L = int(r.seq_lens[0])
        plan = buckets[min(x for x in SERVE_BUCKETS if x >= L)]
        plan.update(r)
        plan.run(dp.data_ptr(), dd.data_ptr(), sp)
        torch.cuda.synchronize()
        _ = dp[:int(r.opt_offsets[-1])].cpu()

    def one_fresh(r):
        plan = model.plan(r)
        plan.run(dp.data_ptr(), dd.data_ptr(), sp)
        torch.cuda.synchronize()
        _ = dp[:int(r.opt_offsets[-1])].cpu()
        plan.free()

    out = {"requests": n_requests, "request_mix": "one sequence, L ~ U[256, 2048], 1-6 questions",
           "buckets": list(SERVE_BUCKETS)}
    for name, fn in (("c1_bucket_graphs", one_bucket), ("c1_plan_per_request", one_fresh)):
        for L in SERVE_BUCKETS:                      # warm-up: capture every bucket's graph once
            fn(random_batch(shape.vocab, [L], seed=[78, L], questions_per_seq=[1]))
        lat = []
        t0 = time.perf_counter()
        for r in reqs:
            a = time.perf_counter()
            fn(r)
            lat.append(time.perf_counter() - a)
        out[name] = stats(lat, time.perf_counter() - t0, sum(r.n_questions for r in reqs))
    for b in buckets.values():
        b.free()
    from s1_workloads.batch import _assemble
    for c in (8, 16):
        groups = [reqs[i:i + c] for i in range(0, n_requests, c)]
        lat, n_dec = [], 0

        def run_group(g):
            qs = [(k, int(r.q_marker[j]), int(r.q_type[j]), r.options_of(j)) for k, r in enumerate(g)
                  for j in range(r.n_questions)]
            packed = _assemble([r.tokens_of(0) for r in g], [-1] * len(g), qs)
            plan = model.plan(packed)
            plan.run(dp.data_ptr(), dd.data_ptr(), sp)
            torch.cuda.synchronize()
            _ = dp[:int(packed.opt_offsets[-1])].cpu()
            plan.free()
        run_group(groups[0])                          # warm-up
        t0 = time.perf_counter()
        for g in groups:
            a = time.perf_counter()
            run_group(g)
            lat.extend([time.perf_counter() - a] * len(g))
            n_dec += sum(r.n_questions for r in g)
        out[f"c{c}_packed"] = stats(lat, time.perf_counter() - t0, n_dec)
    return out


def features_leg(model, batch, shape, stream, args):
    """Full-vocabulary log-probability features of every option token at
    its question's marker row (one candidate per option, one group per
    question), computed after the readout of the same request: the step with
    features against the step without, and the vocabulary log-sum-exp
    kernel against HBM bandwidth (it streams the tied embedding once per
    launch of up to 64 distinct rows)."""
    import torch
    rows, toks, off, grp = [], [], [0], []
    for j in range(batch.n_questions):
        r = int(batch.cu_seqlens[batch.q_seq[j]]) + int(batch.q_marker[j])
        for t in batch.options_of(j):
            rows.append(r)
            toks.append(int(t))
            off.append(len(rows))
            grp.append(j)
    plan = model.plan(batch)
    dp = torch.zeros(max(plan.n_options, 1), dtype=torch.float32, device="cuda")
    dd = torch.zeros((max(plan.n_questions, 1), 6), dtype=torch.float32, device="cuda")
    dlp = torch.zeros(len(rows), dtype=torch.float32, device="cuda")
    dcl = torch.zeros(len(grp), dtype=torch.float32, device="cuda")
    dcn = torch.zeros(len(grp), dtype=torch.float32, device="cuda")
    plan.set_features(rows, toks, off, grp, dlp.data_ptr(), dcl.data_ptr(), dcn.data_ptr())
    sp = stream.cuda_stream
    plan.set_graph(True)
    for _ in range(args.warmup):
        plan.run(dp.data_ptr(), dd.data_ptr(), sp)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        plan.run(dp.data_ptr(), dd.data_ptr(), sp)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    plan.set_graph(False)
    prof = {}
    n_prof = max(1, args.profile_steps)
    for _ in range(n_prof):
        for k, (n, us) in plan.profile(dp.data_ptr(), dd.data_ptr(), sp).items():
            a, b = prof.get(k, (0, 0.0))
            prof[k] = (a + n, b + us)
    plan.free()
    R = len(set(rows))
    bf16 = shape.dtype == "bf16"
    # bf16: one pass over the vocabulary per 64 distinct rows; fp32: one
    launches = -(-(-(-R // 32) * 32) // 64) if bf16 else 1
    n_v, us_v = prof["vocab_lse"]                      # one event interval per run, all passes
    us_launch = us_v / n_v / launches
    bytes_launch = shape.vocab * shape.d_model * (2 if bf16 else 4)   # the tied embedding, read once
    gbps = bytes_launch / (us_launch * 1e-6) / 1e9
    return {"targets": len(rows), "distinct_rows": R, "candidates": len(grp), "groups": int(batch.n_questions),
            "ms_per_step_with_features": round(ms, 4),
            "vocab_lse": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbps / HBM_PEAK_GBS, 4), "bytes_per_launch": bytes_launch,
                          "launches_per_step": launches, "us_per_launch": round(us_launch, 2)},
            "features_other_us_per_step": round(prof.get("features", (0, 0.0))[1] / n_prof, 2)}


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-from":
        traffic_from_counters(sys.argv[2], sys.argv[3], sys.argv[4] if len(sys.argv) > 4 else "4b-single-512")
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="4b-single-512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=5)
    ap.add_argument("--no-serve", action="store_true",
                    help="skip the request-replay leg (length-bucket graphs, concurrency 1 / 8 / 16)")
    ap.add_argument("--no-features", action="store_true",
                    help="skip the full-vocabulary log-prob feature leg")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak probes (MFMA loop, 1 GiB copy)")
    ap.add_argument("--no-readout-stress", action="store_true",
                    help="skip the readout at the declared stress shape (4,096 questions x 10 options)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="with the 4B single request, skip the 16-request and branched workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB elementwise copy kernel (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the decision path has no "
              "multi-GPU code; see the sharding notes in the design document.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import prefill_only_decision_amd as s1
    from s1_workloads import make_batch, make_weights, shape_of

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()      # a real stream: events and kernels on the same queue
    shape = shape_of(args.workload)
    batch = make_batch(args.workload)
    t0 = time.time()
    w = make_weights(shape)
    t_gen = time.time() - t0
    T = batch.n_tokens
    # budgets also cover the request-replay leg (16 packed requests of <= 2048 tokens)
    cfg = s1.make_config(shape, max_tokens=max(T, 16 * 2048), max_seqs=max(batch.n_seqs, 32),
                         max_questions=max(batch.n_questions, 96), max_options=256, max_prefixes=4,
                         max_positions=max(int(batch.seq_lens.max()) * 2, 8192))
    t0 = time.time()
    model = s1.Model(cfg, w.tensors, stream=stream)
    t_load = time.time() - t0
    plan = model.plan(batch)
    dp = torch.zeros(max(plan.n_options, 1), dtype=torch.float32, device="cuda")
    dd = torch.zeros((max(plan.n_questions, 1), 6), dtype=torch.float32, device="cuda")
    sp = stream.cuda_stream

    def timed(graph):
        plan.set_graph(graph)
        for _ in range(args.warmup):
            plan.run(dp.data_ptr(), dd.data_ptr(), sp)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            plan.run(dp.data_ptr(), dd.data_ptr(), sp)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps, (time.perf_counter() - w0) / args.steps

    ms_eager, wall_eager = timed(False)
    plan.set_invariant(True)             # row-invariant schedule, reported beside
    ms_invariant, _ = timed(True)
    plan.set_invariant(False)
    ms_step, wall = timed(True)          # the plan replayed as one HIP graph
    wall *= args.steps
    tokens = plan.tokens
    value = tokens / (ms_step / 1e3)
    reqs = requests_in(batch)

    # per-kernel durations: events recorded by the library after each launch
    plan.set_graph(False)
    prof = {}
    for _ in range(max(1, args.profile_steps)):
        for k, (n, us) in plan.profile(dp.data_ptr(), dd.data_ptr(), sp).items():
            a, b = prof.get(k, (0, 0.0))
            prof[k] = (a + n, b + us)
    steps_p = max(1, args.profile_steps)
    flops = gemm_flops(shape, tokens)
    launches, total_us = prof["gemm_gate_up"]
    avg_us = total_us / launches
    # flops of the whole step over the kernel's time per step: a branched
    # request runs the layer once per pass (prefix, then branches)
    step_flops = flops["gemm_gate_up"] * shape.n_layers     # every layer, every token
    achieved = step_flops / (total_us / steps_p * 1e-6) / 1e12
    kernels = {k: {"launches_per_step": n // steps_p, "us_per_step": round(us / steps_p, 1),
                   "us_per_launch": round(us / n, 2)} for k, (n, us) in sorted(prof.items())}
    gemm_us = sum(prof[k][1] for k in ("gemm_la_in", "gemm_fa_qkv", "gemm_o", "gemm_gate_up", "gemm_down")
                  if k in prof) / steps_p
    all_gemm_flops = 2 * tokens * shape.linear_params()
    roofline = {"bound": "mfma", "kernel": "gemm_gate_up (bf16 MFMA GEMM + SwiGLU epilogue)",
                "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": stored_traffic(args.workload),
                "traffic_unit": "bytes per launch (HBM, counter-measured)",
                "flops_per_step": step_flops, "launches_per_step": launches // steps_p,
                "us_per_launch": round(avg_us, 2),
                "all_gemms_tflops": round(all_gemm_flops / (gemm_us * 1e-6) / 1e12, 1)}

    scan = scan_roofline(shape, batch, tokens, prof, steps_p)
    attn = attention_roofline(shape, batch, prof, steps_p)
    gemm_fracs = {}
    for k in ("gemm_la_in", "gemm_fa_qkv", "gemm_o", "gemm_gate_up", "gemm_down"):
        if k in prof and flops.get(k):
            n_k, us_k = prof[k]
            tf = flops[k] * (n_k // steps_p) / (us_k / steps_p * 1e-6) / 1e12
            gemm_fracs[k] = {"tflops": round(tf, 1), "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                             "us_per_launch": round(us_k / n_k, 2)}
    roofline["all_gemms_frac"] = round(roofline["all_gemms_tflops"] / BF16_PEAK_TFLOPS, 4)
    roofline["per_gemm"] = gemm_fracs

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_request": round(ms_step / reqs, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "tokens_per_step": int(tokens), "requests_per_step": reqs,
                   "questions_per_step": int(batch.n_questions), "layers": shape.n_layers,
                   "d_model": shape.d_model, "weights": "seeded random init N(0, 0.02), LoRA r32 merged"},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "execution": "HIP graph replay of the plan",
        "ms_per_step_eager_launches": round(ms_eager, 4),
        "ms_per_step_row_invariant": round(ms_invariant, 4),
        "load_s": round(t_load, 2), "weight_gen_s": round(t_gen, 2),
        "kernels": kernels, "roofline": roofline, "scan": scan, "attention": attn,
    }
    plan.free()
    out["prefill_decide"] = decide_leg(model, batch, warmup=2, timed=args.steps)
    if args.workload == "4b-single-512" and not args.no_other_workloads:
        out["other_workloads"] = {n: workload_leg(model, n, args, stream)
                                  for n in ("4b-varlen-16", "4b-branch-4096x20")}
    if not args.no_features:
        out["features"] = features_leg(model, batch, shape, stream, args)
    if not args.no_serve and shape.dtype == "bf16":
        out["serving"] = serve_leg(model, shape, stream)
    model.free()
    if not args.no_readout_stress and shape.dtype == "bf16":
        out["readout_stress"] = readout_stress_leg(shape, stream)
    peaks = None if args.no_peaks else measure_peaks(stream)
    if peaks:
        out["peaks"] = peaks
        add_measured_fraction(out["roofline"], peaks, "mfma_bf16_tflops")
        add_measured_fraction(out["scan"], peaks, "hbm")
        add_measured_fraction(out.get("readout_stress"), peaks, "hbm")
        add_measured_fraction((out.get("features") or {}).get("vocab_lse"), peaks, "hbm")
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(3):
                torch.mul(src, 1.0, out=dst)   # an elementwise kernel (a plain copy may go to the DMA engines)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, w, batch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
