"""Benchmark: MLA decode over a paged latent KV cache on one MI355X.

One step = one full decode of one batch (split kernel + log-sum-exp merge,
the two launches ``mla_decode`` makes) on synthetic inputs already resident
in HBM.  Steps rotate over several copies of the KV pool and queries (one per
"layer") so that the 256 MB last-level cache never serves a step from the
previous one.  Prints ONE JSON line (see the ``print`` at the end).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402

METRIC = "MLA decode KV GB/s + tokens/s per GPU; % of HBM/MFMA roofline (1 MI355X)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
LLC_BYTES = 256 << 20          # MI355X Infinity Cache


def algorithmic(w, seq_lens, with_output):
    """Bytes and MFMA flops the decode must touch/do, per the method's data:
    each token's stored row once (a prefix shared by all requests once), the
    queries, the page-table entries and lengths, and the output if written."""
    L = np.asarray(seq_lens, dtype=np.int64)
    row = {"bf16": 2 * w.d, "fp8": w.d + 4, "f32": 4 * w.d}[w.kv_dtype]
    kv_logical = int(L.sum()) * row
    kv_unique = kv_logical - max(0, w.batch - 1) * w.shared_prefix * row
    q_bytes = w.batch * w.rows * w.d * (2 if w.q_dtype == "bf16" else 4)
    out_bytes = w.batch * w.rows * w.d_latent * (2 if w.out_dtype == "bf16" else 4)
    table = int(np.ceil(L / w.page_size).sum()) * 4 + 4 * w.batch
    bytes_ = kv_unique + q_bytes + table + (out_bytes if with_output else 0)
    flops = 2 * w.heads * w.q_len * int(L.sum()) * (w.d + w.d_latent)
    return {"bytes": bytes_, "kv_logical": kv_logical, "kv_unique": kv_unique, "flops": flops}


def device_inputs(inp, copies):
    """Host synth arrays -> `copies` independent device copies of KV and queries."""
    w = inp["workload"]

    def t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    base = {k: t(inp[k]) for k in ("q_abs", "q_rope", "kv", "page_table", "seq_lens")}
    base["kv_scales"] = None if inp["kv_scales"] is None else t(inp["kv_scales"])
    sets = [base]
    for _ in range(copies - 1):
        c = dict(base)
        for k in ("q_abs", "q_rope", "kv", "kv_scales"):
            if base[k] is not None:
                c[k] = base[k].clone()
        sets.append(c)
    del w
    return sets


def cpu_baseline(inp, budget_s):
    """Time the fp64 CPU oracle on a bounded sample of the workload's requests."""
    import oracle
    w = inp["workload"]
    L = inp["seq_lens"]
    threads = oracle.max_threads()
    # calibrate on the shortest request, then take requests until ~budget
    probe = [int(np.argmin(L))]
    t0 = time.perf_counter()
    oracle.attend(inp, req_ids=probe)
    per_token = (time.perf_counter() - t0) / max(1, int(L[probe[0]]))
    pick, est = [], 0.0
    for b in np.random.default_rng(7).permutation(w.batch):
        if est + per_token * int(L[b]) > budget_s and pick:
            break
        pick.append(int(b))
        est += per_token * int(L[b])
    t0 = time.perf_counter()
    oracle.attend(inp, req_ids=pick)
    dt = time.perf_counter() - t0
    sub = algorithmic(w, L[pick], with_output=True)
    return {
        "value": round(sub["kv_logical"] / dt / 1e9, 4), "unit": "GB/s",
        "tokens_per_s": round(len(pick) * w.q_len / dt, 3),
        "cores": threads, "kind": "oracle", **host_info(),
        "sample": f"{len(pick)} of {w.batch} requests ({int(L[pick].sum())} KV tokens, all "
                  f"{w.heads} heads x {w.q_len} query tokens), fp64 C oracle, {dt:.1f} s",
    }


KERNEL_SOURCE = os.path.join(ROOT, "mla_decode_attention_02_amd", "csrc", "mla_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def pmc_summary(pmc_dir, workload, num_splits, calib_mib, out_path=None):
    """Per-launch HBM traffic of the split kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the calibration copy of calib_mib MiB in the same run."""
    import csv
    import glob

    def per_kernel(counter):
        rows = []
        for f in glob.glob(os.path.join(pmc_dir, "*counter_collection.csv")):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        split = [float(r["Counter_Value"]) for r in rows if "mla_split" in r["Kernel_Name"]]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        return split, copies

    # the kernel-source hash the profiled runs printed in their JSON lines
    # (their logs sit beside the counter directory as <dir>_*.log)
    seen, plans = set(), set()
    for logf in glob.glob(pmc_dir.rstrip("/") + "_*.log"):
        for ln in open(logf, errors="replace"):
            if ln.startswith("{") and "kernel_source_sha256_16" in ln:
                rec = json.loads(ln)
                seen.add(rec["kernel_source_sha256_16"])
                plans.add(rec["config"].get("plan_key"))
    if len(seen) > 1 or len(plans) > 1:
        raise SystemExit(f"profiled runs disagree: sources {sorted(seen)}, plans {sorted(map(str, plans))}")
    src_hash = seen.pop() if seen else kernel_source_hash()
    plan_key = plans.pop() if plans else None
    if out_path is None:
        if plan_key is None:
            raise SystemExit("no profiled run log names its plan; pass --pmc-out")
        out_path = traffic_path(workload, plan_key)

    f_split, f_copy = per_kernel("FETCH_SIZE")
    w_split, w_copy = per_kernel("WRITE_SIZE")
    calib_kib = calib_mib * 1024.0
    rf = calib_kib / max(f_copy)
    wf = calib_kib / max(w_copy)
    fetch = float(np.mean(f_split)) * rf * 1024
    write = float(np.mean(w_split)) * wf * 1024
    rel = os.path.relpath(os.path.abspath(pmc_dir), ROOT)
    run = (f"python -u $REPO/bench.py --steps 5 --warmup 2 --no-cpu --no-sub --no-probe --workload {workload}"
           f"{'' if num_splits < 0 else f' --num-splits {num_splits}'} --calib-copy-mib {calib_mib}")
    lines = [
        f"# HBM traffic of {split_kernel_name(next(x for x in synth.WORKLOADS if x.name == workload))}, "
        f"workload {workload}",
        "",
        "Commands (the two profiled runs from /tmp with TMPDIR=/tmp; REPO = repository root):",
        "",
        "```",
        f"timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/{rel} -o pass3 -- {run}",
        f"timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/{rel} -o pass4 -- {run}",
        f"python bench.py --pmc-summary {rel} --workload {workload}"
        f"{'' if num_splits < 0 else f' --num-splits {num_splits}'} --calib-copy-mib {calib_mib}",
        "```",
        "",
        f"kernel_source_sha256_16: {src_hash}",
        f"plan: {plan_key}",
        f"dispatches: {len(f_split)} (FETCH_SIZE run), {len(w_split)} (WRITE_SIZE run)",
        f"FETCH_SIZE per dispatch (KiB, raw): {np.mean(f_split):.1f}",
        f"WRITE_SIZE per dispatch (KiB, raw): {np.mean(w_split):.1f}",
        f"calibration copy {calib_mib} MiB: FETCH_SIZE {max(f_copy):.1f} KiB -> x{rf:.4f}, "
        f"WRITE_SIZE {max(w_copy):.1f} KiB -> x{wf:.4f}",
        f"read_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"traffic_bytes_per_launch: {fetch + write:.0f}",
    ]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def split_kernel_name(w):
    """The split kernel the library runs for workload w: the wave-pair MFMA
    kernel for bf16 and E4M3 KV (the four-wave one under MLA_MFMA_KERNEL=four),
    the VALU one for other widths."""
    if w.d_latent != 512 or w.d_rope != 64 or w.q_dtype != "bf16" or w.kv_dtype not in ("bf16", "fp8"):
        return "mla_split_generic"
    return "mla_split_mfma" if os.environ.get("MLA_MFMA_KERNEL", "").startswith("f") else "mla_split_pair"


def traffic_path(workload, plan_key):
    """Where the HBM-traffic summary of the split kernel for this workload and
    launch configuration (plan key: "balanced", or "s<S>" for S uniform
    chunks per request) lives under profiles/."""
    w = next(x for x in synth.WORKLOADS if x.name == workload)
    return os.path.join(PROFILES, f"{split_kernel_name(w)}__{workload}__{plan_key}__traffic.md")


def recorded_traffic(workload, plan_key):
    """Traffic per launch recorded for this workload and launch configuration,
    if taken on the current kernel source."""
    path = traffic_path(workload, plan_key)
    if not os.path.exists(path):
        return None
    info = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            info[k.strip()] = v.strip()
    if info.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return int(float(info["traffic_bytes_per_launch"]))


def bench_append(mla, args):
    """Paged KV append with FP8 packing: a prefill-sized append (256 requests x
    512 new 576-wide bf16 rows, 64-token pages, permuted page table) into an
    E4M3 cache with per-token scales.  HBM-bound: the algorithmic bytes are
    the source rows read plus the codes and scales written plus the table."""
    B, T, D, P = 256, 512, 576, 64
    MP = T // P + 1
    rng = np.random.default_rng(2024)
    NP = B * MP + 64
    x = (rng.standard_normal((B, T, D)) * 0.5).astype(np.float32)
    rows = torch.from_numpy(x).to(torch.bfloat16).cuda()
    pt = torch.from_numpy(rng.permutation(NP)[: B * MP].reshape(B, MP).astype(np.int32)).cuda()
    pos = torch.from_numpy(rng.integers(0, P, size=B).astype(np.int32)).cuda()
    kv = torch.zeros((NP, P, D), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((NP, P), dtype=torch.float32, device="cuda")
    import ctypes
    lib = mla.library()
    pr = mla.Problem(B, T, 1, D, 0, P, NP, MP, 0, mla.MLA_DTYPE_BF16, mla.MLA_DTYPE_FP8_E4M3,
                     mla.MLA_DTYPE_BF16, 0, 0)
    P_ = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = (ctypes.byref(pr), P_(rows), mla.MLA_DTYPE_BF16, P_(pt), P_(pos), P_(kv), P_(sc), stream)
    for _ in range(args.warmup):
        if lib.mla_append_kv(*call):
            raise RuntimeError("mla_append_kv failed")
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        lib.mla_append_kv(*call)
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = B * T * D * 2 + B * T * (D + 4) + B * MP * 4 + B * 4
    achieved = nbytes / (k_ms / 1e3) / 1e9
    cpu = None
    if not args.no_cpu:
        import oracle
        sub = 16  # requests in the CPU sample
        kv_h = np.zeros((NP, P, D), dtype=np.uint8)
        sc_h = np.zeros((NP, P), dtype=np.float32)
        xs = torch.from_numpy(x[:sub]).to(torch.bfloat16).float().numpy()
        t1 = time.perf_counter()
        oracle.append_rows(xs, pt.cpu().numpy()[:sub], pos.cpu().numpy()[:sub], kv_h, sc_h, dst="fp8")
        dt = time.perf_counter() - t1
        cpu = {"value": round(sub * T * (D * 2 + D + 4) / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "sample": f"{sub} of {B} requests x {T} rows, single-threaded C oracle, {dt:.2f} s"}
    line = {
        "metric": "paged KV append + FP8 pack GB/s (1 MI355X)", "value": round(achieved, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, e4m3 + fp32 scale out",
        "data": "synthetic (seeded N(0,1)*0.5 rows, random page permutation)",
        "config": {"workload": "kv_append_fp8", "requests": B, "rows_per_request": T, "row_width": D,
                   "page_size": P, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "mla_append_kernel",
                     "per_launch_algorithmic": nbytes, "kernel_avg_ms": round(k_ms, 5)},
        "cpu_baseline": cpu,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


def bench_verify(mla, args):
    """Greedy chain verification after the speculative-decode step: 256
    requests x 4 positions of bf16 logits over a 129280-token vocabulary
    (DeepSeek-V3's size, assumed: the pages state none).  HBM-bound: the
    algorithmic bytes are the logits plus drafts read and the results written."""
    B, T, V = 256, 4, 129280
    rng = np.random.default_rng(2025)
    lg = torch.from_numpy(rng.standard_normal((B, T, V)).astype(np.float32)).to(torch.bfloat16).cuda()
    draft = torch.from_numpy(rng.integers(0, V, size=(B, T - 1)).astype(np.int32)).cuda()
    am = torch.empty((B, T), dtype=torch.int32, device="cuda")
    n = torch.empty((B,), dtype=torch.int32, device="cuda")
    out = torch.empty((B, T), dtype=torch.int32, device="cuda")
    import ctypes
    lib = mla.library()
    P_ = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = (B, T, V, P_(lg), mla.MLA_DTYPE_BF16, P_(draft), P_(am), P_(n), P_(out), stream)
    for _ in range(args.warmup):
        if lib.mla_verify_greedy(*call):
            raise RuntimeError("mla_verify_greedy failed")
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        lib.mla_verify_greedy(*call)
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = B * T * V * 2 + B * (T - 1) * 4 + B * (2 * T + 1) * 4
    achieved = nbytes / (k_ms / 1e3) / 1e9
    cpu = None
    if not args.no_cpu:
        import oracle
        sub = 8
        vals = lg[:sub].float().cpu().numpy()
        t1 = time.perf_counter()
        oracle.verify_greedy(vals, draft[:sub].cpu().numpy())
        dt = time.perf_counter() - t1
        cpu = {"value": round(sub * T * V * 2 / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{sub} of {B} requests x {T} positions, single-threaded C oracle, {dt:.2f} s"}
    line = {
        "metric": "greedy draft verification, logits GB/s (1 MI355X)", "value": round(achieved, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 logits, int32 tokens",
        "data": "synthetic (seeded N(0,1) logits rounded to bf16, random drafts)",
        "config": {"workload": "verify_greedy", "requests": B, "positions": T, "vocab": V,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "mla_verify_kernel",
                     "per_launch_algorithmic": nbytes, "kernel_avg_ms": round(k_ms, 5)},
        "cpu_baseline": cpu,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


def bench_project(mla, args):
    """The absorbed per-head projections on either side of one decode step of
    the chosen workload: q_abs = W_UK^T q_nope (d_nope 128 -> d_latent) before
    it and W_UV o (d_latent -> d_v 128) after it, for B*T token rows and all
    heads, with random synthetic bf16 weights.  At decode batch sizes both are
    weight-streaming: the roofline is HBM unless the flops take longer at the
    bf16 MFMA peak."""
    w = next(x for x in synth.WORKLOADS if x.name == args.workload)
    M, G, Dc = w.batch * w.q_len, w.heads, w.d_latent
    sides = [("query", synth.PROJ_D_NOPE, Dc), ("value", Dc, synth.PROJ_D_V)]
    import ctypes
    lib = mla.library()
    P_ = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = sum(2 * (M * G * K + G * N * K + M * G * N) for _, K, N in sides)
    flops = sum(2 * M * G * K * N for _, K, N in sides)
    # In a model, each layer's weights come back only after every other layer's:
    # rotate through enough copies that one pass exceeds twice the last-level
    # cache, so that every launch streams its operands from HBM.
    copies = int(max(1, -(-2 * LLC_BYTES // nbytes)))
    host, sets = [], []
    for i, (name, K, N) in enumerate(sides):
        xb, wb = synth.make_projection_inputs(M, G, K, N, seed=31 + i)
        host.append((xb, wb))
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
        wt = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).cuda()
        sets.append([(x.clone(), wt.clone(), torch.empty((M, G, N), dtype=torch.bfloat16, device="cuda"))
                     for _ in range(copies)])
    calls = [[(M, G, K, N, P_(sets[i][c][0]), P_(sets[i][c][1]), mla.MLA_DTYPE_BF16, P_(sets[i][c][2]), stream)
              for i, (_, K, N) in enumerate(sides)] for c in range(copies)]
    for step in range(args.warmup):
        for c in calls[step % copies]:
            if lib.mla_project(*c):
                raise RuntimeError("mla_project failed")
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for step, (e0, e1) in enumerate(evs):
        e0.record()
        for c in calls[(args.warmup + step) % copies]:
            lib.mla_project(*c)
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))  # both launches
    t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(nbytes / (k_ms / 1e3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / (k_ms / 1e3) / 1e12, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof.update({"frac": round(roof["achieved"] / roof["peak"], 4), "traffic": None,
                 "kernel": "mla_project_kernel (query and value side)", "per_step_algorithmic_bytes": nbytes,
                 "per_step_flops": flops, "kernels_ms_per_step": round(k_ms, 5)})
    cpu = None
    if not args.no_cpu:
        import oracle

        def run_oracle(rows):
            for xb, wb in host:
                oracle.project(synth.bf16_bits_to_f32(xb[:rows]).astype(np.float64),
                               synth.bf16_bits_to_f32(wb).astype(np.float64))
        t1 = time.perf_counter()
        run_oracle(1)                               # calibrate, then take rows for ~the budget
        per_row = time.perf_counter() - t1
        sub = int(max(1, min(M, args.cpu_budget / max(per_row, 1e-6))))
        t1 = time.perf_counter()
        run_oracle(sub)
        dt = time.perf_counter() - t1
        cpu = {"value": round(sub / dt, 2), "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
               "sample": f"{sub} of {M} token rows through both projections, fp64 C oracle, {dt:.2f} s"}
    line = {
        "metric": "absorbed MLA projections (W_UK^T q_nope, W_UV o), tokens/s (1 MI355X)",
        "value": round(M / (k_ms / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5 activations, N(0,1)/sqrt(k) weights, bf16)",
        "config": {"workload": f"project_{w.name}", "token_rows": M, "heads": G, "d_nope": synth.PROJ_D_NOPE,
                   "d_latent": Dc, "d_v": synth.PROJ_D_V, "operand_copies_rotated": copies,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


HEADLINE = "spec_decode_bf16"
# The other graded workloads, measured in the same run and reported inside the
# headline's JSON line: (workload, forced split count or None for the
# library's own plan, label).
SUB_RESULTS = (("deepseek_v3_bf16", None, "library plan"),
               ("agentic_long_bf16", 16, "16 chunks per request, as configured"),
               ("agentic_long_bf16", 0, "library plan"),
               ("fp8_kv", None, "library plan"))


def host_info():
    """Host cores and CPU model, recorded beside the oracle's time."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def measure_decode(mla, w, inp, args, S_req, cascade=False):
    """Time `args.steps` decode steps of workload `w` on the device copies of
    `inp`; returns the measurement record (no CPU baseline)."""
    import ctypes
    kv_bytes = inp["kv"].nbytes + (0 if inp["kv_scales"] is None else inp["kv_scales"].nbytes)
    copies = max(2, min(8, math.ceil(4 * LLC_BYTES / kv_bytes)))
    sets = device_inputs(inp, copies)
    d0 = sets[0]
    pr = mla.make_problem(d0["q_abs"], d0["q_rope"], d0["kv"], d0["page_table"],
                          causal=w.causal, num_splits=S_req, max_seq_len=w.max_seq_len)
    S = mla.num_splits(pr)
    B, T, H, Dc = d0["q_abs"].shape
    R = T * H
    out_dt = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
    out = torch.empty((B, R, Dc), dtype=out_dt, device="cuda")
    lse = torch.empty((B, R), dtype=torch.float32, device="cuda")
    scale = float(inp["scale"])

    # Arguments are marshalled once per KV copy, so that the timed loop only
    # makes the C-ABI calls (the same launches mla_decode makes) and records
    # the HIP events around them on the launch stream.
    lib = mla.library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    prs = mla.make_problem(d0["q_abs"], d0["q_rope"], d0["kv"], d0["page_table"],
                           causal=w.causal, num_splits=S, max_seq_len=w.max_seq_len)
    # mla_decode's own choice: the balanced work list when the library picks
    # the plan, the uniform plan would split, and the MFMA kernels serve the
    # shape (MLA_PLAN=uniform turns it off).  Its two stages are called one
    # by one so that the split kernel can be timed by itself.
    balanced = (S_req == 0 and S > 1 and w.d_latent == 512 and w.d_rope == 64
                and w.q_dtype == "bf16" and w.kv_dtype in ("bf16", "fp8")
                and not os.environ.get("MLA_PLAN", "").startswith("u") and not cascade)
    nw = 0
    if cascade:
        if not w.shared_prefix:
            raise SystemExit("--cascade needs a workload with a shared prefix")
        need = ctypes.c_size_t(0)
        lib.mla_cascade_workspace_size(ctypes.byref(prs), w.shared_prefix, ctypes.byref(need))
        cws = torch.empty(max(1, need.value), dtype=torch.uint8, device="cuda")
        calls = [[(lib.mla_decode_cascade,
                   (ctypes.byref(prs), P(d["q_abs"]), P(d["q_rope"]), P(d["kv"]), P(d["kv_scales"]),
                    P(d["page_table"]), P(d["seq_lens"]), ctypes.c_float(scale), w.shared_prefix, P(out),
                    P(lse), P(cws), cws.numel(), stream))] for d in sets]
        plan = "cascade over the shared prefix (split and merge timed together)"
    elif balanced:
        nw = mla.balanced_workgroups()
        groups = -(-R // mla.BALANCED_ROWS)
        prefix = torch.empty(B * groups + 1, dtype=torch.int32, device="cuda")
        slot_o = torch.empty((2 * nw, mla.BALANCED_ROWS, Dc), dtype=torch.bfloat16, device="cuda")
        slot_l = torch.empty((2 * nw, mla.BALANCED_ROWS), dtype=torch.float32, device="cuda")
        calls = [[(lib.mla_decode_split_balanced,
                   (ctypes.byref(prs), P(d["q_abs"]), P(d["q_rope"]), P(d["kv"]), P(d["kv_scales"]),
                    P(d["page_table"]), P(d["seq_lens"]), ctypes.c_float(scale), nw, P(prefix), P(out),
                    P(lse), P(slot_o), P(slot_l), stream)),
                  (lib.mla_combine_balanced,
                   (ctypes.byref(prs), nw, P(prefix), P(slot_o), P(slot_l), P(out), P(lse), stream))]
                 for d in sets]
        plan = f"balanced work list, {nw} workgroups"
    elif S == 1:
        ws = torch.empty(max(1, mla.workspace_size(prs)), dtype=torch.uint8, device="cuda")
        calls = [[(lib.mla_decode,
                   (ctypes.byref(prs), P(d["q_abs"]), P(d["q_rope"]), P(d["kv"]), P(d["kv_scales"]),
                    P(d["page_table"]), P(d["seq_lens"]), ctypes.c_float(scale), P(out), P(lse), P(ws),
                    ws.numel(), stream))] for d in sets]
        plan = "uniform, 1 chunk per request"
    else:
        part_o = torch.empty((B, S, R, Dc), dtype=torch.float32, device="cuda")
        part_l = torch.empty((B, S, R), dtype=torch.float32, device="cuda")
        calls = [[(lib.mla_decode_split,
                   (ctypes.byref(prs), P(d["q_abs"]), P(d["q_rope"]), P(d["kv"]), P(d["kv_scales"]),
                    P(d["page_table"]), P(d["seq_lens"]), ctypes.c_float(scale), S, P(part_o), P(part_l),
                    stream)),
                  (lib.mla_combine,
                   (B, S, R, Dc, P(part_o), P(part_l),
                    mla.MLA_DTYPE_BF16 if out_dt == torch.bfloat16 else mla.MLA_DTYPE_F32,
                    P(out), P(lse), stream))] for d in sets]
        plan = f"uniform, {S} chunks per request"

    def step(i, evs=None):
        # evs[0] .. evs[1] bracket the split kernel (the first call), evs[1] ..
        # evs[2] the merge (if any)
        seq = calls[i % copies]
        if evs is not None:
            evs[0].record()
        rc = seq[0][0](*seq[0][1])
        if evs is not None:
            evs[1].record()
        for fn, a in seq[1:]:
            rc |= fn(*a)
        if evs is not None:
            evs[2].record()
        if rc:
            raise RuntimeError(f"decode failed: {mla.status_string(rc)}")

    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    split_ms = [e[0].elapsed_time(e[1]) for e in events]
    comb_ms = [e[1].elapsed_time(e[2]) for e in events]
    ms_per_step = wall * 1e3 / args.steps
    del sets, calls
    torch.cuda.empty_cache()

    pkey = "balanced" if balanced else ("cascade" if cascade else f"s{S}")
    L = inp["seq_lens"]
    alg_split = algorithmic(w, L, with_output=(S == 1 or balanced))
    alg_path = algorithmic(w, L, with_output=True)
    split_avg = float(np.mean(split_ms))
    t_hbm = alg_path["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = alg_path["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    if bound == "hbm":
        achieved = alg_split["bytes"] / (split_avg / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = alg_split["flops"] / (split_avg / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None}
    if cascade:
        roof["traffic"] = None
    else:
        roof["traffic"] = recorded_traffic(w.name, pkey)
    roof["kernel"] = split_kernel_name(w)
    roof["per_launch_algorithmic"] = alg_split["bytes"] if bound == "hbm" else alg_split["flops"]
    roof["kernel_avg_ms"] = round(split_avg, 5)
    roof["path_roofline_ms"] = round(max(t_hbm, t_mfma) * 1e3, 5)
    roof["path_frac"] = round(max(t_hbm, t_mfma) * 1e3 / ms_per_step, 4)
    seq_desc = (f"U[{w.seq_lens[1]},{w.seq_lens[2]}]" if w.seq_lens[0] == "uniform"
                else f"fixed {w.seq_lens[1][0]}") + f" seed {1000 + w.index}"
    return {
        "workload": w.name, "plan": plan, "ms_per_step": round(ms_per_step, 5),
        "kv_gbs": round(alg_path["kv_logical"] / (ms_per_step / 1e3) / 1e9, 2),
        "kv_gbs_unique": round(alg_path["kv_unique"] / (ms_per_step / 1e3) / 1e9, 2),
        "tokens_per_s": round(B * T / (ms_per_step / 1e3), 1),
        "split_ms": round(split_avg, 5), "combine_ms": round(float(np.mean(comb_ms)), 5),
        "roofline": roof,
        "config": {"workload": w.name, "batch": B, "q_len": T, "heads": H, "d_latent": w.d_latent,
                   "d_rope": w.d_rope, "page_size": w.page_size, "seq_lens": seq_desc,
                   "kv_dtype": w.kv_dtype, "shared_prefix": w.shared_prefix, "causal": w.causal,
                   "plan": plan, "plan_key": pkey, "kv_copies_rotated": copies,
                   "parallelism": "single GPU"},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=[w.name for w in synth.WORKLOADS])
    ap.add_argument("--num-splits", type=int, default=-1,
                    help="override the split count (default: the workload's, else the library's)")
    ap.add_argument("--no-sub", action="store_true",
                    help="measure only --workload (no sub-results for the other workloads)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="summarise FETCH_SIZE/WRITE_SIZE rocprofv3 CSVs in DIR and exit")
    ap.add_argument("--pmc-out", metavar="FILE", help="where --pmc-summary writes its summary")
    ap.add_argument("--cascade", action="store_true",
                    help="decode with mla_decode_cascade over the workload's shared prefix")
    ap.add_argument("--op", choices=("decode", "append", "verify", "project"), default="decode",
                    help="decode (the default hot path), the paged KV append with FP8 packing, "
                         "the greedy verification of speculative drafts, or the absorbed "
                         "projections around one decode step of --workload")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.workload, args.num_splits, args.calib_copy_mib or 1024,
                    args.pmc_out)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the decode on a single MI355X "
              "(--gpus 1); multi-GPU runs are not part of it.", file=sys.stderr)
        sys.exit(2)
    import mla_decode_attention_02_amd as mla
    mla.library()
    torch.cuda.set_device(0)
    if args.op == "append":
        bench_append(mla, args)
        return
    if args.op == "project":
        bench_project(mla, args)
        return
    if args.op == "verify":
        bench_verify(mla, args)
        return

    w = next(x for x in synth.WORKLOADS if x.name == args.workload)
    inp = synth.make_inputs(w, poison=False)
    S_req = w.num_splits if args.num_splits < 0 else args.num_splits
    head = measure_decode(mla, w, inp, args, S_req, cascade=args.cascade)
    print(f"# {w.name}: {head['plan']}: step {head['ms_per_step']} ms, split {head['split_ms']} ms, "
          f"frac {head['roofline']['frac']}", file=sys.stderr, flush=True)
    probe = None
    if head["roofline"]["bound"] == "hbm" and not args.no_probe:
        probe = hbm_read_probe()
        head["roofline"]["frac_of_read_probe"] = round(head["roofline"]["achieved"] / probe["gbs"], 4)
    cpu = None if args.no_cpu else cpu_baseline(inp, args.cpu_budget)
    del inp

    subs = []
    if not args.no_sub and not args.cascade and args.workload == HEADLINE and args.num_splits < 0:
        cache = {}
        for name, S_sub, label in SUB_RESULTS:
            ws = next(x for x in synth.WORKLOADS if x.name == name)
            if name not in cache:
                cache.clear()
                cache[name] = synth.make_inputs(ws, poison=False)
            rec = measure_decode(mla, ws, cache[name], args, ws.num_splits if S_sub is None else S_sub)
            rec["label"] = label
            print(f"# {name}: {rec['plan']}: step {rec['ms_per_step']} ms, split {rec['split_ms']} ms, "
                  f"frac {rec['roofline']['frac']}", file=sys.stderr, flush=True)
            subs.append(rec)
        cache.clear()

    line = {
        "metric": METRIC, "value": head["kv_gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3 KV, bf16 MFMA", "f32": "f32"}[w.kv_dtype],
        "data": "synthetic (seeded N(0,1)*sigma rows and queries, random page permutation)",
        "config": head["config"],
        "tokens_per_s": head["tokens_per_s"], "kv_gbs_unique": head["kv_gbs_unique"],
        "split_ms": head["split_ms"], "combine_ms": head["combine_ms"],
        "roofline": head["roofline"], "hbm_read_probe": probe, "cpu_baseline": cpu,
        "sub_results": [{k: r[k] for k in ("workload", "label", "plan", "ms_per_step", "tokens_per_s",
                                            "kv_gbs", "kv_gbs_unique", "split_ms", "combine_ms",
                                            "roofline")} for r in subs],
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


def hbm_read_probe(gib=4, reps=10):
    """What a plain streaming read reaches on this GPU, as context for the
    HBM roofline fraction (which stays against the 8 TB/s spec peak): the
    library's streaming-read hook over `gib` GiB, 8 workgroups per compute
    unit, median over `reps` runs timed with events on the current stream."""
    import mla_decode_attention_02_amd as mla
    x = torch.empty((gib << 30) // 4, dtype=torch.int32, device="cuda")
    x.fill_(1)
    sink = torch.empty(8 * mla.balanced_workgroups(), dtype=torch.int32, device="cuda")
    mla.stream_read(x, sink)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        mla.stream_read(x, sink)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del x, sink
    ms = float(np.median(times))
    return {"gbs": round((gib << 30) / (ms / 1e3) / 1e9, 1), "ms": round(ms, 4),
            "how": f"mla_stream_read over {gib} GiB, {reps} runs, median"}


if __name__ == "__main__":
    main()
