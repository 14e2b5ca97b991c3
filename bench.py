"""Throughput of batched draft verification on one MI355X.

python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--workload batched] [--out FILE]

A step is one sv_verify_batch (or sv_verify_greedy) call over one batch of synthetic logits that
is already resident in HBM. Several copies of the inputs at distinct addresses are rotated so that
no step finds its rows in the 256 MB Infinity Cache from the previous step. Prints one JSON line:
verified draft positions per second (the sum over requests of the drafts verified), with the
achieved HBM bandwidth of the verify call against the MI355X peak and against the read-stream
ceiling this device reaches with a plain read probe over the same input copies, and the fp64
CPU oracle timed on a bounded sample of the same workload on this host (one thread, and a pool
of worker processes over requests).
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("verified draft positions/sec and achieved HBM GB/s (% of peak) at V=151936, K=8")
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batched",
                    help="tiny | interactive | batched | heavy | greedy | mixed | schedule | markov | "
                         "markov_sampled | markov_topk | "
                         "sweep_<mode>_<K>_<B>_<dtype>")
    ap.add_argument("--min-rotation-bytes", type=float, default=1.2e9,
                    help="rotate input copies until at least this many bytes are cycled")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU budget of the oracle baseline (0 = skip)")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="worker processes of the pooled oracle baseline (capped by the cores "
                         "this process may use; 0 = skip the pooled baseline)")
    ap.add_argument("--skip-ceiling", action="store_true",
                    help="do not measure the read-stream ceiling")
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    return ap.parse_args()


def pick_workload(name):
    import workloads as W

    named = {"tiny": W.TINY, "interactive": W.INTERACTIVE, "batched": W.BATCHED,
             "heavy": W.HEAVY, "greedy": W.GREEDY, "mixed": W.MIXED}
    if name in named:
        return named[name]
    if name.startswith("sweep_"):
        _, mode, k, b, dt = name.split("_")
        return W.sweep_workload(int(k), int(b), dt, mode)
    raise SystemExit(f"unknown workload {name}")


def algorithmic_bytes(inp):
    """Compulsory bytes of one call: every logit row the outputs depend on, read once, plus the
    small per-request inputs and outputs."""
    w = inp.workload
    s = 2 if w.dtype == "bf16" else 4
    ks = np.array([inp.k_of(b) for b in range(w.B)], dtype=np.int64)
    samples = np.array([w.temperature_of(b) > 0 for b in range(w.B)])
    rows = np.where(samples, 2 * ks + 1, ks + 1)
    logits = int(rows.sum()) * w.V * s
    small = w.B * w.K * 4 + w.B * 4 * (1 if inp.num_draft is not None else 0)  # tokens, k_b
    small += w.B * (w.K + 1) * 4 + w.B * 4  # committed, accepted_len
    if w.mode != "greedy":
        small += w.B * w.K * 4 + w.B * 4 + w.B * w.K * 4  # uniforms, residual, target_prob
    if w.mode == "mixed":
        small += w.B * 4 * 3  # temperatures, row starts
    return logits + small, int(ks.sum())


def measured_traffic(workload_name, source="sv_kernels.hip"):
    """Calibrated HBM bytes per call from the committed rocprofv3 counter summary of this
    workload, or None when there is none or the kernel source changed since it was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_name}.md")
    src = os.path.join(ROOT, "lossless_draft_verification_sv_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and parts[0] in ("source_sha256", "traffic_bytes_per_call"):
            fields[parts[0]] = parts[1]
    if fields.get("source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    return float(fields["traffic_bytes_per_call"]) if "traffic_bytes_per_call" in fields else None


def _oracle_request(task):
    """One request through the fp64 oracle (runs in the bench process or a pool worker).
    Returns (b, k, ambiguous, n, committed, target_prob): the oracle's outputs, which the bench
    later sets beside the GPU's for the same request."""
    import oracle

    b, mode, dtype, tau, K, k, target, draft, tokens, uniforms, residual = task
    if tau > 0:
        r = oracle.verify_request(target, draft, dtype, tokens, uniforms, residual, tau, k, K)
        return b, k, bool(r.ambiguous), r.n, list(r.committed), list(r.target_prob)
    n, com = oracle.verify_greedy_request(target, dtype, tokens, k, K)
    return b, k, False, n, list(com), [0.0] * K


def _task(inp, b):
    w = inp.workload
    return (b, w.mode, w.dtype, w.temperature_of(b), w.K, inp.k_of(b), inp.target[b],
            None if inp.draft is None else inp.draft[b], inp.tokens[b],
            None if inp.uniforms is None else inp.uniforms[b],
            None if inp.residual is None else float(inp.residual[b]))


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo ("unknown" where it is not readable)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_check(results, acc, com, tp):
    """The oracle's outputs for the requests it ran (from the CPU-baseline leg) against the
    GPU's outputs of the timed calls: requests compared, ambiguous requests (a uniform within
    1e-6 of a decision threshold: counted, not compared), decision or token mismatches among
    the others, and the largest |target_prob - oracle|."""
    amb = mism = 0
    err = 0.0
    for b, k, ambiguous, n, committed, target_prob in results.values():
        if len(tp[b]):
            err = max(err, float(np.max(np.abs(tp[b] - np.asarray(target_prob)))))
        if ambiguous:
            amb += 1
        elif acc[b] != n or list(com[b]) != list(committed):
            mism += 1
    return {"requests": len(results), "ambiguous": amb, "mismatches": mism,
            "max_target_prob_err": err}


def cpu_baseline(inp, budget_s):
    """The fp64 oracle, as it stands, on the first requests of the workload until the budget is
    spent (at least one request). One thread (its work is elementwise numpy)."""
    w = inp.workload
    t0 = time.perf_counter()
    done, positions = 0, 0
    results = {}
    while done < w.B:
        r = _oracle_request(_task(inp, done))
        results[r[0]] = r
        positions += r[1]
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": positions / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {w.B} requests of {w.name} ({positions} positions, "
                      f"{dt:.1f} s, fp64 numpy, one thread)"}, results


def cpu_baseline_pool(inp, budget_s, workers):
    """The same oracle over requests in a pool of worker processes (spawned, so they hold no GPU
    state; each imports numpy and the oracle only). Requests are handed out until about
    budget_s of wall time has gone; the rate counts the requests finished by then."""
    import multiprocessing as mp

    w = inp.workload
    cores = min(workers, len(os.sched_getaffinity(0)))
    if cores < 1:
        return None, {}
    ctx = mp.get_context("spawn")
    saved = os.environ.get("OMP_NUM_THREADS")
    os.environ["OMP_NUM_THREADS"] = "1"  # inherited by the workers: one thread each
    try:
        pool = ctx.Pool(cores)
    finally:
        if saved is None:
            del os.environ["OMP_NUM_THREADS"]
        else:
            os.environ["OMP_NUM_THREADS"] = saved
    with pool:
        pool.map(_oracle_request, [_task(inp, 0)] * cores)  # start-up and imports, untimed
        t0 = time.perf_counter()
        done, positions = 0, 0
        results = {}
        pending = []
        b = 0
        while b < w.B or pending:
            while b < w.B and len(pending) < 2 * cores and time.perf_counter() - t0 < budget_s:
                pending.append(pool.apply_async(_oracle_request, (_task(inp, b),)))
                b += 1
            if not pending:
                break
            r = pending.pop(0).get()
            results[r[0]] = r
            positions += r[1]
            done += 1
        dt = time.perf_counter() - t0
    avail = len(os.sched_getaffinity(0))
    return {"value": positions / dt, "unit": "positions/s", "cores": cores, "kind": "oracle",
            "host_cores_available": avail, "cpu_model": cpu_model(),
            "sample": f"{done} of {w.B} requests of {w.name} ({positions} positions, {dt:.1f} s, "
                      f"fp64 numpy, a pool of {cores} worker processes, one request per task; "
                      f"{avail} cores in this process's affinity set, the pool capped at "
                      f"--cpu-workers {workers}: the GPU box's CPU share for one GPU)"}, results


def read_ceiling(lib, call_bytes, dev, stream):
    """Read bandwidth of this device with the library's read probe (every 16-byte word read once
    with non-temporal loads, a plain sum per work-group), the best over a few grid sizes:
    (1) one launch over a 2 GiB buffer, the streaming ceiling; (2) one launch per call-sized
    slice, rotated over disjoint slices of that buffer, the ceiling for a launch of this size
    (start-up and drain included). GB/s of bytes read."""
    import torch

    total = 2 << 30
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    size = max(16, min(call_bytes, total // 4) // 16 * 16)
    slices = [i * size for i in range(total // size)]

    def timed(args, reps):
        for a in args:
            if lib.sv_read_probe(*a) != 0:
                raise RuntimeError("sv_read_probe failed")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for a in args:
                lib.sv_read_probe(*a)
        e1.record(stream)
        torch.cuda.synchronize()
        return sum(a[1] for a in args) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    big = same = 0.0
    for groups in (1024, 2048, 4096, 8192):
        out = torch.empty(groups, dtype=torch.int32, device=dev)
        sp = stream.cuda_stream
        big = max(big, timed([(buf.data_ptr(), total, out.data_ptr(), groups, sp)], 5))
        same = max(same, timed([(buf.data_ptr() + o, size, out.data_ptr(), groups, sp)
                                for o in slices], 5))
    del buf
    return big, same


def bench_schedule(args):
    """The prefix scheduler (sv_schedule_prefix) at B=256, K=16: synthetic confidences and a
    step-time table measured on this device's verify kernel plus a synthetic target step."""
    import torch

    import lossless_draft_verification_sv_amd as sv
    import oracle
    from lossless_draft_verification_sv_amd.schedule import step_time_table
    from workloads import QWEN3_VOCAB, schedule_confidences

    B, K = 256, 16
    conf = schedule_confidences(B, K)
    dev = torch.device("cuda:0")
    tab = step_time_table(B, K, QWEN3_VOCAB, "bf16")
    c_d, t_d = torch.from_numpy(conf).to(dev), torch.from_numpy(tab).to(dev)
    lib = sv.load_library()
    out = torch.empty(B, dtype=torch.int32, device=dev)
    ts = torch.empty(B, dtype=torch.int32, device=dev)
    ds = torch.empty(B, dtype=torch.int32, device=dev)
    summ = torch.empty(2, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    nbytes = int(lib.sv_schedule_workspace_bytes(B, K))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    argv = (c_d.data_ptr(), B, K, t_d.data_ptr(), tab.shape[0], 0.5, out.data_ptr(),
            ts.data_ptr(), ds.data_ptr(), summ.data_ptr(), ws.data_ptr(), nbytes,
            stream.cuda_stream)
    for _ in range(args.warmup):
        assert lib.sv_schedule_prefix(*argv) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        lib.sv_schedule_prefix(*argv)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    num = out.cpu().numpy()
    n_chosen = int(summ[0].item())
    c0 = time.perf_counter()
    reps = 0
    while True:
        oracle.schedule_hardware_aware(conf, tab.astype(np.float64))
        reps += 1
        if time.perf_counter() - c0 > min(args.cpu_seconds, 5.0) or args.cpu_seconds <= 0:
            break
    cpu_s = (time.perf_counter() - c0) / reps
    result = {
        "metric": "scheduled draft tokens/s (sv_schedule_prefix, B*K tokens ranked per call)",
        "value": B * K / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic confidences; step table = measured verify kernel + synthetic target",
        "config": {"workload": "schedule_B256_K16", "B": B, "K": K,
                   "table_entries": int(tab.shape[0])},
        "call_us": {"mean_timed": us},
        "chosen_tokens": n_chosen, "mean_num_draft": float(num.mean()),
        "roofline": {"bound": "latency", "kernel": "sv_schedule_kernel", "achieved": us,
                     "peak": None, "unit": "us per call", "frac": None, "traffic": None},
        "cpu_baseline": {"value": B * K / cpu_s, "unit": "tokens/s", "cores": 1,
                         "kind": "oracle", "sample": f"{reps} full schedules, fp64 python"},
    }
    print(json.dumps(result), flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(json.dumps(result) + "\n")


def bench_markov(args, sampled=False):
    """The Markov-head correction (sv_markov_draft) of a draft block: 64 requests, 8 positions,
    the Qwen3 vocabulary, rank-256 synthetic bf16 factors, bf16 base logits. Two copies of the
    base and output logits alternate between steps. sampled: the sampled head
    (sv_markov_draft_sampled) at temperature 1 with one uniform per position, on base logits
    whose favoured token holds about half the mass (a sampling drafter's rows)."""
    import torch

    import lossless_draft_verification_sv_amd as sv
    import oracle
    from workloads import QWEN3_VOCAB, markov_base, markov_factors, markov_sampling

    B, K, V, R = 64, 8, QWEN3_VOCAB, 256
    dev = torch.device("cuda:0")
    base_h = markov_base(B, K, V, "bf16", lead=14.0 if sampled else 6.0)
    left_h, right_h = markov_factors(V, R)
    anchor_h = np.random.default_rng(1010).integers(0, V, size=B).astype(np.int32)
    tau_h, uni_h = markov_sampling(B, K)

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    bases = [bf16(base_h) for _ in range(2)]
    outs = [torch.empty_like(bases[0]) for _ in range(2)]
    left, right = bf16(left_h), bf16(right_h)
    anchor = torch.from_numpy(anchor_h).to(dev)
    tokens = torch.empty(B, K, dtype=torch.int32, device=dev)
    lib = sv.load_library()
    stream = torch.cuda.current_stream(dev)
    ws_bytes = int(lib.sv_markov_workspace_bytes(B, V))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if sampled:
        tau = torch.from_numpy(tau_h).to(dev)
        uni = torch.from_numpy(uni_h).to(dev)
        call = lib.sv_markov_draft_sampled
        argv = [[bases[i].data_ptr(), 1, B, K, V, left.data_ptr(), right.data_ptr(), R,
                 anchor.data_ptr(), tau.data_ptr(), uni.data_ptr(), tokens.data_ptr(),
                 outs[i].data_ptr(), ws.data_ptr(), ws_bytes, stream.cuda_stream]
                for i in range(2)]
    else:
        call = lib.sv_markov_draft
        argv = [[bases[i].data_ptr(), 1, B, K, V, left.data_ptr(), right.data_ptr(), R,
                 anchor.data_ptr(), tokens.data_ptr(), outs[i].data_ptr(), ws.data_ptr(),
                 ws_bytes, stream.cuda_stream] for i in range(2)]
    for i in range(max(args.warmup, 2)):
        if call(*argv[i % 2]) != 0:
            raise RuntimeError(sv.sv_last_error())
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        call(*argv[i % 2])
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    # algorithmic bytes per call: the right factor once (one call needs it at every position, but
    # nothing forces a second read), and the base and corrected logits of every position (the
    # left rows of the previous tokens, K*B*R*2 bytes, and the hand-off words are noise)
    alg = V * R * 2 + K * 2 * B * V * 2
    gbps = alg / (us * 1e-6) / 1e9
    wl = "markov_sampled_B64_K8_V151936_R256_bf16_t1" if sampled else "markov_B64_K8_V151936_R256_bf16"
    # the oracle on a bounded sample of requests, one by one, its BLAS held to one thread
    from threadpoolctl import threadpool_limits

    c0 = time.perf_counter()
    n_req = 0
    with threadpool_limits(limits=1):
        while n_req < B:
            if sampled:
                oracle.markov_sampled_request(base_h[n_req], "bf16", left_h, right_h,
                                              int(anchor_h[n_req]), float(tau_h[n_req]),
                                              uni_h[n_req])
            else:
                oracle.markov_draft_request(base_h[n_req], "bf16", left_h, right_h,
                                            int(anchor_h[n_req]))
            n_req += 1
            if args.cpu_seconds <= 0 or time.perf_counter() - c0 > args.cpu_seconds:
                break
    cpu_s = time.perf_counter() - c0
    result = {
        "metric": ("sampled Markov draft positions/s (sv_markov_draft_sampled, B*K positions per "
                   "call)" if sampled else
                   "Markov-corrected draft positions/s (sv_markov_draft, B*K positions per call)"),
        "value": B * K / (ms_per_step * 1e-3), "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic N(0, 0.25^2) rank-256 factors and N(0, 2^2) base logits" +
                (" with a +14 favoured token, temperature 1, seeded uniforms" if sampled else ""),
        "config": {"workload": wl, "B": B, "K": K, "V": V, "R": R},
        "call_us": {"mean_timed": us},
        "algorithmic_bytes_per_call": alg,
        "roofline": {"bound": "hbm", "kernel": ("sv_markov_draft_sampled (markov_resident"
                                                if sampled else
                                                "sv_markov_draft (markov_pipe, two request halves") +
                     ": one launch, the right factor in registers across positions)",
                     "achieved": gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(wl, "sv_markov.hip")},
        "cpu_baseline": {"value": n_req * K / cpu_s, "unit": "positions/s", "cores": 1,
                         "kind": "oracle", "sample": f"{n_req} requests x {K} positions, fp64 "
                                                     "numpy, one by one"},
    }
    print(json.dumps(result), flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(json.dumps(result) + "\n")


def bench_markov_topk(args):
    """Top-K Markov drafting (sv_markov_topk): 64 requests, 8 positions, the Qwen3 vocabulary,
    rank-256 synthetic bf16 factors, 64 candidates per position, bf16 base logits. Two copies of
    the base logits alternate between steps."""
    import torch

    import lossless_draft_verification_sv_amd as sv
    import oracle
    from workloads import QWEN3_VOCAB, markov_base, markov_factors

    B, K, V, R, KC = 64, 8, QWEN3_VOCAB, 256, 64
    dev = torch.device("cuda:0")
    base_h = markov_base(B, K, V, "bf16")
    left_h, right_h = markov_factors(V, R)
    anchor_h = np.random.default_rng(1010).integers(0, V, size=B).astype(np.int32)

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    bases = [bf16(base_h) for _ in range(2)]
    left, right = bf16(left_h), bf16(right_h)
    anchor = torch.from_numpy(anchor_h).to(dev)
    tokens = torch.empty(B, K, dtype=torch.int32, device=dev)
    cands = torch.empty(B, K, KC, dtype=torch.int32, device=dev)
    logits = torch.empty(B, K, KC, dtype=torch.float32, device=dev)
    lib = sv.load_library()
    stream = torch.cuda.current_stream(dev)
    ws_bytes = int(lib.sv_markov_topk_workspace_bytes(B, K, V))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    argv = [[bases[i].data_ptr(), 1, B, K, V, left.data_ptr(), right.data_ptr(), R, KC,
             anchor.data_ptr(), tokens.data_ptr(), cands.data_ptr(), logits.data_ptr(),
             ws.data_ptr(), ws_bytes, stream.cuda_stream] for i in range(2)]
    for i in range(max(args.warmup, 2)):
        if lib.sv_markov_topk(*argv[i % 2]) != 0:
            raise RuntimeError(sv.sv_last_error())
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        lib.sv_markov_topk(*argv[i % 2])
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    # algorithmic bytes per call: every base logit once, and the left and right factor rows of
    # every candidate (B*K*KC rows of R bf16 each); outputs and tables are small
    per_call = B * K * V * 2 + 2 * B * K * KC * R * 2
    gbps = per_call / (us * 1e-6) / 1e9
    from threadpoolctl import threadpool_limits

    c0 = time.perf_counter()
    n_req = 0
    with threadpool_limits(limits=1):
        while n_req < B:
            oracle.markov_topk_request(base_h[n_req], "bf16", left_h, right_h,
                                       int(anchor_h[n_req]), KC)
            n_req += 1
            if args.cpu_seconds <= 0 or time.perf_counter() - c0 > args.cpu_seconds:
                break
    cpu_s = time.perf_counter() - c0
    result = {
        "metric": "top-K Markov draft positions/s (sv_markov_topk, B*K positions per call)",
        "value": B * K / (ms_per_step * 1e-3), "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic N(0, 0.25^2) rank-256 factors and N(0, 2^2) base logits",
        "config": {"workload": "markov_topk_B64_K8_V151936_R256_kc64_bf16", "B": B, "K": K,
                   "V": V, "R": R, "kc": KC},
        "call_us": {"mean_timed": us},
        "algorithmic_bytes_per_call": per_call,
        "roofline": {"bound": "hbm", "kernel": "sv_markov_topk (topk_chunk + topk_merge + "
                     "topk_bias + topk_walk)", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": measured_traffic("markov_topk_B64_K8_V151936_R256_kc64_bf16",
                                                 "sv_markov_topk.hip")},
        "cpu_baseline": {"value": n_req * K / cpu_s, "unit": "positions/s", "cores": 1,
                         "kind": "oracle", "sample": f"{n_req} requests x {K} positions, fp64 "
                                                     "numpy, one by one"},
    }
    print(json.dumps(result), flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(json.dumps(result) + "\n")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1 (requests are "
                                   "independent: a multi-GPU run would shard the batch)"}))
        sys.exit(2)

    import torch

    import lossless_draft_verification_sv_amd as sv
    from workloads import flatten, generate

    if args.workload == "schedule":
        return bench_schedule(args)
    if args.workload == "markov":
        return bench_markov(args)
    if args.workload == "markov_sampled":
        return bench_markov(args, sampled=True)
    if args.workload == "markov_topk":
        return bench_markov_topk(args)
    w = pick_workload(args.workload)
    inp = generate(w)
    # the pooled oracle runs first, before this process touches the GPU
    pooled, pooled_results = (cpu_baseline_pool(inp, args.cpu_seconds, args.cpu_workers)
                              if args.cpu_seconds > 0 and args.cpu_workers > 0 else (None, {}))
    dev = torch.device("cuda:0")

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    flat = flatten(inp) if w.mode == "mixed" else None
    t0 = up(inp.target if flat is None else flat.target)
    d0 = up(inp.draft if flat is None else flat.draft)
    per_copy = t0.numel() * t0.element_size() + (0 if d0 is None else d0.numel() * d0.element_size())
    copies = max(1, int(np.ceil(args.min_rotation_bytes / per_copy)))
    targets = [t0] + [t0.clone() for _ in range(copies - 1)]
    drafts = [d0] + ([d0.clone() for _ in range(copies - 1)] if d0 is not None else
                     [None] * (copies - 1))
    tokens, uniforms, residual = up(inp.tokens), up(inp.uniforms), up(inp.residual)
    num_draft = up(inp.num_draft if flat is None else flat.num_draft)
    B, K, V = w.B, w.K, w.V
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    com = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    tp = torch.empty(B, K, dtype=torch.float32, device=dev)
    lib = sv.load_library()
    nbytes = int(lib.sv_workspace_bytes(B, K, V))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)  # zero-filled once
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    code = sv.SV_DTYPE_BF16 if w.dtype == "bf16" else sv.SV_DTYPE_F32
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731

    # Arguments of every step, built once: the timed loop only calls into the library.
    if w.mode == "mixed":
        fn = lib.sv_verify_ragged
        temps, ts, ds = up(flat.temperatures), up(flat.target_row_start), up(flat.draft_row_start)
        rows_d = 0 if d0 is None else d0.shape[0]
        argv = [(P(targets[c]), P(drafts[c]), code, B, K, V, t0.shape[0], rows_d, P(ts), P(ds),
                 P(num_draft), P(temps), P(tokens), P(uniforms), P(residual), P(acc), P(com),
                 P(tp), None, P(ws), nbytes, sptr) for c in range(copies)]
    elif w.mode == "sample":
        fn = lib.sv_verify_batch
        argv = [(P(targets[c]), P(drafts[c]), code, B, K, V, float(w.temperature), P(tokens),
                 P(num_draft), P(uniforms), P(residual), P(acc), P(com), P(tp), None, P(ws),
                 nbytes, sptr) for c in range(copies)]
    else:
        fn = lib.sv_verify_greedy
        argv = [(P(targets[c]), code, B, K, V, P(tokens), P(num_draft), P(acc), P(com), P(ws),
                 nbytes, sptr) for c in range(copies)]

    def step(i):
        st = fn(*argv[i % copies])
        if st != 0:
            raise RuntimeError(f"sv call failed: {st} {sv.sv_last_error()}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K back-to-back calls between two events on the launch stream (the average
    # launch duration), bracketed by device synchronisations for the wall clock.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    avg_us = e0.elapsed_time(e1) * 1e3 / args.steps

    # Spread of single calls (untimed sample, one event pair per call).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(20)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])

    alg_bytes, positions = algorithmic_bytes(inp)
    acc_np = acc.cpu().numpy()
    ks = np.array([inp.k_of(b) for b in range(B)])
    if not (np.all(acc_np >= 0) and np.all(acc_np <= ks)):
        raise RuntimeError(f"accepted lengths outside [0, k_b]: {acc_np.tolist()}")
    gbps = alg_bytes / (avg_us * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": positions / (ms_per_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type of the path (fp32, with fp64 combines and draws); the logits'
        # storage type is logit_dtype
        "dtype": "f32",
        "logit_dtype": w.dtype,
        "data": "synthetic (seeded numpy logits shaped like the pages' workloads; no dataset)",
        "config": {"workload": w.name, "B": B, "K": K, "V": V, "logits": w.dtype,
                   "temperature": w.temperature, "mode": w.mode,
                   "ragged": inp.num_draft is not None, "input_copies_rotated": copies},
        "achieved_gbps": gbps,
        "hbm_peak_frac": gbps / HBM_PEAK_GBPS,
        "call_us": {"mean_timed": avg_us, "single_call_median": float(np.median(call_us)),
                    "single_call_p10": float(np.percentile(call_us, 10)),
                    "single_call_p90": float(np.percentile(call_us, 90))},
        "positions_per_call": positions,
        "algorithmic_bytes_per_call": alg_bytes,
        "mean_acceptance_length": float(np.mean(acc_np + 1)),
        "roofline": {"bound": "hbm",
                     "kernel": {"sample": "sv_verify_sample", "greedy": "sv_verify_greedy",
                                "mixed": "sv_verify_ragged_kernel"}[w.mode],
                     "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": measured_traffic(w.name)},
    }
    if not args.skip_ceiling:
        big, same = read_ceiling(lib, alg_bytes, dev, stream)
        result["read_ceiling_gbps"] = big
        result["frac_of_read_ceiling"] = gbps / big
        result["read_probe_call_size_gbps"] = same
        result["frac_of_call_size_probe"] = gbps / same
    if args.cpu_seconds > 0:
        single, single_results = cpu_baseline(inp, args.cpu_seconds)
        result["cpu_baseline"] = pooled if pooled is not None else single
        result["cpu_baseline_one_thread"] = single
        results = pooled_results if len(pooled_results) >= len(single_results) else single_results
        chk = oracle_check(results, acc_np, com.cpu().numpy(), tp.cpu().numpy())
        result["oracle_check"] = chk
        result["ambiguous"] = chk["ambiguous"]
    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
