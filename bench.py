#!/usr/bin/env python3
"""Benchmark of the Domino head block draft on one MI355X.

One step = one call of domino_head_draft: the whole drafting loop (A_H
precompute, anchor GRU step, then 16 x (low-rank activation, W2 correction +
residual + greedy argmax, embedding gather + GRU step)) over one batch of
seeded synthetic inputs already resident in device memory.

Prints ONE JSON line on stdout.  Diagnostics go to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def logical_bytes(sh, B, store_logits=False, fold=False, lbase_bytes=4, markov=False):
    """Algorithmic bytes of one block draft: every operand each step reads once.

    Per position (K of them): W2 [V,r], the L_base slice [B,V] fp32 and the state
    columns of W1 [r,h].  Per GRU step (K of them: the anchor plus K-1 fed-back
    tokens): W_hh [3h,h] and both bias vectors, plus the input part: W_ih [3h,d]
    and the gathered embedding rows [B,d], or with the folded table one gathered
    row of P [B,3h] fp32.  Once per call: the H columns of W1 [r,d], H [B,K,d] and
    the tokens [B,K].  L_base takes ``lbase_bytes`` per value (2 for bf16 input).
    Markov head: no GRU step and no W1_S product; each position gathers one row of
    the per-token table M [B,r] fp32 instead.
    Returns (total, w2_and_lbase).
    """
    s = 4 if sh.wdtype == "f32" else 2
    K, V, r, h, d = sh.K, sh.V, sh.r, sh.h, sh.d
    if markov:
        per_pos = V * r * s + B * V * lbase_bytes + B * r * 4
        per_gru = 0
    else:
        per_pos = V * r * s + B * V * lbase_bytes + r * h * s
        gru_in = B * 3 * h * 4 if fold else 3 * h * d * s + B * d * s
        per_gru = gru_in + 3 * h * h * s + 6 * h * s
    once = r * d * s + B * K * d * s + B * K * 4
    total = K * per_pos + K * per_gru + once
    if store_logits:
        total += B * K * V * 4
    return total, K * (V * r * s + B * V * lbase_bytes)


def algorithmic_flops(sh, B, fold=False, markov=False):
    """Useful FLOPs of one call (the matrix-core path computes W2 and the state dot
    products twice, on bf16 hi and lo parts; that is not counted).  Returns
    (W2 only, all contractions: W2 + W1 + GRU)."""
    K, V, r, h, d = sh.K, sh.V, sh.r, sh.h, sh.d
    w2 = 2 * B * r * V * K
    if markov:  # only the H columns of W1; the state part is a table gather
        return w2, w2 + 2 * B * r * d * K
    w1 = 2 * B * r * (d + h) * K
    gru = 2 * B * 3 * h * h * K + (0 if fold else 2 * B * 3 * h * d * K)
    return w2, w2 + w1 + gru


MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


# Sources each timed launch kind is compiled from: a counter summary stays valid while these
# files are unchanged (changes elsewhere in the library do not touch the kernel).
KERNEL_SOURCES = {
    "persistent_res": ["domino_head_res.hip", "dh_resident.h", "dh_phases.h", "dh_common.h", "dh_params.h"],
    "markov_res": ["domino_head_res.hip", "dh_resident.h", "dh_phases.h", "dh_common.h", "dh_params.h"],
    "persistent_rb": ["domino_head_rb.hip", "dh_rbatch.h", "dh_phases.h", "dh_common.h", "dh_params.h"],
    "persistent": ["domino_head.hip", "dh_phases.h", "dh_common.h", "dh_params.h"],
    "stepwise": ["domino_head.hip", "domino_head_bat.hip", "dh_batched.h", "dh_phases.h", "dh_common.h",
                 "dh_params.h"],
    "verify": ["domino_verify.hip", "dh_verify.h", "dh_common.h"],
}
# the kernel each persistent launch kind runs (the stepwise kind is a sequence of launches)
KERNEL_NAMES = {"persistent_res": "k_persistent_res", "markov_res": "k_markov_res",
                "persistent_rb": "k_persistent_rb", "persistent": "k_persistent",
                "stepwise": "stepwise launches (whole call)"}


def kernel_source_hash(kind):
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "causal_draft_correction_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kind, fold):
    """HBM bytes per call from the committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE
    over the call's launches, scaled by a plain copy of known size), when it was taken on the
    current kernel sources, the same workload and the same launch kind; else None."""
    import glob

    cur = kernel_source_hash(kind)
    for f in glob.glob(os.path.join(ROOT, "profiles", "*_counters.json")):
        with open(f) as fh:
            d = json.load(fh)
        if (d.get("kernel_source_sha256_16") == cur and d.get("workload") == workload and
                d.get("exec") == kind and bool(d.get("fold_embedding")) == fold):
            return d["traffic_bytes_per_launch"]
    return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def achievable_rates():
    """What the box reaches on plain library work, beside the vendor peaks: a 1 GiB device
    copy (read + write bytes / time) and a 8192^3 bf16 matrix product (torch.mm)."""
    import torch

    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    for _ in range(2):
        dst.copy_(src)
        torch.mm(a, b)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    for _ in range(5):
        dst.copy_(src)
    e[1].record()
    for _ in range(5):
        torch.mm(a, b)
    e[2].record()
    torch.cuda.synchronize()
    copy_s = e[0].elapsed_time(e[1]) * 1e-3 / 5
    mm_s = e[1].elapsed_time(e[2]) * 1e-3 / 5
    del src, dst, a, b
    return {"copy_GBps": 2 * n * 4 / copy_s / 1e9, "bf16_gemm_8192_TFLOPs": 2 * 8192 ** 3 / mm_s / 1e12}


def cpu_baseline(w, inp, budget_s, markov=False):
    """The fp64 oracle as it stands, on this host's cores, on row 0 of the workload; then one
    draft of the same row on one thread.  Returns (drafts, seconds, threads, one-thread seconds)."""
    import oracle

    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.draft(w, inp.H[:1], inp.L_base[:1], inp.last_tok[:1], want_logits=False, want_state=False,
                     markov=markov)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    t1 = time.perf_counter()
    oracle.draft(w, inp.H[:1], inp.L_base[:1], inp.last_tok[:1], want_logits=False, want_state=False,
                 markov=markov, threads=1)
    return n, el, oracle.max_threads(), time.perf_counter() - t1


def run_verify(args, wl):
    """The greedy verify step on the workload's B, K and V: target logits [B, K+1, V] and the
    drafted tokens [B, K] resident on the device, one domino_verify call per step."""
    import numpy as np
    import torch

    import causal_draft_correction_amd as dca
    import domino_synth as ds

    sh = wl.shape
    B, K, V = wl.B, sh.K, sh.V
    eprint("bench: generating verify inputs (B=%d, K=%d, V=%d)" % (B, K, V))
    vi = ds.make_verify_inputs(B, K, V, list(wl.row_key) + [7])
    lg = dca.device_tensor(vi.logits)
    dr = dca.device_tensor(vi.draft)
    ws = torch.empty(max(dca.verify_workspace_size(B, K, V), 16), dtype=torch.uint8, device="cuda")
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy * (1 << 20) // 4, dtype=torch.float32, device="cuda")
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    out = {"accept": torch.empty(B, dtype=torch.int32, device="cuda"),
           "next": torch.empty(B, dtype=torch.int32, device="cuda"),
           "target": torch.empty((B, K + 1), dtype=torch.int32, device="cuda")}
    for _ in range(args.warmup):
        dca.verify(lg, dr, ws, out=out)
    torch.cuda.synchronize()
    # the planted construction fixes the accept lengths
    assert np.array_equal(out["accept"].cpu().numpy(), np.minimum(vi.k, K))
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        dca.verify(lg, dr, ws, out=out)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [a.elapsed_time(b) for a, b in ev]
    avg_ms = float(np.mean(per_call_ms))
    cold_us = None
    if args.cold_calls > 0:
        evict = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_calls)]
        for i in range(args.cold_calls):
            evict.fill_(float(i))
            cev[i][0].record(stream)
            dca.verify(lg, dr, ws, out=out)
            cev[i][1].record(stream)
        torch.cuda.synchronize()
        cold_us = float(np.median([a.elapsed_time(b) for a, b in cev])) * 1e3
        del evict
    # algorithmic bytes: every logit once, the draft, the outputs
    total_bytes = B * (K + 1) * V * 4 + B * K * 4 + B * (K + 1) * 4 + 2 * B * 4
    achieved = total_bytes / (avg_ms * 1e-3) / 1e9
    achieved_cold = None if cold_us is None else total_bytes / (cold_us * 1e-6) / 1e9
    name = "verify_" + wl.name
    traffic = measured_traffic(name, "verify", False)
    hbm_actual = None if traffic is None else traffic / (avg_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = min(B, 4)
        n = 0
        t1 = time.perf_counter()
        while True:
            oracle.verify(vi.logits[:rows], vi.draft[:rows])
            n += rows
            el = time.perf_counter() - t1
            if el >= min(args.cpu_budget, 5.0):
                break
        cpu = {"value": n / el, "unit": "blocks/s", "cores": 1, "kind": "oracle",
               "sample": "%d verify steps of %d-row slices of the same inputs (K=%d, V=%d), C oracle, one thread" % (
                   n // rows, rows, K, V), "cpu_model": cpu_model(), "host_cores": host_cores()}
    rec = {
        "metric": "greedy verify: drafted blocks checked per second (K+1 target rows of V logits each) at 1 GPU",
        "value": B * args.steps / wall,
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "B": B, "K": K, "V": V, "call_avg_us": avg_ms * 1e3,
                   "warm_us_per_call_median": float(np.median(per_call_ms)) * 1e3,
                   "cold_us_per_call_median": cold_us},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic, "algorithmic_bytes": total_bytes,
                     "kernel": "k_verify_rows + k_verify_final", "achieved_cold": achieved_cold,
                     "frac_cold": None if achieved_cold is None else achieved_cold / HBM_PEAK_GBPS,
                     "hbm_actual_GBps": hbm_actual,
                     "hbm_actual_frac": None if hbm_actual is None else hbm_actual / HBM_PEAK_GBPS},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_8b_b1")
    ap.add_argument("--mode", default="auto", choices=["auto", "persistent", "stepwise"])
    ap.add_argument("--stream-w2", action="store_true",
                    help="persistent launch: stream W2 every position instead of keeping it on chip")
    ap.add_argument("--plain-launch", action="store_true",
                    help="persistent launch as an ordinary kernel launch (caller guarantees no concurrent waiting "
                         "kernels); the default is a cooperative launch")
    ap.add_argument("--store-logits", action="store_true")
    ap.add_argument("--no-fold", action="store_true",
                    help="do not precompute the folded input-gate table (GRU input GEMV every step)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the achievable copy / bf16 GEMM rates printed beside the vendor peaks")
    ap.add_argument("--teacher", action="store_true",
                    help="teacher-forced drafting: a seeded uniform teacher token row per batch row")
    ap.add_argument("--position-batched", action="store_true",
                    help="with --teacher: the GRU chain first, then one W2 launch for all positions (B <= 8 too)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one draft call in a HIP graph (torch.cuda.CUDAGraph) and replay it per step")
    ap.add_argument("--lbase-bf16", action="store_true",
                    help="L_base given as bfloat16 (DOMINO_LBASE_BF16): the workload's base logits rounded to bf16")
    ap.add_argument("--markov", action="store_true",
                    help="the Markov head (each position conditioned on the preceding token alone)")
    ap.add_argument("--verify", action="store_true",
                    help="time the greedy verify step (domino_verify) on the workload's B, K and V instead")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="calls timed one by one after writing a 512 MiB buffer that evicts the caches "
                         "(the serving case: the target model's verify pass runs between two drafts)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of MIB MiB before timing (reference for profiler byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        eprint("bench.py runs on one GPU only: the Domino head path here is single-device "
               "(batch rows shard trivially across GPUs with no exchange); --gpus %d is not supported" % args.gpus)
        sys.exit(2)

    import numpy as np
    import torch

    import causal_draft_correction_amd as dca
    import domino_synth as ds

    torch.cuda.set_device(0)
    wl = ds.WORKLOADS[args.workload]
    if args.verify:
        run_verify(args, wl)
        return
    sh = wl.shape
    eprint("bench: generating %s (B=%d, d=%d, h=%d, r=%d, V=%d, %s)" % (wl.name, wl.B, sh.d, sh.h, sh.r, sh.V,
                                                                      sh.wdtype))
    w, inp = ds.make_workload(wl.name)
    mode = {"auto": dca.EXEC_AUTO, "persistent": dca.EXEC_PERSISTENT, "stepwise": dca.EXEC_STEPWISE}[args.mode]
    fold = not args.no_fold and not args.markov
    t_create = time.perf_counter()
    head = dca.DominoHead(dca.head_weights_to_device(w), K=sh.K, max_batch=wl.B,
                          exec_mode=mode | (dca.EXEC_STREAM_W2 if args.stream_w2 else 0) |
                          (dca.EXEC_PLAIN_LAUNCH if args.plain_launch else 0) |
                          (dca.EXEC_POSITION_BATCHED if args.position_batched else 0), fold_embedding=fold,
                          lbase_bf16=args.lbase_bf16, markov=args.markov)
    torch.cuda.synchronize()
    t_create = time.perf_counter() - t_create
    H = dca.device_tensor(inp.H)
    L = dca.device_tensor(ds.round_to_bf16_bits(inp.L_base) if args.lbase_bf16 else inp.L_base)
    lt = dca.device_tensor(inp.last_tok)
    teacher = dca.device_tensor(ds.uniform_tokens(list(wl.row_key) + [9], (wl.B, sh.K), sh.V)) if args.teacher else None
    out = {"tokens": torch.empty((wl.B, sh.K), dtype=torch.int32, device="cuda")}
    if args.store_logits:
        out["L_final"] = torch.empty((wl.B, sh.K, sh.V), dtype=torch.float32, device="cuda")
    info = head.exec_info(wl.B)
    if not info["persistent"]:
        kind = "stepwise"
    elif not info["w2_resident"]:
        kind = "persistent"
    elif wl.B > 8:
        kind = "persistent_rb"
    else:
        kind = "markov_res" if args.markov else "persistent_res"
    exec_name = "persistent" if info["persistent"] else "stepwise"
    if args.teacher and (args.position_batched or not info["persistent"]):
        info = dict(info, persistent=False, w2_resident=False)
        exec_name = "stepwise, position-batched"
        kind = "stepwise"

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        eprint("bench: calibration copy of %d MiB done" % args.calibrate_copy)
        del src, dst

    def call():
        head.draft(H, L, lt, teacher=teacher, out=out)

    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                call()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        torch.cuda.synchronize()
        call = graph.replay  # noqa: F811
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    assert head.check_error() == 0
    eprint("bench: warmup done, timing %d steps" % args.steps)

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    flags = head.check_error()
    assert flags == 0, "device flags %d" % flags
    per_call_ms = [a.elapsed_time(b) for a, b in ev]
    avg_ms = float(np.mean(per_call_ms))

    # cold calls: a 512 MiB write between calls evicts L2 and the 256 MB MALL, so the
    # call reads its weights from HBM as it does between two verify passes
    cold_us = None
    if args.cold_calls > 0:
        evict = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_calls)]
        for i in range(args.cold_calls):
            evict.fill_(float(i))
            cev[i][0].record(stream)
            call()
            cev[i][1].record(stream)
        torch.cuda.synchronize()
        assert head.check_error() == 0
        cold_us = float(np.median([a.elapsed_time(b) for a, b in cev])) * 1e3
        del evict
    ms_per_step = wall * 1e3 / args.steps
    blocks_per_s = wl.B * args.steps / wall

    total_bytes, w2l_bytes = logical_bytes(sh, wl.B, args.store_logits, fold, 2 if args.lbase_bf16 else 4,
                                           args.markov)
    achieved = total_bytes / (avg_ms * 1e-3) / 1e9
    w2l = w2l_bytes / (avg_ms * 1e-3) / 1e9
    w2_on_chip = info["w2_resident"]
    # counters are taken on the plain fp32-L_base free-running call of each workload
    traffic = (measured_traffic(wl.name + ("_markov" if args.markov else ""), kind, fold)
               if not args.lbase_bf16 and not args.teacher and not args.store_logits and not args.graph else None)
    kname = KERNEL_NAMES[kind]
    hbm_actual = None if traffic is None else traffic / (avg_ms * 1e-3) / 1e9
    # a persistent launch runs the K positions as one dependent chain inside one kernel: up to
    # B = 64 its time is set by the per-position latency (phases, grid barriers), not by HBM (the
    # counters show it far from busy) or the matrix cores.  Larger batches stream L_base (155.6 MB
    # per position at B = 256, half of each position's time), like the step launches
    bound = "latency" if info["persistent"] and wl.B <= 64 else "hbm"

    f_w2, f_all = algorithmic_flops(sh, wl.B, fold, args.markov)
    mfma = {"w2_tflops": f_w2 / (avg_ms * 1e-3) / 1e12, "all_tflops": f_all / (avg_ms * 1e-3) / 1e12,
            "peak_tflops": MFMA_PEAK_TFLOPS}
    mfma["w2_frac"] = mfma["w2_tflops"] / MFMA_PEAK_TFLOPS
    mfma["all_frac"] = mfma["all_tflops"] / MFMA_PEAK_TFLOPS

    cpu = None
    if not args.no_cpu_baseline:
        eprint("bench: timing the fp64 oracle on the host (cpu_baseline)")
        n, el, threads, one_s = cpu_baseline(w, inp, args.cpu_budget, args.markov)
        cpu = {"value": n / el, "unit": "blocks/s", "cores": threads, "kind": "oracle",
               "sample": "%d block draft(s) of row 0 of %s (free running, K=%d, V=%d%s), fp64 C oracle on %d "
                         "threads; then one draft of the same row on one thread" % (
                             n, wl.name, sh.K, sh.V, ", Markov head" if args.markov else "", threads),
               "cpu_model": cpu_model(), "host_cores": host_cores(), "one_thread_s_per_block": one_s}
    calib = None
    if not args.no_calibration:
        eprint("bench: achievable copy and bf16 GEMM rates")
        calib = achievable_rates()

    cold_achieved = None if cold_us is None else total_bytes / (cold_us * 1e-6) / 1e9
    rec = {
        "metric": "Domino-head draft blocks/sec (16 tok, V=151936) + achieved HBM GB/s at 1 GPU",
        "value": blocks_per_s,
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sh.wdtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "K": sh.K, "V": sh.V, "d": sh.d, "h": sh.h, "r": sh.r,
                   "weights": sh.wdtype, "accumulate": "f32", "lbase_dtype": "bf16" if args.lbase_bf16 else "f32",
                   "exec": exec_name, "kernel": kname, "grid": info["grid"],
                   "store_logits": bool(args.store_logits), "fold_embedding": fold, "w2_on_chip": w2_on_chip,
                   "launch": "plain" if args.plain_launch else "cooperative", "create_s": t_create,
                   "teacher_forced": bool(args.teacher),
                   "head": "markov" if args.markov else "recurrent (GRU)",
                   "hip_graph": bool(args.graph),
                   "call_avg_us": avg_ms * 1e3, "warm_us_per_call_median": float(np.median(per_call_ms)) * 1e3,
                   "cold_us_per_call_median": cold_us, "us_per_position": avg_ms * 1e3 / sh.K,
                   "w2_lbase_GBps": w2l, "w2_lbase_frac_of_hbm_peak": w2l / HBM_PEAK_GBPS,
                   "matrix_core_use": mfma, "achievable": calib},
        # achieved/frac: algorithmic bytes per call over the mean hipEvent call time of the timed
        # steps (an effective rate: W2 that stays on chip counts once per position); the _cold
        # figures repeat it on calls made after evicting L2 and MALL, the serving case;
        # hbm_actual: the bytes the counters saw per call over the same mean call time
        "roofline": {"bound": bound, "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes": total_bytes, "kernel": kname,
                     "achieved_cold": cold_achieved,
                     "frac_cold": None if cold_achieved is None else cold_achieved / HBM_PEAK_GBPS,
                     "hbm_actual_GBps": hbm_actual,
                     "hbm_actual_frac": None if hbm_actual is None else hbm_actual / HBM_PEAK_GBPS,
                     "us_per_position": avg_ms * 1e3 / sh.K},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
