"""Per-phase timing of one persistent draft call, from device timestamps.

Loads libdomino_trace.so (built beside libdomino_head.so by build.py: the same
library with the phase hooks of the resident persistent kernels recording the
100 MHz device clock per block), drafts a named synthetic workload a few
times, then reads the timestamps of the last call and reports, per phase, the
median over blocks (and the slowest block) of the time between its two marks.
Positions 1..K-2 are summarised by the median over positions; the anchor step,
the first and the last position are listed separately.

    python -m causal_draft_correction_amd.phase_trace qwen3_8b_b1 [qwen3_8b_b32 ...] [--json]
        [--persistent] [--lbase-bf16] [--no-fold] [--plain-launch]

--persistent forces the persistent launch where the automatic choice would take
the step launches (the batched kernel up to B = 256); --lbase-bf16 passes the
base logits as bfloat16; --no-fold drafts without the folded gate table (the GRU
input product runs at every step; B <= 8 only); --plain-launch starts the same
kernel with an ordinary launch instead of a cooperative one (for a process that
runs while another one that has made cooperative launches on the GPU is alive).

Only this tool loads the instrumented library; it needs a GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TICK_US = 0.01  # the device clock runs at 100 MHz
BLOCKS, SLOTS = 256, 1024

# resident B <= 8 kernels (k_persistent_res): hook slot + 64 is the column
RES_BIAS = 64
# (name, first mark, second mark) relative to 32 * position
RES_POSITION = [("w2_wait_u", 0, 1), ("w2_products", 2, 4), ("w2_block_key", 4, 5), ("argmax_exchange", 5, 13),
                ("input_product", 13, 16), ("gru_gates", 16, 18), ("state_sync", 18, 19), ("state_dots", 19, 20), ("u_hop", 20, 32),
                ("position", 0, 32)]
# wave 0's first group of state rows (its u row) in the state dots: products and
# sums, the stores, then the other rows
RES_DOTS = [("dots_first_group", 19, 21), ("dots_first_stores", 21, 22), ("dots_other_rows", 22, 20),
            ("dots_first_setup", 19, 23), ("dots_first_products", 23, 24), ("dots_first_sums", 24, 21),
            ("mark_cost", 13, 15)]
# the argmax exchange (arrival; next L_base slice issued; the wait for every block and
# the reduction) and the gate update (the input token to LDS; the P row, q and state
# loads landed; the cell and its stores)
RES_SPLIT = [("exchange_arrive", 5, 6), ("exchange_lbase_issue", 6, 7), ("exchange_wait", 7, 13),
             ("gates_token", 16, 17), ("gates_loads_landed", 17, 25), ("gates_cell", 25, 18)]
# unfolded head: the input product itself and its grid barrier
RES_UNFOLDED = [("input_product_compute", 13, 14), ("input_product_barrier", 14, 16)]
RES_PROLOGUE = [("slice_and_loads_issued", 511, 508), ("anchor_step", -16, -12), ("prologue", 511, 509)]
# the prologue of a B = 1 launch without initial state (no grid barrier): the first
# L_base slice issued, the state rows to LDS, the A_H entries of the block's u rows;
# then the anchor step's gate update, the W2 slice load issued after it, the dots
RES_PROLOGUE_FAST = [("lbase_issue", 511, 507), ("state_rows_to_lds", 507, 506), ("ah_entries", 506, 505),
                     ("anchor_gates", -16, -14), ("w2_slice_issue", -14, -13), ("anchor_dots", -13, -12),
                     ("anchor_first_dot_group", -13, -11), ("to_first_w2", -12, 0)]

# batched kernel (k_persistent_rb): hook slot is the column; marks relative to 64 * position
RB_POSITION = [("wait_u", 0, 7), ("w2", 7, 1), ("resolve", 1, 2), ("gru_update", 2, 3), ("grid_barrier", 3, 4),
               ("state_dots", 4, 5), ("to_next_position", 5, 64), ("position", 0, 64)]
RB_PROLOGUE = [("w2_slice_load", 1019, 1023), ("anchor_update", 1023, 1022), ("grid_barrier", 1022, 1021),
               ("anchor_dots", 1021, 1020), ("prologue", 1019, 1020)]
# the state dots mark the first round (B <= 64) or the first job (B > 64) of a block at
# slots 64 q + 40..43 of the state q they compute, i.e. 64 + 40.. after the position
# before it.  B <= 64: copies issued, landed, products, reduction and stores; B > 64:
# the first three stages issued, the first stage landed and multiplied, the other
# stages, reduction and stores (with the arrival count)
RB_DOTS = [("dots_copies_issued", 4, 64 + 40), ("dots_copies_landed", 64 + 40, 64 + 41),
           ("dots_products", 64 + 41, 64 + 42), ("dots_reduce_store", 64 + 42, 64 + 43)]


def _span(t, a, b):
    d = (t[:, b] - t[:, a]).astype(np.float64) * TICK_US
    return float(np.median(d)), float(d.max())


def w2_groups(t, K, ngr):
    """Batched kernel: the W2 phase per 16-row group (positions 1..K-2, median over
    positions and blocks, in us): the wait for a group's copies (from the previous
    group's end, or from the end of the wait for u) and its products and epilogue,
    for the first group, the median of the middle ones and the last, and the time
    from the last group's end to the phase's end."""
    mids = range(1, K - 1)
    if not len(mids) or ngr < 1:
        return {}

    def span(a, b):
        return float(np.median(np.concatenate([(t[:, 64 * p + b] - t[:, 64 * p + a]) for p in mids]))) * TICK_US

    wait = [span(7 if g == 0 else 9 + 2 * (g - 1), 8 + 2 * g) for g in range(ngr)]
    work = [span(8 + 2 * g, 9 + 2 * g) for g in range(ngr)]
    out = {"first_wait": wait[0], "first_group": work[0], "last_wait": wait[-1], "last_group": work[-1],
           "after_last_group": span(9 + 2 * (ngr - 1), 1)}
    if ngr > 2:
        out["middle_wait"] = float(np.median(wait[1:-1]))
        out["middle_group"] = float(np.median(work[1:-1]))
    return {k: [round(v, 2), round(v, 2)] for k, v in out.items()}


def summarize(t, K, batched, dots_detail=False, unfolded=False):
    """t: [blocks, SLOTS] int64 timestamps of one call.  Returns a dict of phase -> [median, max] us."""
    if batched:
        col = lambda s: s  # noqa: E731
        per, pro, stride, end = RB_POSITION, RB_PROLOGUE, 64, 64 * (K - 1) + 2
        if dots_detail:
            per = per + RB_DOTS
        start = 1019
    else:
        col = lambda s: s + RES_BIAS  # noqa: E731
        per, pro, stride, end = RES_POSITION + RES_DOTS + RES_SPLIT, RES_PROLOGUE, 32, 32 * (K - 1) + 13
        if unfolded:
            per = per + RES_UNFOLDED
        start = 511
    out = {"kernel_us": round(float((t[:, col(end)].max() - t[:, col(start)].min()) * TICK_US), 1)}
    out["prologue"] = {n: [round(x, 2) for x in _span(t, col(a), col(b))] for n, a, b in pro}
    if not batched and (t[:, col(505)] > 0).all():
        out["prologue"].update({n: [round(x, 2) for x in _span(t, col(a), col(b))] for n, a, b in RES_PROLOGUE_FAST})
    for p in sorted({0, K - 1}):
        out["position_%d" % p] = {n: [round(x, 2) for x in _span(t, col(stride * p + a), col(stride * p + b))]
                                  for n, a, b in per if stride * p + max(a, b) <= end}
    mids = range(1, K - 1)
    if len(mids):
        out["positions_1_to_%d_median" % (K - 2)] = {
            n: [round(float(np.median([_span(t, col(stride * p + a), col(stride * p + b))[i] for p in mids])), 2)
                for i in (0, 1)] for n, a, b in per}
    return out


def run(names, lib_path=None, persistent=False, lbase_bf16=False, fold=True, plain_launch=False):
    sys.path.insert(0, ROOT)
    import torch

    from causal_draft_correction_amd import binding

    lib = binding.load_library(lib_path or os.path.join(HERE, "libdomino_trace.so"))
    import causal_draft_correction_amd as dca
    import domino_synth as ds

    for f in ("domino_trace_read_res", "domino_trace_read_rb"):
        getattr(lib, f).argtypes = [ctypes.c_void_p]
    results = {}
    for name in names:
        wl = ds.WORKLOADS[name]
        sh = wl.shape
        w, inp = ds.make_workload(name)
        mode = (dca.EXEC_PERSISTENT if persistent else dca.EXEC_AUTO) | (dca.EXEC_PLAIN_LAUNCH if plain_launch else 0)
        head = dca.DominoHead(dca.head_weights_to_device(w), K=sh.K, max_batch=wl.B, fold_embedding=fold,
                              exec_mode=mode, lbase_bf16=lbase_bf16)
        info = head.exec_info(wl.B)
        if not (info["persistent"] and info["w2_resident"]):
            raise SystemExit("%s does not take a resident persistent launch (%s)" % (name, info))
        batched = wl.B > 8
        H, lt = dca.device_tensor(inp.H), dca.device_tensor(inp.last_tok)
        L = dca.device_tensor(ds.round_to_bf16_bits(inp.L_base) if lbase_bf16 else inp.L_base)
        out = {"tokens": torch.empty((wl.B, sh.K), dtype=torch.int32, device="cuda")}
        for _ in range(3):
            head.draft(H, L, lt, out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        head.draft(H, L, lt, out=out)
        e1.record()
        torch.cuda.synchronize()
        assert head.check_error() == 0
        buf = np.zeros(BLOCKS * SLOTS, np.uint64)
        rc = (lib.domino_trace_read_rb if batched else lib.domino_trace_read_res)(buf.ctypes.data)
        assert rc == 0, rc
        t = buf.reshape(BLOCKS, SLOTS)[:min(info["grid"], BLOCKS)].astype(np.int64)
        r = {"workload": name + (" bf16 L_base" if lbase_bf16 else "") + ("" if fold else " unfolded"), "B": wl.B,
             "kernel": "k_persistent_rb" if batched else "k_persistent_res", "grid": info["grid"],
             "call_us": round(e0.elapsed_time(e1) * 1e3, 1)}
        # only blocks that compute state dots mark their rounds
        nd = 0
        if batched:
            nd = ((sh.r + 3 * sh.h) // 16 if wl.B <= 64 else
                  min(info["grid"], (sh.r + 3 * sh.h) // 64 * (((wl.B + 15) // 16 + 3) // 4)))
        r.update(summarize(t, sh.K, batched, unfolded=not fold))
        if batched:
            r["w2_groups"] = w2_groups(t, sh.K, (wl.B + 15) // 16)
        if nd:
            r["state_dots_detail"] = summarize(t[:nd], sh.K, batched, dots_detail=True)[
                "positions_1_to_%d_median" % (sh.K - 2)]
            r["state_dots_detail"] = {k: v for k, v in r["state_dots_detail"].items()
                                      if k.startswith("dots_")}
        results[name] = r
        del head
    return results


def to_markdown(r):
    lines = ["### %s (B=%d, %s, %d blocks): call %.1f us, kernel %.1f us" % (
        r["workload"], r["B"], r["kernel"], r["grid"], r["call_us"], r["kernel_us"]), "",
        "| section | phase | median over blocks (us) | slowest block (us) |", "|---|---|---|---|"]
    for sec, ph in r.items():
        if isinstance(ph, dict):
            for n, (m, x) in ph.items():
                lines.append("| %s | %s | %.2f | %.2f |" % (sec, n, m, x))
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--json", action="store_true")
    ap.add_argument("--persistent", action="store_true")
    ap.add_argument("--lbase-bf16", action="store_true")
    ap.add_argument("--no-fold", action="store_true")
    ap.add_argument("--plain-launch", action="store_true")
    args = ap.parse_args()
    res = run(args.workloads, persistent=args.persistent, lbase_bf16=args.lbase_bf16, fold=not args.no_fold,
              plain_launch=args.plain_launch)
    for r in res.values():
        print(json.dumps(r) if args.json else to_markdown(r) + "\n", flush=True)


if __name__ == "__main__":
    main()
