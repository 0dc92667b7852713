"""Benchmark of the MoE dispatch / combine hot path on one MI355X.

One step = ep_layout + ep_dispatch + ep_combine over one batch of the seeded
synthetic workload (default: the V3-shaped headline, T=8192 tokens, hidden
7168, top-8 of 256 experts over 8 simulated ranks, FP8 E4M3 dispatch with
per-128-channel fp32 scales, BF16 combine).  Inputs are resident in HBM before
the timed region; the expert stand-in (seeded bf16 rows in the receive
buffers) is outside the path and is not timed.

Prints ONE JSON line (rank 0, N=1):
  value        = algorithmic bytes of a step / wall time of a step  [GB/s]
  ms_per_step  = wall time over the K timed steps / K
  roofline     = the dominant kernel (combine): algorithmic bytes per launch /
                 its mean HIP-event duration, against 8 TB/s HBM peak
  cpu_baseline = the CPU oracle (single thread) on a bounded sample
  cache_flushed = layout / dispatch / combine medians with a 1 GiB read
                 before each step (cold caches), beside the back-to-back ones
  extras       = the other entry points timed in the same run (router, decode-
                 style steps, steps from the logits, shared-expert combine,
                 combine backward, SiLU re-quantization); --no-extras skips them
--summarize writes the profiles/ summaries from rocprofv3 CSV output.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
CAL_BYTES = 1 << 30  # size of the calibration kernels (elementwise copy, fill)
EXPERT_I = 2048      # expert intermediate size for the SiLU stage (DeepSeek-V3's)
METRIC = "dispatch+combine µs and achieved HBM GB/s at 8K tok, h7168, top-8, 1 GPU"


def algorithmic_bytes(T, H, k, E, R, fp8):
    """Bytes the method must move (reads of x / y / indices / weights, writes
    of rows / scales / output / handle), per call."""
    P = T * k
    nb = H // 128
    layout = 4 * P + 8 * P + 4 * (2 * E + 2 * R + 3)   # read idx, write slot/src, counts/offsets
    if fp8:
        dispatch = 2 * H * T + P * (H + 4 * nb) + 8 * P  # read x, write q + scales, read idx + slot
    else:
        dispatch = 2 * H * T + P * 2 * H + 8 * P
    combine = 2 * H * P + 2 * H * T + 12 * P           # read y, write out, read w + idx + slot
    return dict(layout=layout, dispatch=dispatch, combine=combine)


def extra_bytes(T, H, k):
    """Algorithmic bytes of the entry points outside the forward step."""
    P = T * k
    return {
        # combine plus reading the shared expert's [T,H] bf16 rows
        "combine_shared": 2 * H * P + 2 * H * T + 2 * H * T + 12 * P,
        # read grad_out, read y, write the gradient rows, read w/idx/slot, write grad_w
        "combine_backward": 2 * H * T + 2 * H * P + 2 * H * P + 12 * P + 4 * P,
        # per received row: read 2I bf16, write I codes and I/128 scales (I = 2048)
        "silu_mul_quant": P * (4 * EXPERT_I + EXPERT_I + 4 * (EXPERT_I // 128)),
    }


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def kernel_sources():
    c = os.path.join(ROOT, "combine_ep_layout_03_amd", "csrc")
    # the kernels' own file plus the headers whose constants and helpers they use
    common = [os.path.join(c, "ep_internal.h"), os.path.join(c, "ep_device.h"),
              os.path.join(ROOT, "include", "ep.h")]
    return {"combine": [os.path.join(c, "ep_combine.hip")] + common,
            "dispatch": [os.path.join(c, "ep_dispatch.hip")] + common}


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(kernel_sources()[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(workload_name, sample_tokens, min_seconds):
    """Time the CPU oracle (single thread) on the first `sample_tokens` tokens of
    the workload, repeated until min_seconds of work; GB/s of algorithmic
    bytes."""
    import numpy as np
    import oracle
    from workloads import make_workload, make_expert_rows

    w = make_workload(workload_name)
    Ts = min(sample_tokens, w.T)
    x, idx, wt = w.x[:Ts].copy(), w.topk_idx[:Ts].copy(), w.topk_w[:Ts].copy()
    L0 = oracle.layout(idx, w.E, w.R)
    y = make_expert_rows(Ts * w.k, w.H)
    ys = [y[L0.rank_offsets[r]:L0.rank_offsets[r + 1]] for r in range(w.R)]
    oracle.lib()
    times = []
    t_end = time.perf_counter() + min_seconds
    while len(times) < 2 or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        L = oracle.layout(idx, w.E, w.R)
        if w.fp8:
            oracle.dispatch_fp8(x, idx, L)
        else:
            oracle.dispatch_bf16(x, idx, L)
        oracle.combine(ys, idx, L, wt)
        times.append(time.perf_counter() - t0)
    b = algorithmic_bytes(Ts, w.H, w.k, w.E, w.R, w.fp8)
    step_bytes = sum(b.values())
    mean = statistics.mean(times)
    return {"value": round(step_bytes / mean / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{workload_name} workload, first {Ts} of {w.T} tokens (layout + dispatch + "
                      f"combine), {len(times)} repetitions, mean {mean:.3f} s each, single thread "
                      f"of {os.cpu_count()} host cores"}


# rocprofv3 kernel names ("ep::(anonymous namespace)::combine_kernel<false>(int const*, ...")
# matched by anchored patterns: combine_kernel<false> is ep_combine, <true> ep_combine_shared;
# route_rows_kernel<N, true> is the router that also counts the layout's chunk table
KERNEL_KEYS = {
    "combine": r"::combine_kernel(<false>)?\(",
    "dispatch": r"::dispatch_(fp8|bf16)_kernel\(",
    "layout_count": r"::layout_count_kernel\(",
    "layout_scatter": r"::layout_scatter_kernel\(",
    "layout_small": r"::layout_small_kernel\(",
    "layout_tiny": r"::layout_tiny_kernel\(",
    "route": r"::(route_kernel<\d+>|route_rows_kernel<\d+, false>)\(",
    "route_count": r"::route_rows_kernel<\d+, true>\(",
    "layout_dispatch_small": r"::layout_dispatch_small_kernel<(true|false)>\(",
    "combine_shared": r"::combine_kernel<true>\(",
    "combine_backward": r"::combine_backward_(wave|wg)_kernel\(",
    "silu_mul_quant": r"::silu_mul_quant_kernel\(",
}
CAL_COPY_KEY = "bitwise_not"      # elementwise kernel: reads and writes CAL_BYTES
CAL_FILL_KEY = "FillFunctor<unsigned char>"  # writes CAL_BYTES


def summarize(trace_dir, fetch_dir, write_dir, workload, command_prefix):
    """Write the profiles/ summaries from rocprofv3 CSV output: per-kernel
    durations (--kernel-trace --stats) and HBM bytes per launch (two --pmc
    passes, FETCH_SIZE and WRITE_SIZE, in KiB, each scaled by what the same
    counter reads for a calibration kernel of known size)."""
    import csv
    import glob

    def one(d, suffix):
        f = glob.glob(os.path.join(d, "*" + suffix))
        assert len(f) == 1, (d, suffix, f)
        return list(csv.DictReader(open(f[0])))

    stats = one(trace_dir, "_kernel_stats.csv")
    fetch = one(fetch_dir, "_counter_collection.csv")
    write = one(write_dir, "_counter_collection.csv")

    def per_kernel(rows, key, regex=True):
        hit = (lambda n: re.search(key, n)) if regex else (lambda n: key in n)
        v = [float(r["Counter_Value"]) for r in rows if hit(r["Kernel_Name"])]
        return statistics.median(v) if v else None

    fetch_cal = per_kernel(fetch, CAL_COPY_KEY, False)  # KiB read by a CAL_BYTES-read kernel
    write_cal = per_kernel(write, CAL_FILL_KEY, False)  # KiB written by a CAL_BYTES-write kernel
    f_fetch = CAL_BYTES / fetch_cal
    f_write = CAL_BYTES / write_cal
    cmd_trace = f"{command_prefix} rocprofv3 --kernel-trace --stats -f csv -d {trace_dir} -o {workload} -- python3 bench.py --config {workload} --steps 20 --warmup 3 --skip-cpu"
    lines = [f"# Kernel durations and HBM traffic, {workload} workload", "",
             "Kernel-trace command (run from the repository root):", "", "```", cmd_trace, "```", "",
             "Counter commands (one pass each):", "", "```",
             f"{command_prefix} rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o {workload} -- python3 bench.py --config {workload} --steps 3 --warmup 1 --skip-cpu",
             f"{command_prefix} rocprofv3 --pmc WRITE_SIZE -f csv -d {write_dir} -o {workload} -- python3 bench.py --config {workload} --steps 3 --warmup 1 --skip-cpu",
             "```", "",
             f"Counter calibration: FETCH_SIZE of the elementwise copy kernel ({CAL_BYTES} B read) = "
             f"{fetch_cal:.0f} KiB, so FETCH bytes = FETCH_SIZE x {f_fetch:.4f}; WRITE_SIZE of the fill "
             f"kernel ({CAL_BYTES} B written) = {write_cal:.0f} KiB, so WRITE bytes = WRITE_SIZE x {f_write:.4f}.", "",
             "| kernel | calls | avg us | min us | max us | HBM read MB/launch | HBM write MB/launch |",
             "|---|---|---|---|---|---|---|"]
    traffic = {}
    for short, key in KERNEL_KEYS.items():
        st = [r for r in stats if re.search(key, r["Name"])]
        assert len(st) <= 1, (short, [r["Name"][:80] for r in st])
        if not st:
            continue
        r = st[0]
        fr, wr = per_kernel(fetch, key), per_kernel(write, key)
        rb = fr * f_fetch if fr is not None else None
        wb = wr * f_write if wr is not None else None
        traffic[short] = (rb, wb)
        lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | {float(r['MinNs'])/1e3:.2f} | "
                     f"{float(r['MaxNs'])/1e3:.2f} | {rb/1e6 if rb else float('nan'):.1f} | {wb/1e6 if wb else float('nan'):.1f} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    md = os.path.join(ROOT, "profiles", f"kernels_{workload}.md")
    open(md, "w").write("\n".join(lines) + "\n")
    for kernel in ("combine", "dispatch"):
        if kernel in traffic and traffic[kernel][0] is not None:
            rec = {"kernel": kernel, "workload": workload,
                   "source_sha": source_sha(kernel_sources()[kernel]),
                   "hbm_read_bytes_per_launch": round(traffic[kernel][0]),
                   "hbm_write_bytes_per_launch": round(traffic[kernel][1]),
                   "hbm_bytes_per_launch": round(traffic[kernel][0] + traffic[kernel][1]),
                   "fetch_scale": f_fetch, "write_scale": f_write, "summary": os.path.basename(md)}
            json.dump(rec, open(os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json"), "w"),
                      indent=1)
    print(open(md).read())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="v3")
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU-oracle baseline")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--num-workgroups", type=int, default=0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip timing the other entry points (router, decode-style, backward, expert-side)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 CSV directories and exit")
    ap.add_argument("--command-prefix", default="", help="recorded in the summary (e.g. env settings)")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize, args.config, args.command_prefix)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the expert-parallel ranks are simulated as "
              "destination buffers in one HBM, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from combine_ep_layout_03_amd import build as epbuild
    if not os.path.exists(epbuild.LIB):
        epbuild.build()
    import combine_ep_layout_03_amd as ep
    from combine_ep_layout_03_amd import _lib
    from combine_ep_layout_03_amd.buffers import Handle, RecvBuffers, alloc_workspace
    from workloads import CONFIGS, make_workload

    L = ep.load()
    dev = "cuda"
    w = make_workload(args.config)
    cfg = ep.Config(w.T, w.H, w.k, w.E, w.R, fp8=w.fp8, num_workgroups=args.num_workgroups)
    cap = ep.ep_recv_capacity_rows(cfg)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
    idx, x, wts = up(w.topk_idx), up(w.x), up(w.topk_w)
    h = Handle.alloc(cfg, dev)
    ws = alloc_workspace(cfg, dev)
    recv = RecvBuffers.alloc(cfg, cap, device=dev)
    out = torch.empty((w.T, w.H), dtype=torch.int16, device=dev)

    # layout once to size the expert stand-in rows: seeded N(0,1) bf16 rows in
    # the valid part of each rank buffer
    ep.ep_layout(cfg, idx, h, ws)
    torch.cuda.synchronize()
    rank_counts = h.rank_counts.cpu().tolist()
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    ybufs = []
    for r in range(w.R):
        b = torch.zeros((cap, w.H), dtype=torch.int16, device=dev)
        n = rank_counts[r]
        if n:
            b[:n] = torch.randn((n, w.H), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
        ybufs.append(b)
    torch.cuda.synchronize()

    # prebuilt C arguments for the timed loop (no per-call marshalling)
    ccfg = cfg.c()
    ch = _lib.ep_layout_t(*[getattr(h, n).data_ptr() for n, _ in _lib.ep_layout_t._fields_])
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    rx = (ctypes.c_void_p * w.R)(*[t.data_ptr() for t in recv.x])
    rs = (ctypes.c_void_p * w.R)(*[t.data_ptr() for t in recv.scales]) if recv.scales else None
    ry = (ctypes.c_void_p * w.R)(*[t.data_ptr() for t in ybufs])
    pc, ph = ctypes.byref(ccfg), ctypes.byref(ch)

    def layout():
        st = L.ep_layout(pc, idx.data_ptr(), ph, ws.data_ptr(), sp)
        assert st == 0, st

    def dispatch():
        st = L.ep_dispatch(pc, ph, idx.data_ptr(), x.data_ptr(), rx, rs, cap, sp)
        assert st == 0, st

    def combine():
        st = L.ep_combine(pc, ph, idx.data_ptr(), ry, wts.data_ptr(), out.data_ptr(), cap, sp)
        assert st == 0, st

    # Plain streaming kernels of known size, same run: an elementwise pass that
    # reads 1 GiB and writes 1 GiB (the copy ceiling) and a 1 GiB fill (the
    # write ceiling).  They are also the calibration kernels for the HBM byte
    # counters (see --summarize).
    src = torch.empty(CAL_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=5):
        ms = []
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return statistics.median(ms)

    fill_ms = timed(lambda: src.fill_(1))
    copy_ms = timed(lambda: torch.bitwise_not(src, out=dst))
    copy_gbps = 2 * CAL_BYTES / (copy_ms * 1e-3) / 1e9
    write_gbps = CAL_BYTES / (fill_ms * 1e-3) / 1e9
    del src, dst

    for _ in range(args.warmup):
        layout(); dispatch(); combine()
    torch.cuda.synchronize()
    assert int(h.error_flag.item()) == 0

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        layout()
        e[1].record(stream)
        dispatch()
        e[2].record(stream)
        combine()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(h.error_flag.item()) == 0

    lay = [e[0].elapsed_time(e[1]) * 1e3 for e in ev]
    dis = [e[1].elapsed_time(e[2]) * 1e3 for e in ev]
    com = [e[2].elapsed_time(e[3]) * 1e3 for e in ev]
    dc = [a + b for a, b in zip(dis, com)]
    b = algorithmic_bytes(w.T, w.H, w.k, w.E, w.R, w.fp8)
    step_bytes = sum(b.values())
    ms_per_step = wall / K * 1e3
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    mean_com = statistics.mean(com)
    achieved = b["combine"] / (mean_com * 1e-6) / 1e9

    def pct(v, q):
        s = sorted(v)
        return round(s[min(len(s) - 1, int(q * len(s)))], 2)

    # The same three calls with cold caches: before each step a 1 GiB read
    # (4x the 256 MB MALL, 32x the L2; a read, so it leaves no dirty lines
    # whose write-back would land in the timed kernels) runs outside the
    # kernel events.  The timed loop above is back-to-back steps, as in a
    # layer loop that reuses its buffers.
    flush_buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(min(K, 20))]
    for e in fev:
        flush_buf.view(torch.int64).sum()
        e[0].record(stream)
        layout()
        e[1].record(stream)
        dispatch()
        e[2].record(stream)
        combine()
        e[3].record(stream)
    torch.cuda.synchronize()
    del flush_buf
    assert int(h.error_flag.item()) == 0
    flushed = {name: round(statistics.median(e[a].elapsed_time(e[a + 1]) * 1e3 for e in fev), 2)
               for a, name in enumerate(("layout_us", "dispatch_us", "combine_us"))}

    extras = None
    if not args.no_extras:
        # the other entry points on the same handle and buffers: combine with a
        # shared-expert row, and the backward of combine (gradient rows + grad_w)
        gen.manual_seed(2)
        shared = torch.randn((w.T, w.H), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
        gout = torch.randn((w.T, w.H), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
        grows = [torch.empty((cap, w.H), dtype=torch.int16, device=dev) for _ in range(w.R)]
        gwt = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
        rgp = (ctypes.c_void_p * w.R)(*[t.data_ptr() for t in grows])
        xb = extra_bytes(w.T, w.H, w.k)
        # expert GEMM-1 outputs (gate | up, 2*EXPERT_I bf16) in the receive
        # layout: capacity-sized buffers, seeded rows in the valid part
        act, aq, asc = [], [], []
        for r in range(w.R):
            a = torch.zeros((cap, 2 * EXPERT_I), dtype=torch.int16, device=dev)
            if rank_counts[r]:
                a[:rank_counts[r]] = torch.randn((rank_counts[r], 2 * EXPERT_I), generator=gen,
                                                 device=dev).to(torch.bfloat16).view(torch.int16)
            act.append(a)
            aq.append(torch.empty((cap, EXPERT_I), dtype=torch.uint8, device=dev))
            asc.append(torch.empty((cap, EXPERT_I // 128), dtype=torch.float32, device=dev))
        pa = (ctypes.c_void_p * w.R)(*[t.data_ptr() for t in act])
        pq = (ctypes.c_void_p * w.R)(*[t.data_ptr() for t in aq])
        ps = (ctypes.c_void_p * w.R)(*[t.data_ptr() for t in asc])
        calls = {
            "silu_mul_quant": lambda: L.ep_silu_mul_quant(pc, ph, EXPERT_I, pa, pq, ps, cap, sp),
            "combine_shared": lambda: L.ep_combine_shared(pc, ph, idx.data_ptr(), ry, wts.data_ptr(),
                                                          shared.data_ptr(), out.data_ptr(), cap, sp),
            "combine_backward": lambda: L.ep_combine_backward(pc, ph, idx.data_ptr(), gout.data_ptr(),
                                                              wts.data_ptr(), ry, rgp, gwt.data_ptr(),
                                                              cap, sp),
        }
        extras = {}
        for name, fn in calls.items():
            for _ in range(3):
                assert fn() == 0
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(min(K, 20))]
            for a, b_ in evs:
                a.record(stream)
                assert fn() == 0
                b_.record(stream)
            torch.cuda.synchronize()
            us = statistics.median(a.elapsed_time(b_) * 1e3 for a, b_ in evs)
            extras[name] = {"us": round(us, 2), "algorithmic_bytes": xb[name],
                            "GBps": round(xb[name] / (us * 1e-6) / 1e9, 1)}
        assert int(h.error_flag.item()) == 0
        del shared, gout, grows, gwt, act, aq, asc

        # the router on this workload's logits, into buffers of its own: alone,
        # feeding the layout, and the whole step from logits (route + layout +
        # dispatch + combine)
        rin = w.extra
        El = rin["logits"].shape[1]
        logits_d = up(rin["logits"])
        opt = lambda key: up(rin[key]) if key in rin else None
        bias_d, ro_d, rsl_d = opt("bias"), opt("rep_offsets"), opt("rep_slots")
        dp = lambda t: None if t is None else t.data_ptr()
        crt = ep.Router(El, **rin["router"]).c()
        prt = ctypes.byref(crt)
        idx2, w2 = torch.empty_like(idx), torch.empty_like(wts)
        h2 = Handle.alloc(cfg, dev)
        ws2 = alloc_workspace(cfg, dev)
        ch2 = _lib.ep_layout_t(*[getattr(h2, n).data_ptr() for n, _ in _lib.ep_layout_t._fields_])
        ph2 = ctypes.byref(ch2)
        rt_args = (pc, prt, logits_d.data_ptr(), dp(bias_d), dp(ro_d), dp(rsl_d), idx2.data_ptr(),
                   w2.data_ptr())
        rcall = lambda: L.ep_route(*rt_args, sp)
        rlcall = lambda: L.ep_route_layout(*rt_args, ph2, ws2.data_ptr(), sp)
        route_bytes = (w.T * El * 4 + w.T * w.k * 8 + (El * 4 if bias_d is not None else 0)
                       + (w.T * w.k * 8 if ro_d is not None else 0))
        for name, fn, nbytes in (("route", rcall, route_bytes),
                                 ("route_layout", rlcall, route_bytes + algorithmic_bytes(
                                     w.T, w.H, w.k, w.E, w.R, w.fp8)["layout"])):
            for _ in range(3):
                assert fn() == 0
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(min(K, 20))]
            for a, b_ in evs:
                a.record(stream)
                assert fn() == 0
                b_.record(stream)
            torch.cuda.synchronize()
            us = statistics.median(a.elapsed_time(b_) * 1e3 for a, b_ in evs)
            extras[name] = {"us": round(us, 2), "algorithmic_bytes": nbytes,
                            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        assert int(h2.error_flag.item()) == 0
        assert torch.equal(idx2, idx) and torch.equal(h2.slot_of, h.slot_of)

        # decode-style steps: the one-call layout + dispatch, and the cached-
        # handle step (gating unchanged: dispatch + combine, no layout)
        def step_time(fns):
            for _ in range(3):
                for fn in fns:
                    assert fn() == 0
            torch.cuda.synchronize()
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = max(K, 20)
            a.record(stream)
            for _ in range(n):
                for fn in fns:
                    assert fn() == 0
            b_.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b_) * 1e3 / n

        ld = lambda: L.ep_layout_dispatch(pc, idx.data_ptr(), ph, ws.data_ptr(), x.data_ptr(), rx, rs,
                                          cap, sp)
        cd = lambda: L.ep_dispatch(pc, ph, idx.data_ptr(), x.data_ptr(), rx, rs, cap, sp)
        cc = lambda: L.ep_combine(pc, ph, idx.data_ptr(), ry, wts.data_ptr(), out.data_ptr(), cap, sp)
        extras["layout_dispatch_us"] = round(step_time([ld]), 2)
        extras["fused_step_us"] = round(step_time([ld, cc]), 2)
        extras["cached_handle_step_us"] = round(step_time([cd, cc]), 2)
        rd = lambda: L.ep_dispatch(pc, ph2, idx2.data_ptr(), x.data_ptr(), rx, rs, cap, sp)
        rc = lambda: L.ep_combine(pc, ph2, idx2.data_ptr(), ry, w2.data_ptr(), out.data_ptr(), cap, sp)
        extras["routed_step_us"] = round(step_time([rlcall, rd, rc]), 2)
        # from the logits through the one-call layout + dispatch (one launch
        # at decode sizes): route, layout_dispatch, combine
        rld = lambda: L.ep_layout_dispatch(pc, idx2.data_ptr(), ph2, ws2.data_ptr(), x.data_ptr(), rx,
                                           rs, cap, sp)
        extras["routed_fused_step_us"] = round(step_time([rcall, rld, rc]), 2)
        assert int(h2.error_flag.item()) == 0
        assert int(h.error_flag.item()) == 0

    graph_us = None
    fused_graph_us = None
    if args.graph:
        # one step (layout + dispatch + combine) captured once, replayed K times
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        gsp = gs.cuda_stream
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g, stream=gs):
                assert L.ep_layout(pc, idx.data_ptr(), ph, ws.data_ptr(), gsp) == 0
                assert L.ep_dispatch(pc, ph, idx.data_ptr(), x.data_ptr(), rx, rs, cap, gsp) == 0
                assert L.ep_combine(pc, ph, idx.data_ptr(), ry, wts.data_ptr(), out.data_ptr(), cap, gsp) == 0
        stream.wait_stream(gs)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record()
        for _ in range(K):
            g.replay()
        gb.record()
        torch.cuda.synchronize()
        graph_us = ga.elapsed_time(gb) * 1e3 / K
        assert int(h.error_flag.item()) == 0
        # the fused step (ep_layout_dispatch + ep_combine) as a graph
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g2, stream=gs):
                assert L.ep_layout_dispatch(pc, idx.data_ptr(), ph, ws.data_ptr(), x.data_ptr(), rx,
                                            rs, cap, gsp) == 0
                assert L.ep_combine(pc, ph, idx.data_ptr(), ry, wts.data_ptr(), out.data_ptr(), cap,
                                    gsp) == 0
        stream.wait_stream(gs)
        for _ in range(args.warmup):
            g2.replay()
        torch.cuda.synchronize()
        ga.record()
        for _ in range(K):
            g2.replay()
        gb.record()
        torch.cuda.synchronize()
        fused_graph_us = ga.elapsed_time(gb) * 1e3 / K
        assert int(h.error_flag.item()) == 0

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: x ~ N(0,1) bf16, router logits N(0,1); expert outputs N(0,1) bf16)",
        "config": {"workload": args.config, "T": w.T, "hidden": w.H, "top_k": w.k,
                   "experts": w.E, "ranks": w.R,
                   "dispatch": "fp8_e4m3 + fp32 per-128 scales" if w.fp8 else "bf16",
                   "combine": "bf16 (fp32 accumulate)", "parallelism": "1 GPU, ranks simulated"},
        "roofline": {"bound": "hbm", "kernel": "combine", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": load_traffic("combine", args.config),
                     "algorithmic_bytes_per_launch": b["combine"], "mean_launch_us": round(mean_com, 2)},
        "layout_us": round(statistics.median(lay), 2),
        "dispatch_us": round(statistics.median(dis), 2),
        "combine_us": round(statistics.median(com), 2),
        "dc_us": round(statistics.median(dc), 2),
        "dc_us_p10_p90": [pct(dc, 0.1), pct(dc, 0.9)],
        "dc_GBps": round((b["dispatch"] + b["combine"]) / (statistics.median(dc) * 1e-6) / 1e9, 1),
        "dispatch_GBps": round(b["dispatch"] / (statistics.median(dis) * 1e-6) / 1e9, 1),
        "combine_GBps": round(b["combine"] / (statistics.median(com) * 1e-6) / 1e9, 1),
        "cache_flushed": flushed,
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "write_ceiling_GBps": round(write_gbps, 1),
        "bytes_per_step": step_bytes,
        "graph_step_us": None if graph_us is None else round(graph_us, 2),
        "fused_graph_step_us": None if fused_graph_us is None else round(fused_graph_us, 2),
        "extras": extras,
        "cpu_baseline": None,
    }
    if not args.skip_cpu:
        res["cpu_baseline"] = cpu_baseline(args.config, args.cpu_sample_tokens, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
