"""Benchmark of the Flash PD-SSM forward scan on one MI355X.

One step = one pdssm_scan_fwd call over the whole batch (selection, P D
recurrence, in-chunk composition, chunk carry, fused readout), inputs already
resident in HBM.  The default workload is the LM-layer shape: B=8 H=32
L=4096 N=64 K=64, bf16 router logits, complex64 diagonal, bf16 b/c/y,
complex64 x_final.  Inputs are seeded synthetic data of that shape.

Prints one JSON line with throughput (scanned tokens/s = B*H*L per second),
the roofline of the scan kernel (algorithmic HBM bytes per call over the
measured call time, against 8 TB/s), and the fp64 CPU oracle timed on the
host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scanned tokens/sec (B·H·L) and achieved HBM GB/s vs peak, N=64 L=4096"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
ROUTER_D = 2048                  # router input features per token
MALL_BYTES = 256 << 20           # MI355X last-level cache (Infinity Cache)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "scan_kernel_lm_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "structured_sparse_state_amd", "csrc", f)
                  for f in ("pdssm_scan.hip", "pdssm_device.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(inp, y, xf) -> int:
    """Every input read once and every output written once."""
    n = 0
    for t in (inp.sel_or_logits, inp.dict_idx, inp.diag, inp.b, inp.c, inp.x0, y, xf):
        if t is not None:
            n += t.numel() * t.element_size()
    return n


def counter_traffic(bytes_per_call: int, workload: str):
    """HBM bytes per call from the committed rocprofv3 counter summary (taken
    on the LM workload), or None for another workload or when the kernel
    sources changed since the counters were taken."""
    if workload != "lm" or not os.path.exists(COUNTERS_FILE):
        return None
    vals = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def measure_backward(pk, gen, inp, ws, stream, args):
    """Time pdssm_scan_bwd (and the forward that saves chunk carries) on the
    same inputs, HIP events on the launch stream; returns the summary object
    reported beside the forward's."""
    import torch
    gy, gxf = gen.make_grads(inp, seed=1)
    bws = pk.bwd_workspace_for(inp)
    _, _, xch, sel = pk.scan_save(inp, workspace=ws, stream=stream, want_sel=True)
    out = pk.scan_bwd(inp, xch, gy, gxf, workspace=bws, stream=stream, sel=sel)
    steps = max(10, args.steps // 4)

    def timed(fn):
        for _ in range(max(3, args.warmup // 4)):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e-3

    t_bwd = timed(lambda: pk.scan_bwd(inp, xch, gy, gxf, workspace=bws, stream=stream, out=out,
                                      sel=sel))
    t_bwd_det = timed(lambda: pk.scan_bwd(inp, xch, gy, gxf, workspace=bws, stream=stream, out=out,
                                          sel=sel, deterministic=True))
    t_save = timed(lambda: pk.scan_save(inp, workspace=ws, stream=stream, want_sel=True))
    ins = (sel, inp.dict_idx, inp.diag, inp.b, inp.c, inp.x0, xch, gy, gxf)
    alg = sum(t.numel() * t.element_size() for t in ins + tuple(out) if t is not None)
    tokens = inp.B * inp.H * inp.L
    print(f"[bench] backward: {t_bwd * 1e6:.1f} us/call, {alg / t_bwd / 1e9:.0f} GB/s algorithmic; "
          f"forward with saved carries {t_save * 1e6:.1f} us", file=sys.stderr, flush=True)
    return {"us_per_call": t_bwd * 1e6, "tokens_per_s": tokens / t_bwd,
            "algorithmic_bytes_per_call": alg, "achieved_GBps": alg / t_bwd / 1e9,
            "frac": alg / t_bwd / 1e9 / HBM_PEAK_GBS, "steps": steps,
            "fwd_save_us_per_call": t_save * 1e6,
            "deterministic_us_per_call": t_bwd_det * 1e6,
            "note": "pdssm_scan_bwd: gradients of b, c, diag, x0 from dy and dx_final, fed "
                    "with the forward's saved chunk carries and int16 selections; algorithmic "
                    "bytes = every input read once and every gradient written once"}


def _event_time(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e-3


def measure_hbm_practical(nbytes: int, stream):
    """What plain streaming kernels reach on this GPU over the same number of
    bytes (context for the roofline fraction, whose peak stays 8 TB/s):
    torch's row sums (read only) and an elementwise add (read + write)."""
    import torch
    n = (nbytes // 4) // 1024 * 1024
    x = torch.randn(n, device="cuda:0")
    y = torch.empty_like(x)
    rows = x.view(-1, 1024)
    t_read = _event_time(lambda: rows.sum(dim=1), 20, 3, stream)
    t_rw = _event_time(lambda: torch.add(x, 1.0, out=y), 20, 3, stream)
    del x, y, rows
    torch.cuda.empty_cache()
    return {"read_GBps": n * 4 / t_read / 1e9, "read_write_GBps": 2 * n * 4 / t_rw / 1e9,
            "bytes": n * 4,
            "note": "torch row sums (read) and elementwise add (read+write) over the same bytes "
                    "as one scan call; the practical streaming rate on this GPU, for context"}


def measure_aux(pk, gen, inp, stream, workload):
    """The dictionary pre-compute and one decode step at the workload's
    shape, HIP events on the launch stream."""
    import torch
    B, H, N, K = inp.B, inp.H, inp.N, inp.K
    dev = inp.diag.device
    m = gen.make_dense_dict(H, K, N, device=dev)
    dct = pk.dict_hardmax(m, stream=stream)
    t_hm = _event_time(lambda: pk.dict_hardmax(m, stream=stream, out=dct), 50, 5, stream)
    hm_bytes = m.numel() * m.element_size() + dct.numel() * dct.element_size()

    # Copies (clone), not views: with B = H = 1 a step's slice is already
    # contiguous, and its address would be that of the step inside the
    # sequence, which the library's 16-byte alignment rule rejects.
    if inp.sel_mode.startswith("sel"):
        sel = inp.sel_or_logits[:, :, 0].clone()
    else:
        sel = inp.sel_or_logits[:, :, 0, :].clone()
    d, b, c = (t[:, :, 0].clone() for t in (inp.diag, inp.b, inp.c))
    x = torch.zeros((B, H, N, 2) if inp.complex else (B, H, N), device=dev, dtype=torch.float32)
    y = torch.empty((B, H), device=dev, dtype=torch.bfloat16 if inp.y_bf16 else torch.float32)

    def dec():
        pk.decode_step(sel, inp.dict_idx, d, b, c, x, sel_mode=inp.sel_mode, complex=inp.complex,
                       bc_bf16=inp.bc_bf16, y_bf16=inp.y_bf16, y=y, stream=stream)

    t_dec = _event_time(dec, 200, 20, stream)

    # The same step as a decoding window: 64 consecutive steps captured in
    # one HIP graph (the state stays in place, every step's inputs at fixed
    # addresses), so the window costs one launch instead of 64.
    T_win = min(64, inp.L)
    win = []
    for t in range(T_win):
        ws_ = (inp.sel_or_logits[:, :, t].clone() if inp.sel_mode.startswith("sel")
               else inp.sel_or_logits[:, :, t, :].clone())
        win.append((ws_, inp.diag[:, :, t].clone(), inp.b[:, :, t].clone(),
                    inp.c[:, :, t].clone(), torch.empty_like(y)))
    xw = x.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def window():
        for (s_, d_, b_, c_, y_) in win:
            pk.decode_step(s_, inp.dict_idx, d_, b_, c_, xw, sel_mode=inp.sel_mode, complex=inp.complex,
                           bc_bf16=inp.bc_bf16, y_bf16=inp.y_bf16, y=y_)

    with torch.cuda.stream(side):
        window()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        window()
    t_win = _event_time(lambda: graph.replay(), 50, 5, stream)
    del graph, win, xw
    # A window of known steps can also run as one scan call of L = 64 that
    # starts from the carried state (x0) and hands its state on (x_final):
    # the steps then overlap inside the kernel instead of following each
    # other's memory latencies.
    wl_inp = gen.make_inputs(workload, device=dev, L=T_win, with_x0=True)
    wl_ws = pk.workspace_for(wl_inp)
    wl_y = torch.empty((B, H, T_win), device=dev, dtype=torch.bfloat16 if inp.y_bf16 else torch.float32)
    wl_xf = torch.empty_like(wl_inp.x0)
    t_swin = _event_time(lambda: pk.scan(wl_inp, workspace=wl_ws, y=wl_y, x_final=wl_xf, stream=stream),
                         50, 5, stream)
    del wl_inp, wl_ws, wl_y, wl_xf

    # Router scores + argmax from the step inputs (D = 2048 features per
    # token), only the int16 selections written; the fused kernel takes up
    # to 128 scores per head (heads padded to 64 or 128 score columns).
    D = ROUTER_D
    if K > 128:
        dec_bytes = sum(t.numel() * t.element_size() for t in (sel, d, b, c, y)) + 2 * x.numel() * 4
        print(f"[bench] dict hardmax {t_hm * 1e6:.1f} us ({hm_bytes / t_hm / 1e9:.0f} GB/s); decode step "
              f"{t_dec * 1e6:.2f} us ({B * H / t_dec:.3g} tokens/s); router: K={K} > 128, not run",
              file=sys.stderr, flush=True)
        return {
            "dict_hardmax": {"us_per_call": t_hm * 1e6, "shape": f"H={H} K={K} N={N} fp32",
                             "algorithmic_bytes_per_call": hm_bytes,
                             "achieved_GBps": hm_bytes / t_hm / 1e9,
                             "frac": hm_bytes / t_hm / 1e9 / HBM_PEAK_GBS},
            "decode_step": {"us_per_call": t_dec * 1e6, "tokens_per_s": B * H / t_dec,
                            "shape": f"B={B} H={H} N={N} K={K}, one step per sequence",
                            "algorithmic_bytes_per_call": dec_bytes},
            "router_select": None,
        }
    ru, rw = gen.make_router_inputs(B, inp.L, H, K, D, seed=4, device=dev)
    rwp = pk.router_pack_weights(rw, stream=stream)
    rsel = pk.router_select(ru, rwp, stream=stream)
    # The matrix cores reach their sustained clock only after a while of
    # load: warm up for about a second before timing.
    t_end = time.perf_counter() + 1.0
    while time.perf_counter() < t_end:
        for _ in range(10):
            pk.router_select(ru, rwp, out=rsel, stream=stream)
        torch.cuda.synchronize()
    # Packed weights (the layout of router_pack_weights, packed once per
    # weight update) and the [H,K,D] layout as given; the packing itself.
    t_rt = _event_time(lambda: pk.router_select(ru, rwp, out=rsel, stream=stream), 50, 3, stream)
    t_rt_plain = _event_time(lambda: pk.router_select(ru, rw, out=rsel, stream=stream), 50, 3, stream)
    t_pack = _event_time(lambda: pk.router_pack_weights(rw, stream=stream), 20, 3, stream)
    rt_flops = 2.0 * B * inp.L * H * K * D
    rt_pad_flops = 2.0 * B * inp.L * H * (64 if K <= 64 else 128) * D
    del ru, rw, rwp, rsel
    dec_bytes = sum(t.numel() * t.element_size() for t in (sel, d, b, c, y)) + 2 * x.numel() * 4
    print(f"[bench] dict hardmax {t_hm * 1e6:.1f} us ({hm_bytes / t_hm / 1e9:.0f} GB/s); decode step "
          f"{t_dec * 1e6:.2f} us ({B * H / t_dec:.3g} tokens/s), in a {T_win}-step graph "
          f"{t_win / T_win * 1e6:.2f} us per step, as one scan call {t_swin / T_win * 1e6:.2f} us per step; "
          f"router D={D} {t_rt * 1e6:.1f} us ({rt_flops / t_rt / 1e12:.0f} TFLOP/s), "
          f"weights as [H,K,D] {t_rt_plain * 1e6:.1f} us, packing {t_pack * 1e6:.1f} us",
          file=sys.stderr, flush=True)
    return {
        "dict_hardmax": {"us_per_call": t_hm * 1e6, "shape": f"H={H} K={K} N={N} fp32",
                         "algorithmic_bytes_per_call": hm_bytes,
                         "achieved_GBps": hm_bytes / t_hm / 1e9,
                         "frac": hm_bytes / t_hm / 1e9 / HBM_PEAK_GBS},
        "decode_step": {"us_per_call": t_dec * 1e6, "tokens_per_s": B * H / t_dec,
                        "shape": f"B={B} H={H} N={N} K={K}, one step per sequence",
                        "algorithmic_bytes_per_call": dec_bytes,
                        "note": "launch- and latency-bound: one step reads and writes "
                                f"{dec_bytes} bytes",
                        "graph_window": {"steps": T_win, "us_per_step": t_win / T_win * 1e6,
                                         "tokens_per_s": B * H * T_win / t_win,
                                         "note": "the same step, a window of consecutive steps "
                                                 "captured in one HIP graph and replayed"},
                        "scan_window": {"steps": T_win, "us_per_step": t_swin / T_win * 1e6,
                                        "tokens_per_s": B * H * T_win / t_swin,
                                        "note": "the window as one pdssm_scan_fwd call from the carried "
                                                "state (x0) to the handed-on state (x_final)"}},
        "router_select": {"us_per_call": t_rt * 1e6, "tokens_per_s": B * inp.L * H / t_rt,
                          "shape": f"B={B} L={inp.L} H={H} K={K} D={D}, bf16 inputs, fp32 sums",
                          "weights": "packed (pdssm_router_pack_weights, once per weight update)",
                          "us_per_call_weights_hkd": t_rt_plain * 1e6,
                          "us_per_pack": t_pack * 1e6,
                          "roofline": {"bound": "mfma", "achieved": rt_flops / t_rt / 1e12,
                                       "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": rt_flops / t_rt / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                                       "flops_per_call": rt_flops,
                                       "issued_flops_per_call": rt_pad_flops}},
    }


def cpu_threads() -> int:
    """Every core this process may run on."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, n)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="lm", choices=["lm", "long", "verylong", "small", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (known bytes) so that "
                         "rocprofv3 byte counters can be scaled")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the timings reported beside the forward (backward scan, dictionary "
                         "pre-compute, decode step, router, practical HBM rates)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets cycled through by the timed calls (0: enough sets to be "
                         "twice the 256 MB last-level cache, at most 8)")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle over the batch for at least this long")
    ap.add_argument("--settle-seconds", type=float, default=1.5,
                    help="untimed scan calls for this long before the warm-up calls, so the GPU "
                         "reaches its sustained clock whatever the warm-up count")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the scan is measured on a single MI355X.", file=sys.stderr)
        return 2

    import torch
    import structured_sparse_state_amd as pk
    from structured_sparse_state_amd import inputs as gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    inp = gen.make_inputs(args.workload, device=dev)
    B, H, L, N, K = inp.B, inp.H, inp.L, inp.N, inp.K
    y = torch.empty((B, H, L), device=dev, dtype=torch.bfloat16 if inp.y_bf16 else torch.float32)
    xf = torch.empty((B, H, N, 2) if inp.complex else (B, H, N), device=dev, dtype=torch.float32)
    ws = pk.workspace_for(inp)
    stream = torch.cuda.current_stream()
    # Inputs small enough to stay in the last-level cache (MALL) between calls
    # are timed over several seeded sets in turn, so that every call reads
    # them from HBM.
    nrot = args.rotate if args.rotate > 0 else min(8, max(1, -(-2 * MALL_BYTES // inp.input_bytes())))
    sets = [inp] + [gen.make_inputs(args.workload, device=dev, seed=1000 + i) for i in range(1, nrot)]
    calls = [0]

    def step():
        pk.scan(sets[calls[0] % nrot], workspace=ws, y=y, x_final=xf, stream=stream)
        calls[0] += 1

    print(f"[bench] workload {args.workload}: B={B} H={H} L={L} N={N} K={K}; {nrot} input set(s); "
          f"settle {args.settle_seconds} s, warmup {args.warmup}", file=sys.stderr, flush=True)
    # Clock settle: the GPU needs a while under load to reach its sustained
    # clock; without this phase the timed calls depend on the warm-up count.
    settle_calls = 0
    t_end = time.perf_counter() + args.settle_seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        settle_calls += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for s in range(args.steps):
        step()
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [ev[s].elapsed_time(ev[s + 1]) for s in range(args.steps)]
    sorted_ms = sorted(per_call_ms)
    median_us = sorted_ms[len(sorted_ms) // 2] * 1e3
    min_us = sorted_ms[0] * 1e3
    total_ms = ev[0].elapsed_time(ev[-1])
    ms_per_step = total_ms / args.steps
    tokens = B * H * L
    value = tokens / (ms_per_step * 1e-3)
    alg_bytes = algorithmic_bytes(inp, y, xf)
    avg_call_s = sum(per_call_ms) / len(per_call_ms) * 1e-3
    achieved = alg_bytes / avg_call_s / 1e9
    traffic = counter_traffic(alg_bytes, args.workload)
    print(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (median {median_us:.1f}, min "
          f"{min_us:.1f}), {achieved:.0f} GB/s algorithmic, wall {wall:.3f} s",
          file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x {src.numel()} bytes copied", file=sys.stderr, flush=True)
        del src, dst

    # PDSSM_DETERMINISTIC: the same calls, timed the same way, with and
    # without the flag.
    def det_step(det):
        def f():
            pk.scan(sets[calls[0] % nrot], workspace=ws, y=y, x_final=xf, stream=stream,
                    deterministic=det)
            calls[0] += 1
        return f

    det_steps = max(20, args.steps // 2)
    t_def = _event_time(det_step(False), det_steps, 10, stream)
    t_det = _event_time(det_step(True), det_steps, 10, stream)
    det = {"fwd_us_per_call": t_def * 1e6, "fwd_deterministic_us_per_call": t_det * 1e6,
           "fwd_cost": t_det / t_def - 1.0, "steps": det_steps}
    print(f"[bench] deterministic forward: {t_det * 1e6:.1f} us vs {t_def * 1e6:.1f} us "
          f"({100 * (t_det / t_def - 1):+.1f}%)", file=sys.stderr, flush=True)

    bwd = None if args.no_backward else measure_backward(pk, gen, inp, ws, stream, args)
    if bwd:
        det["bwd_us_per_call"] = bwd["us_per_call"]
        det["bwd_deterministic_us_per_call"] = bwd["deterministic_us_per_call"]
        det["bwd_cost"] = bwd["deterministic_us_per_call"] / bwd["us_per_call"] - 1.0
    aux = None if args.no_backward else measure_aux(pk, gen, inp, stream, args.workload)
    hbm = None if args.no_backward else measure_hbm_practical(alg_bytes, stream)
    if hbm:
        print(f"[bench] practical HBM: read {hbm['read_GBps']:.0f} GB/s, read+write "
              f"{hbm['read_write_GBps']:.0f} GB/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = cpu_threads()
        host = inp.to("cpu")
        orc = oracle.get()
        times = []
        t_start = time.perf_counter()
        while len(times) < args.cpu_reps or time.perf_counter() - t_start < args.cpu_seconds:
            c0 = time.perf_counter()
            orc.scan_inputs(host, nthreads=threads)
            times.append(time.perf_counter() - c0)
        times.sort()
        med = times[len(times) // 2]
        cpu = {"value": tokens / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "nproc": os.cpu_count(), "cpu_model": cpu_model(),
               "sample": f"the whole {args.workload} batch (B={B} H={H} L={L} N={N}), fp64 "
                         f"sequential oracle, OpenMP over the {B * H} sequences on every core "
                         f"the process may use, median of {len(times)} runs ({med:.3f} s each)"}
        best = med
        print(f"[bench] cpu oracle: {best:.2f} s on {threads} threads", file=sys.stderr, flush=True)

    cfgdesc = {
        "lm": "LM-layer scan: bf16 logits argmax over K, complex64 diag, bf16 b/c, bf16 y, "
              "complex64 x_final",
        "long": "time-series scan: int32 selection, permutation dictionary, complex64 "
                "diag/b/c, fp32 y",
        "verylong": "very long scan: int16 selection, complex64 diag, bf16 b/c/y",
        "small": "small real scan: fp32 logits, fp32 diag/b/c/y",
        "tiny": "tiny real scan: int32 selection, fp32 diag/b/c/y",
    }[args.workload]
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "us_per_call_median": median_us,
        "us_per_call_min": min_us,
        "settle_s": args.settle_seconds,
        "settle_calls": settle_calls,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {cfgdesc}", "B": B, "H": H, "L": L, "N": N,
                   "K": K, "global_batch": B * H, "seq_len": L, "parallelism": "single GPU",
                   "input_sets": nrot},
        "achieved_GBps": achieved,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_call": alg_bytes},
        "cpu_baseline": cpu,
        "backward": bwd,
        "deterministic": det,
        "next_rows": aux,
        "hbm_practical": hbm,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
