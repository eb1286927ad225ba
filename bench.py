#!/usr/bin/env python3
"""Benchmark of the H-BitLinear forward on one MI355X.

Headline workload: all seven linears of one 7B-class BitNet v2 block in batched prefill,
M = 16384 tokens, hidden 4096, FFN 8192, INT4 activations: Q, K, V, gate and up are BitLinear
on N(0,1) inputs, Wo (K = 4096) and Wdown (K = 8192) H-BitLinear on outlier-heavy inputs.  One
step = the four activation stages (Q/K/V share one, gate/up another) and the seven product
launches.  value = M * steps / time (tokens/s through the whole block); the roofline object is
the product kernel's int8 matrix-core rate against the 5.0 POPS dense int8 peak.

Also reported (same JSON line): decode shapes (plain BitLinear W1.58A8, K = N = 4096, grouped
over 128 distinct weight matrices and layer by layer, M = 16, 4, 1) against HBM bandwidth on the
packed weights; Wo (M = 4096) and Wdown (M = 8192) alone; the block with fused launches; the
activation stage with the RMS norm; the tiny parity configuration (M = 16, K = N = 256).

Inputs are seeded synthetic data (seeded_inputs) resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA
METRIC = "H-BitLinear tokens/s + effective int-TOPS, % of HBM/int8-MFMA roofline"


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=128)
    p.add_argument("--M", type=int, default=16)
    p.add_argument("--large-steps", type=int, default=10)
    p.add_argument("--no-large", action="store_true", help="skip the large-M workloads")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", choices=["headline", "decode", "decode_grouped", "wo", "wdown",
                                      "block_fused", "qkv_states", "tiny"],
                   default=None,
                   help="run one workload only (profiling): 'headline' is the 7B block alone; "
                        "'decode_grouped' the grouped M = --M decode launch alone")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device-to-device copy of --copy-mib MiB five times "
                        "(the reference point for the HBM byte counters)")
    p.add_argument("--copy-mib", type=int, default=1024)
    p.add_argument("--vendor-int8", action="store_true",
                   help="only time the vendor library's dense int8 GEMM at the large-M shapes "
                        "(context for the int8 MFMA roofline)")
    p.add_argument("--summarize-counters", metavar="DIR", default=None,
                   help="write the HBM-traffic summary from the four counter runs under DIR "
                        "(fetch/, write/, cal_fetch/, cal_write/) to --out")
    p.add_argument("--summarize-trace", metavar="DIR", default=None,
                   help="write the kernel-trace statistics found under DIR to --out")
    p.add_argument("--summarize-pmc", metavar="DIR", default=None,
                   help="write the per-dispatch means of all counters recorded for --kernel under "
                        "DIR (rocprofv3 --pmc output) to --out")
    p.add_argument("--kernel", default="gemm_decode_kernel")
    p.add_argument("--command", default="", help="command line recorded in a summary")
    p.add_argument("--out", default=None)
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """HIP events around every launch of one kernel, recorded on the launching stream."""

    def __init__(self, torch, n):
        self.pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(n)]
        self.i = 0

    def begin(self, stream):
        self.pairs[self.i][0].record(stream)

    def end(self, stream):
        self.pairs[self.i][1].record(stream)
        self.i += 1

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs[: self.i]) / max(self.i, 1)

    def median_ms(self):
        v = sorted(a.elapsed_time(b) for a, b in self.pairs[: self.i])
        return v[len(v) // 2] if v else 0.0


def canonical_packed_bytes(N, K):
    # five trits per byte with nothing wasted: the algorithmic weight bytes
    return N * ((K + 4) // 5)


# --------------------------------------------------------------------------- decode ----

def make_decode(torch, tb, si, M, L, unique=4):
    """L distinct packed 4096x4096 weight buffers (copies of `unique` seeded matrices at
    distinct addresses) and L distinct seeded inputs."""
    K = N = 4096
    dev = torch.device("cuda:0")
    packs = []
    for u in range(unique):
        W = si.gaussian_weights(2, N, K, layer=u)
        packed, g = tb.bitnet_pack_weights(W)
        packs.append((torch.from_numpy(packed).to(dev), g))
    ws, gs = [], []
    for l in range(L):
        p, g = packs[l % unique]
        ws.append(p.clone())
        gs.append(g)
    x = torch.from_numpy(si.normal(si.seed_for(2, 0), L * M * K).reshape(L, M, K)).to(dev)
    ptrs = torch.tensor([w.data_ptr() for w in ws], dtype=torch.int64, device=dev)
    wsc = torch.tensor(gs, dtype=torch.float32, device=dev)
    return dict(M=M, K=K, N=N, L=L, x=x, w=ws, g=gs, packs=packs, ptrs=ptrs, wsc=wsc)


def decode_gemm_bytes(M, K, N):
    return canonical_packed_bytes(N, K) + M * K + 4 * M + 4 * M * N


def run_decode_grouped(torch, tb, d, steps, warmup):
    """One step = the activation stage over all L*M rows, then one grouped product launch
    over the L layers (what hbitlinear_forward_grouped runs).

    After the warmup steps the `steps` steps are captured once as a HIP graph, and replayed
    untimed for about 0.2 s so that the clocks settle.  Then two passes over `steps` steps
    each.  The launch pass runs them eagerly with HIP events around every launch on the
    launching stream: the per-launch durations of the two kernels.  The timed pass is one
    replay of the graph, so that the host's launch overhead (two library calls per step) does
    not leave the GPU idle between kernels; its wall time gives the throughput.  Every replay's
    output must equal the eager output bit for bit."""
    M, K, N, L = d["M"], d["K"], d["N"], d["L"]
    dev = torch.device("cuda:0")
    codes = torch.empty(tb.hbitlinear_codes_bytes(L * M, K, 8), dtype=torch.uint8, device=dev)
    scales = torch.empty(L * M, dtype=torch.float32, device=dev)
    y = torch.empty((L, M, N), dtype=torch.float32, device=dev)
    xf = d["x"].view(L * M, K)

    def step(stream, tq=None, tg=None):
        if tq: tq.begin(stream)
        tb.hbitlinear_quantize(xf, 8, False, codes=codes, scales=scales, stream=stream)
        if tq: tq.end(stream)
        if tg: tg.begin(stream)
        tb.hbitlinear_gemm_dequant_grouped(codes, scales, L, M, K, N, 8, d["ptrs"], d["wsc"], out=y,
                                           stream=stream)
        if tg: tg.end(stream)

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step(stream)
    torch.cuda.synchronize()
    y_eager = y.clone()
    # the steps as one graph (captured on a side stream, as torch requires)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for _ in range(steps):
            step(cap)

    def check():
        if not torch.equal(y, y_eager):
            raise RuntimeError("graph replay of the decode step differs from the eager result")

    y.zero_()
    graph.replay()
    torch.cuda.synchronize()
    check()
    # untimed replays for about 0.2 s, so that the clocks have settled before either pass
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        graph.replay()
        torch.cuda.synchronize()
    # launch pass
    tq, tg = Timer(torch, steps), Timer(torch, steps)
    for _ in range(steps):
        step(stream, tq, tg)
    torch.cuda.synchronize()
    gemm_ms = tg.mean_ms()
    gemm_ms_median = tg.median_ms()
    check()
    # timed pass
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    check()
    del graph
    bytes_gemm = L * decode_gemm_bytes(M, K, N)
    return dict(seconds=dt, ms_per_step=1e3 * dt / steps, tokens_per_s=M * L * steps / dt,
                int_tops=2.0 * M * N * K * L * steps / dt / 1e12, gemm_us=1e3 * gemm_ms,
                gemm_us_median=1e3 * gemm_ms_median,
                quant_us=1e3 * tq.mean_ms(), gemm_bytes=bytes_gemm,
                gemm_gbs=bytes_gemm / (gemm_ms * 1e-3) / 1e9)


def run_decode(torch, tb, d, steps, warmup):
    """Layer after layer: one activation stage and one product launch per layer (what a model
    running one layer at a time does).  As for the grouped step, the steps are captured once as
    a HIP graph and one replay is timed (so the host's launch overhead does not leave the GPU
    idle between launches); an eager pass with HIP events around every launch gives the
    per-launch durations.  Every replay's output must equal the eager output bit for bit."""
    M, K, N, L = d["M"], d["K"], d["N"], d["L"]
    dev = torch.device("cuda:0")
    codes = torch.empty(tb.hbitlinear_codes_bytes(M, K, 8), dtype=torch.uint8, device=dev)
    scales = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty((L, M, N), dtype=torch.float32, device=dev)

    def step(stream, tq=None, tg=None):
        for l in range(L):
            if tq: tq.begin(stream)
            tb.hbitlinear_quantize(d["x"][l], 8, False, codes=codes, scales=scales, stream=stream)
            if tq: tq.end(stream)
            if tg: tg.begin(stream)
            tb.hbitlinear_gemm_dequant(codes, scales, M, K, N, 8, d["w"][l], d["g"][l], out=y[l],
                                       stream=stream)
            if tg: tg.end(stream)

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step(stream)
    torch.cuda.synchronize()
    y_eager = y.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for _ in range(steps):
            step(cap)

    def check():
        if not torch.equal(y, y_eager):
            raise RuntimeError("graph replay of the layer-by-layer decode differs from the eager result")

    y.zero_()
    graph.replay()
    torch.cuda.synchronize()
    check()
    # launch pass (eager, events around every launch)
    tq, tg = Timer(torch, steps * L), Timer(torch, steps * L)
    for _ in range(steps):
        step(stream, tq, tg)
    torch.cuda.synchronize()
    check()
    # timed pass: one replay
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    check()
    del graph
    gemm_ms = tg.mean_ms()
    bytes_gemm = decode_gemm_bytes(M, K, N)
    return dict(seconds=dt, ms_per_step=1e3 * dt / steps, tokens_per_s=M * L * steps / dt,
                us_per_layer=1e6 * dt / (steps * L),
                int_tops=2.0 * M * N * K * L * steps / dt / 1e12, gemm_us=1e3 * gemm_ms,
                quant_us=1e3 * tq.mean_ms(), gemm_bytes=bytes_gemm,
                gemm_gbs=bytes_gemm / (gemm_ms * 1e-3) / 1e9)


def cpu_baseline_decode(si, oracle, d, tb, min_seconds=10.0, max_seconds=30.0):
    """The oracle forward over the decode layers (host only), layer after layer, until at
    least `min_seconds` have passed (or all layers are done); a layer is never cut short, and
    no new layer starts after `max_seconds`."""
    M, K, N, L = d["M"], d["K"], d["N"], d["L"]
    xs = d["x"].cpu().numpy()
    unique = len(d["packs"])
    # the oracle's own packing of the same seeded matrices (make_decode's recipe)
    packs = []
    for u in range(unique):
        p, g, _t = oracle.pack_weights(si.gaussian_weights(2, N, K, layer=u))
        packs.append((p, g))
    layers = 0
    t0 = time.perf_counter()
    while layers < L:
        p, g = packs[layers % unique]
        oracle.forward(xs[layers], p, g, N, 8, False)
        layers += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el >= max_seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=M * layers / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{layers} of the {L} layers at M={M} (unpack + quantise + add/sub "
                       f"product + epilogue per layer), {dt:.1f} s")


def cpu_baseline_large(si, oracle, config, rows_max=256, chunk=16):
    """The oracle forward of every linear of a large-M workload on its first `rows_max` token
    rows (seeded, as the GPU runs them), `chunk` rows at a time per linear: tokens/s for the
    whole workload (a token goes through every linear)."""
    M_full = si.workload(config).linears[0].M
    # the seeded generators are counter-based and row-major: the first rows of the workload are
    # the workload built with that many rows
    wl = si.workload(config, M=min(M_full, rows_max))
    lins = []
    for lin in wl.linears:
        x = si.activations(config, lin)
        packed, g, _t = oracle.pack_weights(si.weights(config, lin))
        lins.append((lin, x, packed, g))
    rows, t_total = 0, 0.0
    while rows + chunk <= wl.linears[0].M:
        t0 = time.perf_counter()
        for lin, x, packed, g in lins:
            oracle.forward(x[rows:rows + chunk], packed, g, lin.N, lin.act_bits, lin.use_hadamard)
        t_total += time.perf_counter() - t0
        rows += chunk
    return dict(value=rows / t_total, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"the first {rows} of {M_full} token rows through all "
                       f"{len(lins)} linear(s) (quantise + unpack + add/sub product + epilogue), "
                       f"{t_total:.1f} s")


# ------------------------------------------------------------- counters and traces ----

# kernel name prefix -> the sources it is compiled from (a counter summary is void once they change)
KERNEL_SOURCES = {
    "gemm_decode_kernel": ["gemm_decode.hip", "common.h"],
    "gemm_tern_kernel": ["gemm.hip", "common.h"],
    "gemm_tern4_kernel": ["gemm.hip", "common.h"],
    "quantize_rows_kernel": ["quant.hip", "common.h"],
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "ternary_weight_bit_bitlinear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_calibration(torch, mib):
    """A plain device-to-device copy of `mib` MiB, five times: each launch reads and writes
    exactly mib MiB, which fixes the scale of the HBM byte counters."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(7)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(0)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert int(dst[n - 1]) == 7
    return {"copy_bytes_per_launch": n, "launches": 5}


def vendor_int8(torch):
    """Context for the large-M roofline: the vendor library's dense int8 GEMM (torch._int_mm,
    int8 x int8 -> int32, hipBLASLt on ROCm) at the shapes of the three large-M workloads, on
    plain int8 operands.  It has no ternary decoding, no activation stage and no epilogue; it
    shows what a tuned int8 MFMA kernel reaches on this GPU at these sizes."""
    out = {}
    for name, (M, K, N) in (("wo", (4096, 4096, 4096)), ("wdown", (8192, 16384, 4096)),
                            ("qkv_gate_up", (16384, 4096, 8192))):
        g = torch.Generator(device="cuda:0").manual_seed(5)
        a = torch.randint(-8, 8, (M, K), dtype=torch.int8, device="cuda:0", generator=g)
        b = torch.randint(-1, 2, (N, K), dtype=torch.int8, device="cuda:0", generator=g)
        bt = b.t()
        for _ in range(3):
            c = torch._int_mm(a, bt)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 10
        e0.record()
        for _ in range(n):
            c = torch._int_mm(a, bt)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n * 1e3
        out[name] = dict(M=M, K=K, N=N, us=us, tops=2.0 * M * N * K / (us * 1e-6) / 1e12)
        log(f"[bench] vendor int8 GEMM {name} {M}x{K}x{N}: {us:.1f} us, {out[name]['tops']:.0f} TOP/s")
        del a, b, bt, c
    return out


def _counter_means(d, kernel_prefix, counter):
    """Mean per dispatch of `counter` over the dispatches of kernels whose name holds
    `kernel_prefix` (values of one dispatch summed over its instances)."""
    import csv
    import glob
    per = {}
    for f in sorted(glob.glob(os.path.join(d, "**", "*_counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel_prefix in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    key = (f, r["Dispatch_Id"])
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} values for {kernel_prefix} under {d}")
    return per


def summarize_counters(args):
    """HBM bytes per launch of one kernel from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the plain copy of known size."""
    d = args.summarize_counters
    fetch = list(_counter_means(os.path.join(d, "fetch"), args.kernel, "FETCH_SIZE").values())
    write = list(_counter_means(os.path.join(d, "write"), args.kernel, "WRITE_SIZE").values())
    cal_f = _counter_means(os.path.join(d, "cal_fetch"), COPY_KERNEL, "FETCH_SIZE")
    cal_w = _counter_means(os.path.join(d, "cal_write"), COPY_KERNEL, "WRITE_SIZE")
    copy_bytes = args.copy_mib << 20
    # the five big copies are the largest copy dispatches of the calibration run
    cf = sorted(cal_f.values())[-5:]
    cw = sorted(cal_w.values())[-5:]
    f_scale = copy_bytes / (1024.0 * sum(cf) / len(cf))
    w_scale = copy_bytes / (1024.0 * sum(cw) / len(cw))
    f_kib = sum(fetch) / len(fetch)
    w_kib = sum(write) / len(write)
    traffic = 1024.0 * (f_kib * f_scale + w_kib * w_scale)
    lines = [
        f"# HBM traffic of {args.kernel}: rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated",
        f"kernel: {args.kernel}",
        f"source_digest: {source_digest(args.kernel)}",
        f"dispatches_fetch: {len(fetch)}",
        f"dispatches_write: {len(write)}",
        f"fetch_kib_per_dispatch: {f_kib:.1f}",
        f"write_kib_per_dispatch: {w_kib:.1f}",
        f"copy_bytes_per_dispatch: {copy_bytes}",
        f"copy_fetch_kib_per_dispatch: {sum(cf) / len(cf):.1f}",
        f"copy_write_kib_per_dispatch: {sum(cw) / len(cw):.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        "commands:",
    ] + ["  " + c for c in args.command.split(" ;; ") if c]
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text, end="")


def summarize_pmc(args):
    """Means per dispatch of every counter a set of rocprofv3 --pmc runs recorded for one
    kernel, with the MFMA cross-check: each v_mfma_i32_16x16x64_i8 wave instruction is
    16 * 16 * 64 multiply-adds = 32768 integer operations."""
    import csv
    import glob
    names = set()
    for f in glob.glob(os.path.join(args.summarize_pmc, "**", "*_counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if args.kernel in r["Kernel_Name"]:
                    names.add(r["Counter_Name"])
    if not names:
        raise SystemExit(f"no counters for {args.kernel} under {args.summarize_pmc}")
    means = {}
    for n in sorted(names):
        v = list(_counter_means(args.summarize_pmc, args.kernel, n).values())
        means[n] = (sum(v) / len(v), len(v))
    lines = [f"# rocprofv3 --pmc counters of {args.kernel}, mean per dispatch", "commands:"]
    lines += ["  " + c for c in args.command.split(" ;; ") if c]
    lines.append("")
    for n, (m, k) in means.items():
        lines.append(f"{n}: {m:.6g}   ({k} dispatches)")
    if "SQ_INSTS_MFMA" in means:
        ops = means["SQ_INSTS_MFMA"][0] * 32768.0
        lines.append(f"int8 operations from SQ_INSTS_MFMA x 32768: {ops:.6g}")
    if "SQ_INSTS_VALU_MFMA_MOPS_I8" in means:
        lines.append(f"int8 operations from SQ_INSTS_VALU_MFMA_MOPS_I8 x 512: "
                     f"{means['SQ_INSTS_VALU_MFMA_MOPS_I8'][0] * 512.0:.6g}")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in means and "GRBM_GUI_ACTIVE" in means:
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs; the MFMA busy cycles over the 1024 SIMDs
        busy = means["SQ_VALU_MFMA_BUSY_CYCLES"][0] / 1024.0
        act = means["GRBM_GUI_ACTIVE"][0] / 8.0
        lines.append(f"MFMA busy cycles per SIMD: {busy:.6g}; active cycles per XCD: {act:.6g}; "
                     f"busy fraction {busy / act:.3f}")
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text, end="")


def summarize_trace(args):
    """The per-kernel statistics table of a rocprofv3 --kernel-trace --stats run, as text."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_stats.csv"),
                             recursive=True))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {args.summarize_trace}")
    rows = []
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            rows.append(r)
    lines = ["# rocprofv3 --kernel-trace --stats summary", "command:"]
    lines += ["  " + c for c in args.command.split(" ;; ") if c]
    lines.append("")
    lines.append(f"{'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'share%':>7}  kernel")
    for r in rows:
        name = r["Name"]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):7.2f}  {name}")
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text, end="")


def recorded_traffic(kernel, workload):
    """traffic_bytes_per_launch from the committed counter summary of `kernel` on `workload`,
    or None when there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest(kernel):
        return None
    return float(kv["traffic_bytes_per_launch"])


# -------------------------------------------------------------------------- large M ----

def run_large(torch, tb, si, config, steps, warmup):
    wl = si.workload(config)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    lins = []
    xcache = {}
    qcache = {}
    for lin in wl.linears:
        key = lin.x_kind
        if key not in xcache:
            xcache[key] = torch.from_numpy(si.activations(config, lin)).to(dev)
        W = si.weights(config, lin)
        packed, g = tb.bitnet_pack_weights(W)
        del W
        # Linears that read the same activations with the same mode (Q, K, V; gate, up) share
        # one activation stage: its codes and scales are the same for all of them.
        qkey = (key, lin.act_bits, lin.use_hadamard)
        first = qkey not in qcache
        if first:
            qcache[qkey] = (torch.empty(tb.hbitlinear_codes_bytes(lin.M, lin.K, lin.act_bits),
                                        dtype=torch.uint8, device=dev),
                            torch.empty(lin.M, dtype=torch.float32, device=dev))
        codes, scales = qcache[qkey]
        out = torch.empty((lin.M, lin.N), dtype=torch.float32, device=dev)
        lins.append((lin, xcache[key], torch.from_numpy(packed).to(dev), g, codes, scales, out, first))
    n = len(lins)

    def step(tq=None, tg=None):
        for j, (lin, x, pw, g, codes, scales, out, first) in enumerate(lins):
            if first:
                if tq: tq[j].begin(stream)
                tb.hbitlinear_quantize(x, lin.act_bits, lin.use_hadamard, codes=codes, scales=scales,
                                       stream=stream)
                if tq: tq[j].end(stream)
            if tg: tg[j].begin(stream)
            tb.hbitlinear_gemm_dequant(codes, scales, lin.M, lin.K, lin.N, lin.act_bits, pw, g,
                                       out=out, stream=stream)
            if tg: tg[j].end(stream)

    for _ in range(warmup):
        step()
    # untimed steps for about 0.3 s more, so that the clocks have settled before timing
    torch.cuda.synchronize()
    t_end = time.perf_counter() + 0.3
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    tq = [Timer(torch, steps) for _ in range(n)]
    tg = [Timer(torch, steps) for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(tq, tg)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    M = wl.linears[0].M
    ops = sum(2.0 * l.M * l.N * l.K for l in wl.linears)
    # HBM bytes of a step at the algorithmic minimum: every activation stage reads x and writes
    # codes and scales once; every product reads codes, scales and packed weights (canonical
    # five trits per byte) and writes y.
    e2e_bytes = 0.0
    for lin, *_r, first in lins:
        cb = lin.M * lin.K * lin.act_bits // 8
        if first:
            e2e_bytes += 4 * lin.M * lin.K + cb + 4 * lin.M
        e2e_bytes += cb + 4 * lin.M + canonical_packed_bytes(lin.N, lin.K) + 4 * lin.M * lin.N
    gemm_s = sum(t.mean_ms() for t in tg) * 1e-3
    quant_s = sum(t.mean_ms() for t, l in zip(tq, lins) if l[-1]) * 1e-3
    per = {}
    for j, (lin, *_rest) in enumerate(lins):
        g_ms = tg[j].mean_ms()
        qbytes = 4 * lin.M * lin.K + lin.M * lin.K * lin.act_bits // 8 + 4 * lin.M
        per[lin.name] = dict(gemm_us=1e3 * g_ms,
                             gemm_tops=2.0 * lin.M * lin.N * lin.K / (g_ms * 1e-3) / 1e12)
        if lins[j][-1]:
            q_ms = tq[j].mean_ms()
            per[lin.name].update(quant_us=1e3 * q_ms, quant_gbs=qbytes / (q_ms * 1e-3) / 1e9)
        else:
            per[lin.name].update(quant_shared=True)
    res = dict(workload=wl.name, M=M, ms_per_step=1e3 * dt / steps,
               ops_per_step=ops, gemm_us_per_step=1e6 * gemm_s,
               tokens_per_s=M * steps / dt, int_tops=ops * steps / dt / 1e12,
               gemm_int_tops=ops / gemm_s / 1e12,
               gemm_mfma_frac=ops / gemm_s / 1e12 / INT8_PEAK_TOPS,
               end_to_end_mfma_frac=ops * steps / dt / 1e12 / INT8_PEAK_TOPS,
               end_to_end_roofline_frac=max(e2e_bytes / (HBM_PEAK_GBS * 1e9),
                                            ops / (INT8_PEAK_TOPS * 1e12)) / (dt / steps),
               quant_share=quant_s / (quant_s + gemm_s), linears=per)
    del lins, xcache
    torch.cuda.empty_cache()
    return res


def run_block_fused(torch, tb, si, steps, warmup):
    """The 7B-class BitNet v2 block of the block workload (same inputs and weights) with fused
    launches: Q, K and V as one three-segment product launch; gate and up as one launch whose
    epilogue writes SwishGLU(gate, up); Wdown (H-BitLinear) reading that output, its real input
    in a block.  The SwishGLU glue is work the unfused block workload does not do."""
    import numpy as np
    wl = si.workload(5)
    L = {l.name: l for l in wl.linears}
    M = L["q"].M
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    up = lambda a: torch.from_numpy(a).to(dev)
    x_qkv = up(si.activations(5, L["q"]))
    x_wo = up(si.activations(5, L["wo"]))
    x_ffn = up(si.activations(5, L["gate"]))
    seg_n = [L["q"].N, L["k"].N, L["v"].N]
    Wqkv = np.concatenate([si.weights(5, L[n]) for n in ("q", "k", "v")])
    p_qkv, g_qkv = tb.bitnet_pack_weights_segments(Wqkv, seg_n)
    del Wqkv
    p_wo, g_wo = tb.bitnet_pack_weights(si.weights(5, L["wo"]))
    p_gu, g_gate, g_up = tb.bitnet_pack_gate_up(si.weights(5, L["gate"]), si.weights(5, L["up"]))
    p_wd, g_wd = tb.bitnet_pack_weights(si.weights(5, L["wdown"]))
    p_qkv, p_wo, p_gu, p_wd = up(p_qkv), up(p_wo), up(p_gu), up(p_wd)
    F = L["gate"].N
    Kq, Kd = L["q"].K, L["wdown"].K

    def stage(K):
        return (torch.empty(tb.hbitlinear_codes_bytes(M, K, 4), dtype=torch.uint8, device=dev),
                torch.empty(M, dtype=torch.float32, device=dev))
    c_qkv, c_wo, c_ffn, c_wd = stage(Kq), stage(Kq), stage(Kq), stage(Kd)
    y_qkv = torch.empty((M, sum(seg_n)), dtype=torch.float32, device=dev)
    y_wo = torch.empty((M, L["wo"].N), dtype=torch.float32, device=dev)
    h = torch.empty((M, F), dtype=torch.float32, device=dev)
    y_wd = torch.empty((M, L["wdown"].N), dtype=torch.float32, device=dev)

    names = ["qkv", "wo", "gate_up_swiglu", "wdown"]
    hads = {"qkv": False, "wo": True, "gate_up_swiglu": False, "wdown": True}

    def step(tq=None, tg=None):
        def q(j, x, c):
            if tq: tq[j].begin(stream)
            tb.hbitlinear_quantize(x, 4, hads[names[j]], codes=c[0], scales=c[1], stream=stream)
            if tq: tq[j].end(stream)

        def g(j, fn):
            if tg: tg[j].begin(stream)
            fn()
            if tg: tg[j].end(stream)
        q(0, x_qkv, c_qkv)
        g(0, lambda: tb.hbitlinear_gemm_dequant_segments(c_qkv[0], c_qkv[1], M, Kq, seg_n, 4, p_qkv,
                                                         g_qkv, out=y_qkv, stream=stream))
        q(1, x_wo, c_wo)
        g(1, lambda: tb.hbitlinear_gemm_dequant(c_wo[0], c_wo[1], M, Kq, L["wo"].N, 4, p_wo, g_wo,
                                                out=y_wo, stream=stream))
        q(2, x_ffn, c_ffn)
        g(2, lambda: tb.hbitlinear_gemm_swiglu(c_ffn[0], c_ffn[1], M, Kq, F, 4, p_gu, g_gate, g_up,
                                               out=h, stream=stream))
        q(3, h, c_wd)
        g(3, lambda: tb.hbitlinear_gemm_dequant(c_wd[0], c_wd[1], M, Kd, L["wdown"].N, 4, p_wd, g_wd,
                                                out=y_wd, stream=stream))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + 0.3
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    tq = [Timer(torch, steps) for _ in names]
    tg = [Timer(torch, steps) for _ in names]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(tq, tg)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    shapes = {"qkv": (Kq, sum(seg_n), sum(seg_n)), "wo": (Kq, L["wo"].N, L["wo"].N),
              "gate_up_swiglu": (Kq, 2 * F, F), "wdown": (Kd, L["wdown"].N, L["wdown"].N)}
    ops = sum(2.0 * M * n * k for k, n, _o in shapes.values())
    e2e_bytes = 0.0
    per = {}
    for j, name in enumerate(names):
        k, n, n_out = shapes[name]
        cb = M * k // 2
        qbytes = 4 * M * k + cb + 4 * M
        e2e_bytes += qbytes + cb + 4 * M + canonical_packed_bytes(n, k) + 4 * M * n_out
        g_ms, q_ms = tg[j].mean_ms(), tq[j].mean_ms()
        per[name] = dict(gemm_us=1e3 * g_ms, gemm_tops=2.0 * M * n * k / (g_ms * 1e-3) / 1e12,
                         quant_us=1e3 * q_ms, quant_gbs=qbytes / (q_ms * 1e-3) / 1e9)
    gemm_s = sum(t.mean_ms() for t in tg) * 1e-3
    quant_s = sum(t.mean_ms() for t in tq) * 1e-3
    res = dict(workload=f"bitnet_v2_7b_block_fused_int4_M{M}", M=M, ms_per_step=1e3 * dt / steps,
               tokens_per_s=M * steps / dt, int_tops=ops * steps / dt / 1e12,
               gemm_int_tops=ops / gemm_s / 1e12,
               gemm_mfma_frac=ops / gemm_s / 1e12 / INT8_PEAK_TOPS,
               end_to_end_mfma_frac=ops * steps / dt / 1e12 / INT8_PEAK_TOPS,
               end_to_end_roofline_frac=max(e2e_bytes / (HBM_PEAK_GBS * 1e9),
                                            ops / (INT8_PEAK_TOPS * 1e12)) / (dt / steps),
               quant_share=quant_s / (quant_s + gemm_s), launches=per,
               fused="qkv: one 3-segment product launch; gate/up: one launch with SwishGLU in the "
                     "epilogue; wdown reads the SwishGLU output")
    del x_qkv, x_wo, x_ffn, h, y_qkv, y_wo, y_wd
    torch.cuda.empty_cache()
    return res


def run_qkv_states(torch, tb, si, steps):
    """The block's Q, K and V projections (M = 16384, K = 4096, one three-segment product launch
    on one activation stage) with the low-bit states fused into the epilogue (Q 4 bits, K and V
    3 bits, heads of 128: int8 codes and a scale per head) against the same launch writing the
    fp32 projections."""
    import numpy as np
    wl = si.workload(5)
    L = {l.name: l for l in wl.linears}
    M, K = L["q"].M, L["q"].K
    seg_n = [L[n].N for n in ("q", "k", "v")]
    N = sum(seg_n)
    bits, group = [4, 3, 3], 128
    x = torch.from_numpy(si.activations(5, L["q"])).cuda()
    W = np.concatenate([si.weights(5, L[n]) for n in ("q", "k", "v")])
    packed, gs = tb.bitnet_pack_weights_segments(W, seg_n)
    del W
    pw = torch.from_numpy(packed).cuda()
    codes, scales = tb.hbitlinear_quantize(x, 4, False)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    sc = torch.empty((M, N), dtype=torch.int8, device="cuda")
    ss = torch.empty((M, N // group), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = dict(M=M, K=K, seg_n=seg_n, state_bits=bits, group=group)
    for mode in ("fp32", "states"):
        def once():
            if mode == "fp32":
                tb.hbitlinear_gemm_dequant_segments(codes, scales, M, K, seg_n, 4, pw, gs, out=y,
                                                    stream=stream)
            else:
                tb.hbitlinear_gemm_qkv_states(codes, scales, M, K, seg_n, 4, pw, gs, bits, group,
                                              state_codes=sc, state_scales=ss, stream=stream)
        for _ in range(2):
            once()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + 0.3      # settle the clocks
        while time.perf_counter() < t_end:
            once()
            torch.cuda.synchronize()
        t = Timer(torch, steps)
        for _ in range(steps):
            t.begin(stream)
            once()
            t.end(stream)
        torch.cuda.synchronize()
        us = 1e3 * t.mean_ms()
        out_bytes = 4 * M * N if mode == "fp32" else M * N + 4 * M * (N // group)
        res[mode] = dict(launch_us=us, tops=2.0 * M * N * K / (us * 1e-6) / 1e12,
                         output_bytes=out_bytes)
    res.update(workload=f"bitnet_v2_qkv_states_int4_M{M}_K{K}", ms_per_step=res["states"]["launch_us"] / 1e3,
               tokens_per_s=M / (res["states"]["launch_us"] * 1e-6))
    del x, y, sc, ss, codes, scales
    torch.cuda.empty_cache()
    return res


def run_qkv_states_decode(torch, tb, si, steps, M=16):
    """The block's Q, K and V projections at a decode step (M = 16 tokens, K = 4096, one
    three-segment launch of the decode kernel) with the low-bit states in the epilogue -- the
    rows a 3-bit KV cache takes on each step -- against the same launch writing fp32, with
    INT8 and INT4 activations."""
    import numpy as np
    wl = si.workload(5, M=M)                  # the block's first M token rows
    L = {l.name: l for l in wl.linears}
    K = L["q"].K
    seg_n = [L[n].N for n in ("q", "k", "v")]
    N = sum(seg_n)
    bits, group = [4, 3, 3], 128
    x = torch.from_numpy(si.activations(5, L["q"])).cuda()
    W = np.concatenate([si.weights(5, L[n]) for n in ("q", "k", "v")])
    packed, gs = tb.bitnet_pack_weights_segments(W, seg_n)
    del W
    pw = torch.from_numpy(packed).cuda()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    sc = torch.empty((M, N), dtype=torch.int8, device="cuda")
    ss = torch.empty((M, N // group), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    wbytes = canonical_packed_bytes(N, K)
    res = dict(workload=f"bitnet_v2_qkv_states_decode_M{M}_K{K}", M=M, K=K, seg_n=seg_n,
               state_bits=bits, group=group, packed_weight_bytes=wbytes)
    for act in (8, 4):
        codes, scales = tb.hbitlinear_quantize(x, act, False)
        for mode in ("fp32", "states"):
            def once():
                if mode == "fp32":
                    tb.hbitlinear_gemm_dequant_segments(codes, scales, M, K, seg_n, act, pw, gs, out=y,
                                                        stream=stream)
                else:
                    tb.hbitlinear_gemm_qkv_states(codes, scales, M, K, seg_n, act, pw, gs, bits, group,
                                                  state_codes=sc, state_scales=ss, stream=stream)
            for _ in range(3):
                once()
            torch.cuda.synchronize()
            t = Timer(torch, steps)
            for _ in range(steps):
                t.begin(stream)
                once()
                t.end(stream)
            torch.cuda.synchronize()
            us = 1e3 * t.mean_ms()
            res[f"a{act}_{mode}"] = dict(launch_us=us, weight_gbs=wbytes / (us * 1e-6) / 1e9)
    del x, y, sc, ss, pw
    torch.cuda.empty_cache()
    return res


def run_k1_rmsnorm(torch, tb, si, steps):
    """The activation stage with and without the RMS norm folded in, at the large-M shapes: the
    norm adds a reduction and a gain read but no pass over x."""
    out = {}
    for name, (M, K, had) in (("wo", (4096, 4096, True)), ("wdown", (8192, 16384, True)),
                              ("block_qkv", (16384, 4096, False))):
        x = torch.from_numpy(si.wo_activations(M, K)).cuda()
        gain = torch.from_numpy(si.normal(si.seed_for(5, 12), K, 1.0, 0.1)).cuda()
        codes = torch.empty(tb.hbitlinear_codes_bytes(M, K, 4), dtype=torch.uint8, device="cuda")
        scales = torch.empty(M, dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()
        res = {}
        for mode in ("plain", "rmsnorm"):
            def once():
                if mode == "plain":
                    tb.hbitlinear_quantize(x, 4, had, codes=codes, scales=scales, stream=stream)
                else:
                    tb.hbitlinear_quantize_rmsnorm(x, gain, 1e-6, 4, had, codes=codes, scales=scales,
                                                   stream=stream)
            for _ in range(3):
                once()
            t = Timer(torch, steps)
            for _ in range(steps):
                t.begin(stream)
                once()
                t.end(stream)
            torch.cuda.synchronize()
            nbytes = 4 * M * K + M * K // 2 + 4 * M + (4 * K if mode == "rmsnorm" else 0)
            res[mode] = dict(us=1e3 * t.mean_ms(), gbs=nbytes / (t.mean_ms() * 1e-3) / 1e9)
        res["M"], res["K"], res["hadamard"] = M, K, had
        out[name] = res
        del x
    torch.cuda.empty_cache()
    return out


def run_tiny(torch, tb, si, steps=50):
    """The tiny parity configuration (M = 16, K = N = 256, H-BitLinear INT8): one forward per
    step, HIP events around each call; launch latency dominates at this size."""
    lin = si.workload(1).linears[0]
    x = torch.from_numpy(si.activations(1, lin)).cuda()
    packed, g = tb.bitnet_pack_weights(si.weights(1, lin))
    pw = torch.from_numpy(packed).cuda()
    out = torch.empty((lin.M, lin.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(tb.hbitlinear_workspace_bytes(lin.M, lin.K, lin.act_bits), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(5):
        tb.hbitlinear_forward(x, lin.N, lin.act_bits, lin.use_hadamard, pw, g, out=out, workspace=ws)
    t = Timer(torch, steps)
    for _ in range(steps):
        t.begin(stream)
        tb.hbitlinear_forward(x, lin.N, lin.act_bits, lin.use_hadamard, pw, g, out=out, workspace=ws,
                              stream=stream)
        t.end(stream)
    torch.cuda.synchronize()
    us = 1e3 * t.mean_ms()
    return dict(workload=f"hbitlinear_int8_tiny_M{lin.M}_K{lin.K}_N{lin.N}", forward_us=us,
                tokens_per_s=lin.M / (us * 1e-6))


def cpu_baseline_tiny(si, oracle, min_seconds=3.0):
    """The oracle forward of the tiny configuration, repeated for at least `min_seconds`."""
    lin = si.workload(1).linears[0]
    x = si.activations(1, lin)
    packed, g, _t = oracle.pack_weights(si.weights(1, lin))
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_seconds:
        oracle.forward(x, packed, g, lin.N, lin.act_bits, lin.use_hadamard)
        n += 1
    dt = time.perf_counter() - t0
    return dict(value=lin.M * n / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} forwards of the whole M={lin.M} K={lin.K} N={lin.N} configuration, "
                       f"{dt:.1f} s")


def decode_report(torch, tb, si, args):
    """Decode shapes: grouped over L distinct matrices (M = --M, then 1 and 4) and layer by
    layer.  The HBM fraction counts the packed weights at five trits per byte only; the codes,
    scales and outputs a launch also moves are reported beside it."""
    out = {}
    log(f"[bench] decode: preparing M={args.M}, {args.layers} layers")
    d = make_decode(torch, tb, si, args.M, args.layers)
    M, K, N, L = d["M"], d["K"], d["N"], d["L"]
    weight_bytes = L * canonical_packed_bytes(N, K)
    r = run_decode_grouped(torch, tb, d, args.steps, args.warmup)
    gbs = weight_bytes / (r["gemm_us"] * 1e-6) / 1e9
    traffic = recorded_traffic("gemm_decode_kernel", f"M{M}_L{L}")
    out["grouped"] = dict(
        workload=f"bitlinear_w158a8_decode_M{M}_K{K}_N{N}_grouped_L{L}",
        launch="one grouped product launch over L distinct weight matrices (the layers' weights "
               "together exceed the Infinity Cache), after one activation stage over L*M rows",
        tokens_per_s=r["tokens_per_s"], ms_per_step=r["ms_per_step"], int_tops=r["int_tops"],
        quant_kernel_us=r["quant_us"],
        roofline={"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                  "kernel": "gemm_decode_kernel<8,true,4,0>", "launch_us": r["gemm_us"],
                  "launch_us_median": r["gemm_us_median"],
                  "algorithmic_bytes_per_launch": weight_bytes,
                  "other_bytes_per_launch": L * (M * K + 4 * M + 4 * M * N)})
    log(f"[bench] decode grouped M={M}: {r['tokens_per_s']:.4g} tokens/s, gemm {r['gemm_us']:.1f} us "
        f"({gbs:.0f} GB/s on packed weights), quant {r['quant_us']:.1f} us")
    if args.only == "decode_grouped":
        return out
    rs = run_decode(torch, tb, d, max(2, args.steps // 4), 1)
    wl_bytes = canonical_packed_bytes(N, K)
    out["sequential"] = dict(
        launch="per layer: one activation stage and one product launch",
        tokens_per_s=rs["tokens_per_s"], us_per_layer=rs["us_per_layer"],
        timed_as="the steps captured as a HIP graph, one replay timed; launch times from HIP "
                 "events in an eager pass",
        gemm_us_per_layer=rs["gemm_us"], quant_us_per_layer=rs["quant_us"],
        weight_gbs=wl_bytes / (rs["gemm_us"] * 1e-6) / 1e9,
        hbm_frac=wl_bytes / (rs["gemm_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
        hbm_frac_per_layer_step=wl_bytes / (rs["us_per_layer"] * 1e-6) / 1e9 / HBM_PEAK_GBS)
    log(f"[bench] decode sequential: {rs['tokens_per_s']:.4g} tokens/s ({rs['us_per_layer']:.2f} us "
        f"per layer), gemm launch {rs['gemm_us']:.2f} us")
    for m in (1, 4):
        dm = make_decode(torch, tb, si, m, args.layers)
        rm = run_decode_grouped(torch, tb, dm, max(2, args.steps // 2), 1)
        g2 = weight_bytes / (rm["gemm_us"] * 1e-6) / 1e9
        out[f"grouped_M{m}"] = dict(tokens_per_s=rm["tokens_per_s"], gemm_us=rm["gemm_us"],
                                    weight_gbs=g2, hbm_frac=g2 / HBM_PEAK_GBS,
                                    quant_kernel_us=rm["quant_us"])
        log(f"[bench] decode grouped M={m}: {rm['tokens_per_s']:.4g} tokens/s, gemm "
            f"{rm['gemm_us']:.1f} us ({g2:.0f} GB/s on packed weights)")
        del dm
    if not args.no_cpu_baseline:
        import oracle
        out["cpu_baseline"] = cpu_baseline_decode(si, oracle, d, tb, min_seconds=5.0, max_seconds=15.0)
        nthr = oracle.num_threads()
        oracle.set_num_threads(1)
        try:
            out["cpu_baseline_1thread"] = cpu_baseline_decode(si, oracle, d, tb, min_seconds=2.0,
                                                              max_seconds=6.0)
        finally:
            oracle.set_num_threads(nthr)
    del d
    torch.cuda.empty_cache()
    return out


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library runs the layer on one GPU and has no multi-GPU path.", flush=True)
        sys.exit(2)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_pmc:
        return summarize_pmc(args)

    import numpy as np  # noqa: F401
    import torch

    import seeded_inputs as si
    import ternary_weight_bit_bitlinear_amd as tb
    tb.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(torch, args.copy_mib)), flush=True)
        return
    if args.vendor_int8:
        print(json.dumps({"vendor_int8_gemm": vendor_int8(torch)}), flush=True)
        return

    result = {}
    if args.only in (None, "headline"):
        # the headline: all seven linears of the 7B block (configuration 5)
        log("[bench] block (headline): preparing")
        r = run_large(torch, tb, si, 5, args.steps, args.warmup)
        launches = len(r["linears"])
        k2_us = r["gemm_us_per_step"] / launches
        ops_launch = r["ops_per_step"] / launches
        tops = ops_launch / (k2_us * 1e-6) / 1e12
        log(f"[bench] block: {r['tokens_per_s']:.4g} tokens/s, product kernel {tops:.0f} TOP/s "
            f"({100 * tops / INT8_PEAK_TOPS:.1f}% of int8 peak), mean launch {k2_us:.1f} us")
        cpu = None
        if not args.no_cpu_baseline:
            import oracle
            cpu = cpu_baseline_large(si, oracle, 5)
            log(f"[bench] block: cpu oracle {cpu['value']:.4g} tokens/s ({cpu['sample']})")
        result = {
            "metric": METRIC,
            "value": r["tokens_per_s"],
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": r["ms_per_step"],
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "int8",
            "data": "synthetic",
            "config": {"workload": r["workload"], "M": r["M"], "hidden": 4096, "ffn": 8192,
                       "act_bits": 4,
                       "linears": "q, k, v (4096->4096), gate, up (4096->8192): BitLinear on "
                                  "N(0,1) inputs; wo (4096->4096), wdown (8192->4096): H-BitLinear "
                                  "on outlier-heavy inputs",
                       "step": "4 activation-stage launches (q/k/v and gate/up share theirs) + 7 "
                               "product launches, eager on one stream",
                       "tokens_per_s": "M * steps / seconds (a token goes through all seven linears)"},
            "int_tops": r["int_tops"],
            "roofline": {"bound": "mfma", "achieved": tops, "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                         "frac": tops / INT8_PEAK_TOPS,
                         "traffic": recorded_traffic("gemm_tern4_kernel", "block"),
                         "kernel": "gemm_tern4_kernel<true,0>", "launch_us": k2_us,
                         "launches_per_step": launches,
                         "algorithmic_ops_per_launch": ops_launch,
                         "timed_as": "HIP events on the launch stream around every product "
                                     "launch of the timed steps; achieved = the step's 2*M*N*K "
                                     "over the launches' summed durations"},
            "end_to_end_roofline_frac": r["end_to_end_roofline_frac"],
            "quant_share": r["quant_share"],
            "linears": r["linears"],
            "cpu_baseline": cpu,
        }
        torch.cuda.empty_cache()

    if args.only in (None, "decode", "decode_grouped"):
        dec = decode_report(torch, tb, si, args)
        if result:
            result["decode"] = dec
        else:
            g = dec["grouped"]
            result = {"metric": METRIC, "value": g["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "ms_per_step": g["ms_per_step"],
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                      "dtype": "int8", "data": "synthetic", "config": {"workload": g["workload"]},
                      "roofline": g["roofline"], "decode": dec}

    if not args.no_large and args.only in (None, "wo", "wdown", "block_fused", "qkv_states"):
        large = {}
        for name, cfg in (("wo", 3), ("wdown", 4), ("block_fused", 5)):
            if args.only not in (None, name):
                continue
            log(f"[bench] {name}: preparing")
            if name == "block_fused":
                r = run_block_fused(torch, tb, si, args.large_steps, 2)
            else:
                r = run_large(torch, tb, si, cfg, args.large_steps, 2)
                if not args.no_cpu_baseline and args.only is None:
                    import oracle
                    r["cpu_baseline"] = cpu_baseline_large(si, oracle, cfg, rows_max=256)
                    log(f"[bench] {name}: cpu oracle {r['cpu_baseline']['value']:.4g} tokens/s "
                        f"({r['cpu_baseline']['sample']})")
                    if cfg == 3:
                        # configurations 1-3 also get the oracle on one thread
                        nthr = oracle.num_threads()
                        oracle.set_num_threads(1)
                        try:
                            r["cpu_baseline_1thread"] = cpu_baseline_large(si, oracle, cfg, rows_max=16)
                        finally:
                            oracle.set_num_threads(nthr)
                        log(f"[bench] {name}: cpu oracle on one thread "
                            f"{r['cpu_baseline_1thread']['value']:.4g} tokens/s")
            log(f"[bench] {name}: {r['tokens_per_s']:.4g} tokens/s, gemm {r['gemm_int_tops']:.0f} "
                f"TOP/s ({100 * r['gemm_mfma_frac']:.1f}% of int8 peak)")
            large[name] = r
        if args.only in (None, "qkv_states"):
            large["qkv_states"] = r = run_qkv_states(torch, tb, si, args.large_steps)
            log(f"[bench] qkv states: fp32 out {r['fp32']['launch_us']:.1f} us, states fused "
                f"{r['states']['launch_us']:.1f} us")
            large["qkv_states_decode"] = r = run_qkv_states_decode(torch, tb, si, 50)
            log(f"[bench] qkv states at M = {r['M']}: " + ", ".join(
                f"{k} {v['launch_us']:.1f} us" for k, v in r.items() if isinstance(v, dict)))
        if args.only is None:
            log("[bench] activation stage with the RMS norm folded in")
            large["k1_rmsnorm"] = run_k1_rmsnorm(torch, tb, si, 20)
            for nm, v in large["k1_rmsnorm"].items():
                log(f"[bench] k1 {nm}: plain {v['plain']['us']:.1f} us, rmsnorm {v['rmsnorm']['us']:.1f} us")
        if result:
            result["large_m"] = large
        else:
            name, r = next(iter(large.items()))
            result = {"metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                      "steps": args.large_steps, "warmup": 2, "ms_per_step": r["ms_per_step"],
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                      "dtype": "int8", "data": "synthetic", "config": {"workload": r["workload"]},
                      "large_m": large}

    if args.only in (None, "tiny"):
        t = run_tiny(torch, tb, si)
        if not args.no_cpu_baseline:
            import oracle
            t["cpu_baseline"] = cpu_baseline_tiny(si, oracle)
            nthr = oracle.num_threads()
            oracle.set_num_threads(1)
            try:
                t["cpu_baseline_1thread"] = cpu_baseline_tiny(si, oracle, min_seconds=2.0)
            finally:
                oracle.set_num_threads(nthr)
        log(f"[bench] tiny: forward {t['forward_us']:.1f} us")
        if result:
            result["tiny"] = t
        else:
            result = {"metric": METRIC, "value": t["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                      "steps": 50, "warmup": 5, "ms_per_step": t["forward_us"] / 1e3,
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                      "dtype": "int8", "data": "synthetic", "config": {"workload": t["workload"]},
                      "tiny": t}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
