"""Benchmark: W8A8 FP8 linear layers at 8B-model prefill shapes on one MI355X.

Default workload ("prefill"): one step = the four prefill linears of an 8B model at
M = 2048 tokens (QKV 4096->6144, O 4096->4096, gate+up 4096->28672, down 14336->4096), each
as dynamic per-token E4M3FN quantization of its bf16 activations followed by the FP8 GEMM
with the fused diag(s_x) . diag(s_w) epilogue writing bf16. Weights are quantized per
output channel once, before timing (static weights). Inputs are seeded synthetic draws
(module `synthetic`), resident in HBM before the timed region.

Prints one JSON line: throughput in TFLOP/s (2MNK per GEMM, quantize time included), the
GEMM kernel's roofline position (per-launch duration from HIP events on the launch
stream), per-kernel figures, and the CPU oracle timed on a bounded sample.

Other workloads (`--workload decode|blockscaled|mxfp4|all`) print one JSON line each:
  decode       few-token sweep M in {1,8,32,128,512}, K = 4096, N in {4096, 14336}, FP8 and
               SmoothQuant INT8 (smoothing folded offline); weights rotated over >512 MB
               of copies so that no call finds them in the 256 MB last-level cache.
  blockscaled  M = 4096, K = 7168, N = 18432 with 1x128 activation groups and 128x128
               weight blocks (group quantize + block-scaled GEMM timed).
  mxfp4        M = N = K = 8192, MXFP4 operands (MX quantize of X + FP4 GEMM timed).
  w4a16        weight-only INT4 (G = 128, fp16 scales) decode GEMM on bf16 activations,
               M in {1,8,32,128}, K = 4096, N in {4096, 14336}; weights rotated over
               >512 MB of copies.
  nvfp4        the same 8192^3 inputs as NVFP4 (tensor-scale pass + quantize of X, and the
               GEMM on the fp16 matrix cores, timed).
  epilogue     the prefill linears with the full epilogue: + bf16 bias, SiLU, and FP8
               output requantized with a static scale (calibrated once, untimed), against
               the plain bf16 epilogue on the same inputs.
  static       static per-tensor FP8 quantization with the saturation counter and running
               amax, against the dynamic per-token quantizer, on the prefill activations
               (2048 x 4096 and 2048 x 14336).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (INT8: 5000 TOPS)
FP4_PEAK_TFLOPS = 10100.0     # MI355X dense FP4 MFMA
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
FP16_PEAK_TFLOPS = 2500.0     # MI355X dense fp16 / bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fp8_gemm_prefill_8b_traffic.txt")
GEMM_SOURCES = [os.path.join(ROOT, "fp4_w8a8_quantized_amd", "csrc", f)
                for f in ("gemm_pp.hip", "gemm_solo.hip", "common.h")]


def _parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="prefill",
                   choices=["prefill", "msweep", "qsweep", "decode", "blockscaled", "mxfp4", "nvfp4", "w4a16",
                            "epilogue", "static", "all"])
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--cpu-rows", type=int, default=2048,
                   help="tokens per linear in the prefill oracle sample (rows are independent)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB three times (the reference for "
                        "rocprofv3's FETCH_SIZE / WRITE_SIZE) and exit")
    p.add_argument("--traffic-summary", nargs=4, metavar=("COPY_FETCH", "COPY_WRITE", "GEMM_FETCH", "GEMM_WRITE"),
                   help="write the traffic summary from four rocprofv3 counter_collection.csv files "
                        "(copy and prefill runs, FETCH_SIZE then WRITE_SIZE) and exit; no GPU needed")
    p.add_argument("--copy-mib", type=int, default=256, help="size used with --calibrate-copy")
    p.add_argument("--mfma-summary", nargs=4, metavar=("OUT", "TITLE", "COMMAND", "CSV"),
                   help="write a matrix-core utilisation summary from a rocprofv3 --pmc counter_collection.csv "
                        "and exit; no GPU needed")
    return p.parse_args()


QUANT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quantize_per_token_8b_traffic.txt")
QUANT_SOURCES = [os.path.join(ROOT, "fp4_w8a8_quantized_amd", "csrc", f) for f in ("quantize.hip", "common.h")]


def quant_source_hash() -> str:
    h = hashlib.sha256()
    for f in QUANT_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """Per-launch HBM bytes from the committed rocprofv3 counter summary, if it was taken
    on the current GEMM source; None otherwise."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _counter_rows(path):
    """(kernel name, counter value) per dispatch, in dispatch order, from a rocprofv3
    counter_collection.csv."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            val = r.get("Counter_Value") or r.get("Counter-Value")
            did = r.get("Dispatch_Id") or r.get("Dispatch-Id") or len(rows)
            if val is not None:
                rows.append((int(did), name, float(val)))
    return [(n, v) for _, n, v in sorted(rows)]


# the counter passes run `--steps 2 --warmup 1`: GEMM dispatches 4..11 are the two timed steps
TRAFFIC_STEPS, TRAFFIC_WARMUP = 2, 1


def traffic_summary(args):
    """HBM bytes per FP8 GEMM launch of the prefill step from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reports for a plain copy of
    args.copy_mib MiB (which moves exactly that many bytes each way)."""
    import numpy as np
    import synthetic
    cf, cw, gf, gw = args.traffic_summary
    copy_bytes = args.copy_mib * 2**20

    def copy_kib(path):
        v = [x for n, x in _counter_rows(path) if "opy" in n]
        return float(np.median(v)) if v else float("nan")

    def gemm_kib(path):
        nl = len(synthetic.PREFILL_SHAPES)
        v = [x for n, x in _counter_rows(path) if "gemm_pp_kernel" in n or "gemm_solo_kernel" in n]
        v = v[nl * TRAFFIC_WARMUP: nl * (TRAFFIC_WARMUP + TRAFFIC_STEPS)]   # the timed steps
        return float(np.mean(v)), len(v)

    f_scale = copy_bytes / (copy_kib(cf) * 1024.0)
    w_scale = copy_bytes / (copy_kib(cw) * 1024.0)
    fk, nf = gemm_kib(gf)
    wk, nw = gemm_kib(gw)
    fetch = fk * 1024.0 * f_scale
    write = wk * 1024.0 * w_scale
    alg = np.mean([2048 * K + N * K + 2 * 2048 * N for _, K, N in synthetic.PREFILL_SHAPES])
    text = f"""# HBM traffic of the FP8 GEMM in the 8B prefill step (mean per launch over QKV, O, gate+up, down)
# commands (from the repository root, on one MI355X; each --pmc pass in a run of its own):
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_copy_fetch -o copy -- python3 bench.py --calibrate-copy {args.copy_mib}
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_copy_write -o copy -- python3 bench.py --calibrate-copy {args.copy_mib}
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_gemm_fetch -o gemm -- python3 bench.py --steps {TRAFFIC_STEPS} --warmup {TRAFFIC_WARMUP} --no-cpu-baseline
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_gemm_write -o gemm -- python3 bench.py --steps {TRAFFIC_STEPS} --warmup {TRAFFIC_WARMUP} --no-cpu-baseline
#   python3 bench.py --traffic-summary <the four counter_collection.csv files> (this file)
# copy calibration ({args.copy_mib} MiB each way): FETCH_SIZE scale {f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f}
# GEMM dispatches averaged: the {nf} (FETCH_SIZE pass) and {nw} (WRITE_SIZE pass) of the timed steps
# algorithmic bytes per launch (MK + NK + 2MN, mean over the four shapes): {alg:.0f}
gemm_source_sha256_16 = {gemm_source_hash()}
fetch_bytes_per_launch = {fetch:.0f}
write_bytes_per_launch = {write:.0f}
hbm_bytes_per_launch = {fetch + write:.0f}
traffic_over_algorithmic = {(fetch + write) / alg:.3f}
"""
    with open(TRAFFIC_FILE, "w") as f:
        f.write(text)
    print(text)

    # The per-token quantizer in the same runs: median over all of its dispatches (the
    # timed steps, the passes over rotating X copies and the repeated pass on one X).
    def quant_kib(path, tag):
        v = [x for n, x in _counter_rows(path) if tag in n]
        return float(np.median(v)), len(v)

    qlines = []
    for tag, K in (("quant_rows_kernel<2", 4096), ("quant_rows_kernel<7", 14336)):
        qf, nqf = quant_kib(gf, tag)
        qw, nqw = quant_kib(gw, tag)
        fb, wb = qf * 1024.0 * f_scale, qw * 1024.0 * w_scale
        M = 2048
        qlines.append(f"# {tag}> (2048 x {K} bf16 -> E4M3FN): median of {nqf} / {nqw} dispatches\n"
                      f"K{K}_algorithmic_read_bytes = {2 * M * K}\n"
                      f"K{K}_algorithmic_write_bytes = {M * K + 4 * M}\n"
                      f"K{K}_fetch_bytes_per_launch = {fb:.0f}\n"
                      f"K{K}_write_bytes_per_launch = {wb:.0f}\n"
                      f"K{K}_traffic_over_algorithmic = {(fb + wb) / (3 * M * K + 4 * M):.3f}\n")
    qtext = (f"""# HBM traffic of the per-token E4M3FN quantizer (quant_rows_kernel) in the 8B prefill bench
# commands: the four rocprofv3 --pmc runs listed in {os.path.basename(TRAFFIC_FILE)} (copy calibration and
# the prefill bench under FETCH_SIZE, then WRITE_SIZE), then python3 bench.py --traffic-summary <the four csv>
# copy calibration ({args.copy_mib} MiB each way): FETCH_SIZE scale {f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f}
quant_source_sha256_16 = {quant_source_hash()}
""" + "".join(qlines))
    with open(QUANT_TRAFFIC_FILE, "w") as f:
        f.write(qtext)
    print(qtext)


def _counter_table(path):
    """{dispatch id: (kernel name, duration s, {counter: value})} from a rocprofv3
    counter_collection.csv (which carries each dispatch's start and end timestamps)."""
    import csv
    by = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            did = int(r.get("Dispatch_Id") or r.get("Dispatch-Id"))
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            ent = by.setdefault(did, (name, dur, {}))
            ent[2][r.get("Counter_Name") or r.get("Counter-Name")] = float(
                r.get("Counter_Value") or r.get("Counter-Value"))
    return by


# MI355X: 8 XCDs, 32 shader engines, 1024 SIMDs. SQ_VALU_MFMA_BUSY_CYCLES is summed over
# the SIMDs, SQ_BUSY_CYCLES over the shader engines and GRBM_GUI_ACTIVE over the XCDs.
N_XCD, N_SE, N_SIMD = 8, 32, 1024


def mfma_summary(args):
    """Per kernel: FLOPs from the MFMA op counters against 2MNK, the matrix cores' busy
    cycles per SIMD, and the cycles the shader engines had waves, from one rocprofv3 --pmc
    pass (SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE and the MOPS counters)."""
    import numpy as np
    out, title, cmd, path = args.mfma_summary
    by = _counter_table(path)
    groups = {}
    for did, (name, dur, c) in sorted(by.items()):
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in c or c["SQ_VALU_MFMA_BUSY_CYCLES"] <= 0:
            continue
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("w8a8::", "")
        flop = sum(c.get(k, 0.0) for k in ("SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_I8",
                                            "SQ_INSTS_VALU_MFMA_MOPS_F6F4")) * 512
        groups.setdefault((short, flop), []).append((dur, c))
    lines = [f"# {title}",
             "# command (from the repository root, on one MI355X; one --pmc pass in a run of its own):",
             f"#   {cmd}",
             f"#   python3 bench.py --mfma-summary <this file> <title> <command> <counter_collection.csv>",
             "# Counters are summed over instances by rocprofv3: SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs,",
             "# SQ_BUSY_CYCLES over the 32 shader engines, GRBM_GUI_ACTIVE over the 8 XCDs; MOPS counters count",
             "# 512 flops (or int ops) each. Per dispatch, averaged over the dispatches of each kernel:",
             "#   flop            = (SQ_INSTS_VALU_MFMA_MOPS_F8 + _I8 + _F6F4) * 512",
             "#   mfma_busy       = SQ_VALU_MFMA_BUSY_CYCLES / 1024   (matrix-core busy cycles per SIMD)",
             "#   se_busy         = SQ_BUSY_CYCLES / 32               (cycles with waves resident, per shader engine)",
             "#   window          = GRBM_GUI_ACTIVE / 8               (counting window per XCD; it runs a few us past the kernel)",
             "#   busy_of_active  = mfma_busy / se_busy               (matrix cores busy while the kernel's waves were resident)",
             "#   mfma_util       = mfma_busy / window                (rocprofv3's MfmaUtil)",
             "#   se_clock_GHz    = se_busy / duration                (a lower bound on the shader clock during the dispatch)",
             "# Under --pmc every dispatch runs alone, between counter reads, so the clock is not the one of",
             "# back-to-back launches; the bench's clock probe gives that one.",
             "kernel | dispatches | mean_us | flop_per_dispatch | mfma_busy | se_busy | window | busy_of_active | mfma_util | se_clock_GHz"]
    for (short, _), ds in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        dur = np.array([d for d, _ in ds])
        get = lambda k: np.array([c.get(k, 0.0) for _, c in ds])
        flop = (get("SQ_INSTS_VALU_MFMA_MOPS_F8") + get("SQ_INSTS_VALU_MFMA_MOPS_I8")
                + get("SQ_INSTS_VALU_MFMA_MOPS_F6F4")) * 512
        busy = get("SQ_VALU_MFMA_BUSY_CYCLES") / N_SIMD
        seb = get("SQ_BUSY_CYCLES") / N_SE
        win = get("GRBM_GUI_ACTIVE") / N_XCD
        lines.append(f"{short} | {len(ds)} | {dur.mean() * 1e6:.1f} | {flop.mean():.4e} | {busy.mean():.0f} | "
                     f"{seb.mean():.0f} | {win.mean():.0f} | {np.mean(busy / np.maximum(seb, 1)):.3f} | "
                     f"{np.mean(busy / np.maximum(win, 1)):.3f} | {np.mean(seb / dur) / 1e9:.3f}")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    print(text)


def _threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max((i.get("num_threads", 1) for i in threadpool_info()), default=1))
    except Exception:  # pragma: no cover
        return 1


class Ctx:
    """Device, stream and the raw C ABI handle shared by the workloads."""

    def __init__(self):
        import torch
        import fp4_w8a8_quantized_amd as w8
        self.torch, self.w8 = torch, w8
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.L = w8.lib()
        self.stream = torch.cuda.current_stream(self.dev)
        self.sh = self.stream.cuda_stream

    def bf16(self, bits):
        import numpy as np
        return self.torch.from_numpy(bits.view(np.int16)).view(self.torch.bfloat16).to(self.dev)

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def check(self, st):
        assert st == 0, self.w8.status_string(st)


def _base_record(args, metric, value, unit, ms_per_step, dtype, config, higher=True):
    return {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": higher, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "config": config}


SPEC_SCLK_GHZ = 2.4           # the clock the MFMA peaks above are quoted at


def sclk_during(c: Ctx, launch, n: int, window_ms: float = 15.0):
    """Shader clock (GHz) the chip held while `launch(0) .. launch(n - 1)` ran back to back
    on the bench stream: the library's clock probe runs on a second stream (one wave on one
    CU of each XCD), enqueued behind the first launches so that its window falls inside the
    run. A probe that can find no free wave slot starts late; if it ends after the run (an
    event behind it on its stream against one behind the run), its window took in idle time,
    and the run is repeated at twice the length (at most twice more). Returns the median over
    the XCDs and the per-XCD figures."""
    import numpy as np
    torch = c.torch
    out = torch.zeros((16,), dtype=torch.int64, device=c.dev)
    side = torch.cuda.Stream(device=c.dev)
    for attempt in range(3):
        e_start, e_end, e_probe = c.event(), c.event(), c.event()
        torch.cuda.synchronize()
        e_start.record(c.stream)
        for i in range(n):
            launch(i)
            if i == min(2, n - 1):
                c.check(c.L.w8a8_sclk_probe(out.data_ptr(), 8, int(window_ms * 1e5), side.cuda_stream))
                e_probe.record(side)
        e_end.record(c.stream)
        torch.cuda.synchronize()
        if e_start.elapsed_time(e_probe) <= e_start.elapsed_time(e_end):
            break
        n *= 2
    o = out.cpu().numpy().reshape(8, 2).astype(np.float64)
    ghz = o[:, 1] / np.maximum(o[:, 0], 1) * 0.1
    return float(np.median(ghz)), [round(float(g), 3) for g in ghz]


def _launch_mean_s(c: Ctx, fn, reps: int) -> float:
    """Mean duration in seconds of fn(0) .. fn(reps - 1), launched back to back on the bench
    stream between one pair of HIP events. An event recorded between two launches costs a
    gap and a cache flush that the measured kernel would then carry, so none is."""
    e0, e1 = c.event(), c.event()
    c.torch.cuda.synchronize()
    e0.record(c.stream)
    for i in range(reps):
        fn(i)
    e1.record(c.stream)
    c.torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def _graph_mean_s(c: Ctx, fn, reps: int) -> float:
    """Mean duration in seconds of fn(0, s) .. fn(reps - 1, s) captured into one HIP graph on a
    side stream s and replayed once between two HIP events: the kernels back to back with no
    host launch cost between them (a kernel of a few microseconds launched from Python through
    the C ABI is otherwise bounded by the host's launch rate). The library records no memset
    or allocation, so its launches capture as they are."""
    torch = c.torch
    side = torch.cuda.Stream(device=c.dev)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(reps):
                fn(i, side.cuda_stream)
    torch.cuda.synchronize()
    g.replay()                                          # warm: the graph's first launch
    torch.cuda.synchronize()
    e0, e1 = c.event(), c.event()
    e0.record(c.stream)
    g.replay()
    e1.record(c.stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


# ----------------------------------------------------------------------------- prefill
def prefill_cpu_baseline(layers, rows: int):
    """The oracle as it stands on a sample of the same step: `rows` tokens of each linear
    (per-token work is row-independent), weights quantized beforehand (untimed, like the
    GPU path). Returns the record for the JSON line."""
    import numpy as np
    from oracle import gemm as G
    from oracle import quant as Q

    prepared = []
    for name, xb, wb in layers:
        wq, sw = Q.quantize_weight_per_channel_fp8(wb)
        prepared.append((xb[:rows], wq, sw))
    flops = 0.0
    t0 = time.perf_counter()
    for xs, wq, sw in prepared:
        xq, sx = Q.quantize_per_token_fp8(xs)
        y = G.gemm_fp8_ref(xq, sx, wq, sw)
        flops += 2.0 * xs.shape[0] * wq.shape[0] * wq.shape[1]
        np.asarray(y).sum()
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _threads(),
            "kind": "oracle",
            "sample": f"{rows} of 2048 tokens of each of the 4 prefill linears (quantize + fp64 "
                      f"contraction + scales), weights pre-quantized untimed; {dt:.1f} s"}


def run_prefill(args, c: Ctx):
    import numpy as np
    import synthetic
    torch, w8, L, sh, stream = c.torch, c.w8, c.L, c.sh, c.stream

    layers = [synthetic.prefill(i) for i in range(len(synthetic.PREFILL_SHAPES))]
    dl = []
    for name, xb, wb in layers:
        x, w = c.bf16(xb), c.bf16(wb)
        wq, sw = w8.quantize_weight_per_channel(w)             # offline: static weights
        del w
        M, K = x.shape
        N = wq.shape[0]
        xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=c.dev)
        sx = torch.empty((M,), dtype=torch.float32, device=c.dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=c.dev)
        dl.append(dict(name=name, x=x, xq=xq, sx=sx, wq=wq, sw=sw, y=y, M=M, N=N, K=K))
    torch.cuda.synchronize()

    def quant(d, x=None):
        x = d["x"] if x is None else x
        c.check(L.w8a8_quantize_per_token(x.data_ptr(), d["M"], d["K"], 0, d["xq"].data_ptr(),
                                          d["sx"].data_ptr(), sh))

    def gemm(d, wq):
        c.check(L.w8a8_gemm(d["xq"].data_ptr(), d["sx"].data_ptr(), wq.data_ptr(),
                            d["sw"].data_ptr(), d["M"], d["N"], d["K"], 0, d["y"].data_ptr(), sh))

    # weight copies for the per-kernel passes below: at least 600 MB and 10 launches per layer
    copies = []
    for d in dl:
        n = max(10, math.ceil(600e6 / (d["N"] * d["K"])))
        copies.append([d["wq"]] + [d["wq"].clone() for _ in range(n - 1)])
    for _ in range(args.warmup):
        for d in dl:
            quant(d)
            gemm(d, d["wq"])
    torch.cuda.synchronize()

    # timed region: K whole steps and nothing else on the stream
    nl = len(dl)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for d in dl:
            quant(d)
            gemm(d, d["wq"])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    flops_step = sum(2.0 * d["M"] * d["N"] * d["K"] for d in dl)
    value = flops_step * args.steps / elapsed / 1e12
    ms_per_step = elapsed / args.steps * 1e3

    # Per-kernel durations. Each pass launches one kernel back to back between two HIP events
    # (an event between two launches costs a gap and a cache flush). Two untimed steps go
    # first, so that the chip is as warm as in the timed steps and the host has queued the
    # whole pass before the GPU reaches it (short kernels would otherwise wait on launches).
    # The GEMMs rotate over copies of the weights and the quantizer over copies of X (each
    # >600 MB per layer), so that every launch reads its operands from HBM as in the step,
    # where the weight stream pushes X out of the 256 MB last-level cache. A third pass
    # repeats the quantizer on one X, which then stays in that cache, and a fourth runs the
    # library's same-split stream kernel (2 bytes read, 1 written per element, like the
    # quantizer, with no arithmetic) over the same rotating X copies: what HBM gives an
    # elementwise codec at these sizes.
    def spacer():
        for _ in range(2):
            for d in dl:
                quant(d)
                gemm(d, d["wq"])

    def timed_pass(fn, n):
        e0, e1 = c.event(), c.event()
        torch.cuda.synchronize()
        spacer()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n                  # ms per launch

    reps = max(args.steps, 10)
    g_ms, q_ms, qc_ms, cp_ms = [], [], [], []
    for li, d in enumerate(dl):
        g_ms.append(timed_pass(lambda i, d=d, w=copies[li]: gemm(d, w[i]), len(copies[li])))
        xc = [d["x"]] + [d["x"].clone() for _ in range(max(reps, math.ceil(600e6 / d["x"].nbytes)) - 1)]
        q_ms.append(timed_pass(lambda i, d=d, xc=xc: quant(d, xc[i]), len(xc)))
        del xc
        qc_ms.append(timed_pass(lambda i, d=d: quant(d), reps))
        xc = [d["x"]] + [d["x"].clone() for _ in range(max(reps, math.ceil(600e6 / d["x"].nbytes)) - 1)]
        n = d["M"] * d["K"]
        cp_ms.append(timed_pass(lambda i, d=d, xc=xc, n=n: c.check(L.w8a8_stream_probe(
            xc[i % len(xc)].data_ptr(), n, d["xq"].data_ptr(), sh)), len(xc)))
        del xc
    g_ms, q_ms, qc_ms, cp_ms = map(np.array, (g_ms, q_ms, qc_ms, cp_ms))

    # dominant kernel: the FP8 GEMM (algorithmic 2MNK per launch over its mean duration)
    gemm_flops = np.array([2.0 * d["M"] * d["N"] * d["K"] for d in dl])
    achieved = float(gemm_flops.mean() / (g_ms.mean() * 1e-3) / 1e12)
    traffic = measured_traffic()
    # quantize kernel: 2 B read + 1 B written per element + 4 B per row scale
    q_bytes = np.array([3.0 * d["M"] * d["K"] + 4.0 * d["M"] for d in dl])
    q_gbps = float(q_bytes.mean() / (q_ms.mean() * 1e-3) / 1e9)
    qc_gbps = float(q_bytes.mean() / (qc_ms.mean() * 1e-3) / 1e9)
    cp_gbps = float(q_bytes.mean() / (cp_ms.mean() * 1e-3) / 1e9)

    per_layer = {d["name"]: {"M": d["M"], "N": d["N"], "K": d["K"],
                             "gemm_us": round(g_ms[i] * 1e3, 2),
                             "gemm_tflops": round(gemm_flops[i] / (g_ms[i] * 1e-3) / 1e12, 1),
                             "quant_us": round(q_ms[i] * 1e3, 2),
                             "quant_GBps": round(q_bytes[i] / (q_ms[i] * 1e-3) / 1e9, 1),
                             "quant_cached_us": round(qc_ms[i] * 1e3, 2),
                             "stream_same_split_us": round(cp_ms[i] * 1e3, 2)}
                 for i, d in enumerate(dl)}

    rec = _base_record(
        args, "W8A8 FP8 GEMM TFLOP/s (quant+GEMM+epilogue) at 8B shapes; % of FP8 MFMA peak",
        value, "TFLOP/s", ms_per_step, "fp8_e4m3fn",
        {"workload": "8B-style prefill FP8 W8A8 linears, M=2048 tokens, "
                     "(K,N) in {(4096,6144),(4096,4096),(4096,28672),(14336,4096)}, "
                     "per-token/per-channel scales, bf16 out",
         "tokens": 2048, "shapes_KN": [[d["K"], d["N"]] for d in dl]})
    rec["pct_of_fp8_peak"] = round(100.0 * value / FP8_PEAK_TFLOPS, 2)
    rec["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                       "traffic": traffic}
    # The shader clock over a run of the four GEMMs back to back (weights rotated as in the
    # per-kernel passes) and over whole steps, from the clock probe on a second stream.
    nrot = [len(w) for w in copies]
    f_gemm, f_gemm_xcd = sclk_during(c, lambda i: gemm(dl[i % nl], copies[i % nl][(i // nl) % nrot[i % nl]]),
                                     4 * nl * 16)
    f_step, f_step_xcd = sclk_during(c, lambda i: (quant(dl[i % nl]), gemm(dl[i % nl], dl[i % nl]["wq"])),
                                     4 * nl * 16)
    rec["sclk"] = {"gemm_pass_GHz": round(f_gemm, 3), "step_GHz": round(f_step, 3),
                   "gemm_pass_per_xcd_GHz": f_gemm_xcd, "step_per_xcd_GHz": f_step_xcd,
                   "spec_GHz": SPEC_SCLK_GHZ,
                   "method": "w8a8_sclk_probe on a second stream: shader cycles over 100 MHz "
                             "real-time ticks, one wave per XCD, 15 ms window inside the run"}
    rec["pct_of_peak_at_measured_clock"] = round(100.0 * value / (FP8_PEAK_TFLOPS * f_step / SPEC_SCLK_GHZ), 2)
    rec["gemm_frac_at_measured_clock"] = round(achieved / (FP8_PEAK_TFLOPS * f_gemm / SPEC_SCLK_GHZ), 4)
    rec["kernels"] = {"gemm_fp8_mean_us": round(float(g_ms.mean()) * 1e3, 2),
                      "quantize_fp8_mean_us": round(float(q_ms.mean()) * 1e3, 2),
                      "quantize_fp8_GBps": round(q_gbps, 1),
                      "quantize_fp8_hbm_frac": round(q_gbps / HBM_PEAK_GBPS, 4),
                      "quantize_fp8_cached_GBps": round(qc_gbps, 1),
                      "stream_same_split_GBps": round(cp_gbps, 1),
                      "quantize_over_stream": round(q_gbps / cp_gbps, 4),
                      "per_layer": per_layer,
                      "gemm_source_sha256_16": gemm_source_hash()}
    del copies
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = prefill_cpu_baseline(layers, args.cpu_rows)
    return rec


# ----------------------------------------------------------------------------- token sweep
MSWEEP_TOKENS = (2048, 4096, 8192)


def run_msweep(args, c: Ctx):
    """The four 8B linears at M = 2048, 4096 and 8192 tokens: the FP8 GEMM alone (weights
    rotated over >600 MB, behind two untimed launches) and the whole quantize + GEMM pair,
    to show how the fraction of the FP8 peak moves with the token count."""
    import numpy as np
    import synthetic
    torch, w8, L, sh, stream = c.torch, c.w8, c.L, c.sh, c.stream
    per_m, tot_flops, tot_gemm_s = [], 0.0, 0.0
    for M in MSWEEP_TOKENS:
        layers, flops, g_s, pair_s = [], 0.0, 0.0, 0.0
        for i in range(len(synthetic.PREFILL_SHAPES)):
            name, xb, wb = synthetic.prefill(i, M=M)
            x = c.bf16(xb)
            wq, sw = w8.quantize_weight_per_channel(c.bf16(wb))
            del xb, wb
            N, K = wq.shape
            xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=c.dev)
            sx = torch.empty((M,), dtype=torch.float32, device=c.dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=c.dev)
            ws = [wq] + [wq.clone() for _ in range(max(4, math.ceil(600e6 / (N * K))) - 1)]

            def quant():
                c.check(L.w8a8_quantize_per_token(x.data_ptr(), M, K, 0, xq.data_ptr(), sx.data_ptr(), sh))

            def gemm(w):
                c.check(L.w8a8_gemm(xq.data_ptr(), sx.data_ptr(), w.data_ptr(), sw.data_ptr(), M, N, K, 0,
                                    y.data_ptr(), sh))

            quant()
            for w in ws[:2]:
                gemm(w)
            # A first pass sizes the timed ones to about 20 ms each (at least one rotation) and
            # warms the chip after the weight copies; a pass of a few launches read 10-20% slow.
            g0 = _launch_mean_s(c, lambda i, ws=ws: gemm(ws[i]), len(ws))
            reps = max(len(ws), math.ceil(20e-3 / g0))
            g = _launch_mean_s(c, lambda i, ws=ws: gemm(ws[i % len(ws)]), reps)
            pair = _launch_mean_s(c, lambda i, ws=ws: (quant(), gemm(ws[i % len(ws)])), reps)
            f_ghz, _ = sclk_during(c, lambda i, ws=ws: gemm(ws[i % len(ws)]), 4 + math.ceil(25e-3 / g))
            f = 2.0 * M * N * K
            layers.append({"layer": name, "N": N, "K": K, "gemm_us": round(g * 1e6, 1), "sclk_GHz": round(f_ghz, 3),
                           "gemm_frac_at_measured_clock": round(2.0 * M * N * K / g / 1e12 / (FP8_PEAK_TFLOPS * f_ghz / SPEC_SCLK_GHZ), 4),
                           "gemm_tflops": round(f / g / 1e12, 1), "quant_gemm_us": round(pair * 1e6, 1)})
            flops, g_s, pair_s = flops + f, g_s + g, pair_s + pair
            del ws, x, xq, y
            torch.cuda.empty_cache()
        per_m.append({"M": M, "gemm_tflops": round(flops / g_s / 1e12, 1),
                      "gemm_frac": round(flops / g_s / 1e12 / FP8_PEAK_TFLOPS, 4),
                      "quant_gemm_tflops": round(flops / pair_s / 1e12, 1), "layers": layers})
        tot_flops, tot_gemm_s = flops, g_s
    value = per_m[-1]["gemm_tflops"]
    rec = _base_record(args, "FP8 GEMM TFLOP/s at the 8B prefill linears vs tokens (largest M)", value,
                       "TFLOP/s", tot_gemm_s * 1e3, "fp8_e4m3fn",
                       {"workload": "8B-style FP8 W8A8 linears at M in {2048, 4096, 8192} tokens, "
                                    "(K,N) in {(4096,6144),(4096,4096),(4096,28672),(14336,4096)}"})
    rec["roofline"] = {"bound": "mfma", "achieved": round(value, 1), "peak": FP8_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(value / FP8_PEAK_TFLOPS, 4), "traffic": None}
    rec["sweep"] = per_m
    return rec


# ----------------------------------------------------------------------------- quantizer sweep
QSWEEP_M = (2048, 4096, 8192, 16384)
QSWEEP_K = (4096, 14336)


def run_qsweep(args, c: Ctx):
    """The per-token E4M3FN quantizer (and the static per-tensor one) against the
    same-split stream kernel (2 bytes read, 1 byte written per element, the quantizers'
    traffic) at M in {2048 .. 16384} tokens, K in {4096, 14336}: X rotated over copies of at
    least 600 MB, so that every launch reads it from HBM. Inputs: N(0,1) with 0.1% of the
    channels scaled by 50-500, drawn on the device from a seeded generator."""
    torch, L, sh = c.torch, c.L, c.sh
    rows = []
    for K in QSWEEP_K:
        for M in QSWEEP_M:
            gen = torch.Generator(device=c.dev)
            gen.manual_seed(7000 + M + K)
            n = M * K
            copies = max(2, math.ceil(600e6 / (2 * n)))
            ch = torch.randperm(K, generator=gen, device=c.dev)[:max(1, round(0.001 * K))]
            fac = 50.0 * torch.exp(torch.rand(len(ch), generator=gen, device=c.dev) * math.log(10.0))
            xs = []
            for _ in range(copies):
                x = torch.randn((M, K), generator=gen, device=c.dev)
                x[:, ch] *= fac
                xs.append(x.to(torch.bfloat16))
                del x
            q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=c.dev)
            sx = torch.empty((M,), dtype=torch.float32, device=c.dev)
            # the static scale calibrated on every copy, so that nothing saturates: the codec alone
            scale = torch.tensor([max(float(xc.abs().max().float()) for xc in xs) / 448.0],
                                 dtype=torch.float32, device=c.dev)
            sat = torch.zeros((1,), dtype=torch.int32, device=c.dev)
            amax = torch.zeros((1,), dtype=torch.float32, device=c.dev)
            reps = 3 * copies
            for i in range(2 * copies):                      # untimed: clocks and caches settle
                c.check(L.w8a8_quantize_per_token(xs[i % copies].data_ptr(), M, K, 0, q.data_ptr(),
                                                  sx.data_ptr(), sh))
            dyn = _launch_mean_s(c, lambda i: c.check(L.w8a8_quantize_per_token(
                xs[i % copies].data_ptr(), M, K, 0, q.data_ptr(), sx.data_ptr(), sh)), reps)
            sta = _launch_mean_s(c, lambda i: c.check(L.w8a8_quantize_static(
                xs[i % copies].data_ptr(), M, K, 0, scale.data_ptr(), q.data_ptr(), sat.data_ptr(),
                amax.data_ptr(), sh)), reps)
            stream = _launch_mean_s(c, lambda i: c.check(L.w8a8_stream_probe(
                xs[i % copies].data_ptr(), n, q.data_ptr(), sh)), reps)
            byt = 3.0 * n
            rows.append({"M": M, "K": K, "bytes": int(byt + 4 * M),
                         "dynamic_us": round(dyn * 1e6, 2), "dynamic_GBps": round((byt + 4 * M) / dyn / 1e9, 1),
                         "dynamic_hbm_frac": round((byt + 4 * M) / dyn / 1e9 / HBM_PEAK_GBPS, 4),
                         "static_us": round(sta * 1e6, 2), "static_GBps": round(byt / sta / 1e9, 1),
                         "stream_us": round(stream * 1e6, 2), "stream_GBps": round(byt / stream / 1e9, 1),
                         "dynamic_over_stream": round(stream / dyn, 4)})
            del xs, q
            torch.cuda.empty_cache()
    top = rows[-1]
    rec = _base_record(args, "Per-token E4M3FN quantize HBM GB/s vs tokens (largest M, K=14336)",
                       top["dynamic_GBps"], "GB/s", top["dynamic_us"] / 1e3, "bf16->fp8_e4m3fn",
                       {"workload": "per-token dynamic E4M3FN quantization of bf16 X, M in {2048, 4096, 8192, "
                                    "16384} tokens, K in {4096, 14336}; X rotated over >600 MB of copies"})
    rec["roofline"] = {"bound": "hbm", "achieved": top["dynamic_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": top["dynamic_hbm_frac"], "traffic": None}
    rec["sweep"] = rows
    return rec


# ----------------------------------------------------------------------------- epilogue
def run_epilogue(args, c: Ctx):
    """Prefill linears: quantize + GEMM with bias, SiLU and FP8 output vs the plain GEMM."""
    import numpy as np
    import synthetic
    torch, w8, L, sh = c.torch, c.w8, c.L, c.sh
    dl = []
    for i in range(len(synthetic.PREFILL_SHAPES)):
        name, xb, wb = synthetic.prefill(i)
        x, w = c.bf16(xb), c.bf16(wb)
        wq, sw = w8.quantize_weight_per_channel(w)
        del w
        M, K = x.shape
        N = wq.shape[0]
        xq, sx = w8.quantize_per_token(x)
        rng = np.random.default_rng(1000 + i)
        bias = c.bf16(synthetic.to_bf16_bits(rng.standard_normal(N) * 0.1))
        y0 = w8.gemm(xq, sx, wq, sw)                          # calibration of the static scale
        s_out = float(torch.nn.functional.silu(y0.float() + bias.float()).abs().max()) / 448.0
        y8 = torch.empty((M, N), dtype=torch.float8_e4m3fn, device=c.dev)
        dl.append(dict(name=name, x=x, xq=xq, sx=sx, wq=wq, sw=sw, y0=y0, y8=y8, bias=bias,
                       s_out=s_out, M=M, N=N, K=K))
    torch.cuda.synchronize()

    def quant(d):
        c.check(L.w8a8_quantize_per_token(d["x"].data_ptr(), d["M"], d["K"], 0, d["xq"].data_ptr(),
                                          d["sx"].data_ptr(), sh))

    def plain(d):
        c.check(L.w8a8_gemm(d["xq"].data_ptr(), d["sx"].data_ptr(), d["wq"].data_ptr(), d["sw"].data_ptr(),
                            d["M"], d["N"], d["K"], 0, d["y0"].data_ptr(), sh))

    def full(d):
        c.check(L.w8a8_gemm_ex(d["xq"].data_ptr(), d["sx"].data_ptr(), d["wq"].data_ptr(), d["sw"].data_ptr(),
                               d["M"], d["N"], d["K"], 0, d["bias"].data_ptr(), 2, 1, d["s_out"],
                               d["y8"].data_ptr(), sh))

    res = {}
    for tag, fn in (("plain_bf16", plain), ("bias_silu_fp8", full)):
        per = {}
        tot_g, tot_w = 0.0, 0.0
        for d in dl:
            wall, q_s, g_s = _timed_pair(args, c, lambda d=d: quant(d), lambda d=d, fn=fn: fn(d))
            per[d["name"]] = round(2.0 * d["M"] * d["N"] * d["K"] / g_s / 1e12, 1)
            tot_g += g_s
            tot_w += wall
        res[tag] = {"gemm_tflops_per_layer": per, "gemm_us_total": round(tot_g * 1e6, 1),
                    "step_ms": round(tot_w * 1e3, 4)}
    flops = sum(2.0 * d["M"] * d["N"] * d["K"] for d in dl)
    g_full = res["bias_silu_fp8"]["gemm_us_total"] * 1e-6
    achieved = flops / len(dl) / (g_full / len(dl)) / 1e12
    rec = _base_record(args, "W8A8 FP8 GEMM TFLOP/s with bias + SiLU + FP8 requantized output, 8B prefill",
                       flops / (res["bias_silu_fp8"]["step_ms"] * 1e-3) / 1e12, "TFLOP/s",
                       res["bias_silu_fp8"]["step_ms"], "fp8_e4m3fn",
                       {"workload": "8B-style prefill FP8 W8A8 linears at M=2048 with the full epilogue "
                                    "(bf16 bias, SiLU, E4M3FN output with a static scale)", "tokens": 2048})
    rec["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": None}
    rec["variants"] = res
    return rec


# ----------------------------------------------------------------------------- static
def run_static(args, c: Ctx):
    """Static per-tensor quantize (+ saturation count + amax) vs dynamic per-token."""
    import numpy as np
    import synthetic
    torch, L, sh = c.torch, c.L, c.sh
    rows = []
    for i in (0, 3):                                    # K = 4096 and K = 14336 activations
        name, xb, _ = synthetic.prefill(i, n_limit=1)
        x = c.bf16(xb)
        M, K = x.shape
        q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=c.dev)
        sx = torch.empty((M,), dtype=torch.float32, device=c.dev)
        amax0 = float(x.float().abs().max())
        scale = torch.tensor([amax0 / 448.0 / 2], dtype=torch.float32, device=c.dev)  # saturates the top
        sat = torch.zeros((1,), dtype=torch.int32, device=c.dev)
        amax = torch.zeros((1,), dtype=torch.float32, device=c.dev)

        def dyn():
            c.check(L.w8a8_quantize_per_token(x.data_ptr(), M, K, 0, q.data_ptr(), sx.data_ptr(), sh))

        def sta():
            c.check(L.w8a8_quantize_static(x.data_ptr(), M, K, 0, scale.data_ptr(), q.data_ptr(),
                                           sat.data_ptr(), amax.data_ptr(), sh))

        _, d_s, s_s = _timed_pair(args, c, dyn, sta)
        byt = 3.0 * M * K
        rows.append({"name": name, "M": M, "K": K, "dynamic_us": round(d_s * 1e6, 2),
                     "static_us": round(s_s * 1e6, 2),
                     "dynamic_GBps": round((byt + 4 * M) / d_s / 1e9, 1),
                     "static_GBps": round(byt / s_s / 1e9, 1),
                     "saturated_per_call": int(sat.item()) // (args.steps + args.warmup)})
    tot_b = sum(3.0 * r["M"] * r["K"] for r in rows)
    tot_s = sum(r["static_us"] for r in rows) * 1e-6
    achieved = tot_b / tot_s / 1e9
    rec = _base_record(args, "Static per-tensor FP8 quantize with saturation monitor, HBM GB/s",
                       achieved, "GB/s", tot_s * 1e3, "fp8_e4m3fn",
                       {"workload": "prefill activations 2048x4096 and 2048x14336, one static scale "
                                    "(set to half the tensor amax / 448, so the top values saturate), "
                                    "saturation counter and running amax on"})
    rec["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                       "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None}
    rec["cases"] = rows
    return rec


# ----------------------------------------------------------------------------- decode
def decode_cpu_baseline():
    """Oracle on the M = 8, N = 4096 decode case, FP8 path (quantize + fp64 contraction)."""
    import numpy as np
    import synthetic
    from oracle import gemm as G
    from oracle import quant as Q
    x = synthetic.decode_x()[:8]
    wq, sw = Q.quantize_weight_per_channel_fp8(synthetic.decode_w(4096))
    reps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < 2.0:
        xq, sx = Q.quantize_per_token_fp8(x)
        np.asarray(G.gemm_fp8_ref(xq, sx, wq, sw)).sum()
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    byt = 4096 * 4096 + 8 * 4096 + 2 * 8 * 4096
    return {"value": round(byt / dt / 1e9, 3), "unit": "GB/s", "cores": _threads(), "kind": "oracle",
            "sample": f"M=8, N=4096, K=4096 FP8 (quantize + fp64 contraction + scales), "
                      f"weights pre-quantized; {reps} repetitions, {dt * 1e3:.1f} ms each"}


def run_decode(args, c: Ctx):
    import numpy as np
    import synthetic
    torch, w8, L, sh, stream = c.torch, c.w8, c.L, c.sh, c.stream
    K = synthetic.DECODE_K
    xall = c.bf16(synthetic.decode_x())
    xcal = c.bf16(synthetic.decode_calibration())
    cases = []
    for N in synthetic.DECODE_NS:
        w = c.bf16(synthetic.decode_w(N))
        wq8, sw8 = w8.quantize_weight_per_channel(w)
        s = w8.smoothquant_scales(w8.channel_absmax(xcal), w8.channel_absmax(w), 0.5)
        wqi, swi = w8.quantize_weight_per_channel(w8.smooth_apply(w, s, "weight"), "int8")
        xh = w8.smooth_apply(xall, s, "activation")   # folded into the previous layer offline
        del w
        copies = max(2, math.ceil(600e6 / (N * K)))
        weights = {0: ([wq8] + [wq8.clone() for _ in range(copies - 1)], sw8, xall),
                   1: ([wqi] + [wqi.clone() for _ in range(copies - 1)], swi, xh)}
        torch.cuda.synchronize()
        for M in synthetic.DECODE_MS:
            for fmt in (0, 1):
                ws, sw, xsrc = weights[fmt]
                x = xsrc[:M]
                xq = torch.empty((M, K), dtype=torch.float8_e4m3fn if fmt == 0 else torch.int8, device=c.dev)
                sx = torch.empty((M,), dtype=torch.float32, device=c.dev)
                y = torch.empty((M, N), dtype=torch.bfloat16, device=c.dev)

                def quant(i, s=sh):
                    c.check(L.w8a8_quantize_per_token(x.data_ptr(), M, K, fmt, xq.data_ptr(), sx.data_ptr(), s))

                def gemm(i, s=sh):
                    c.check(L.w8a8_gemm(xq.data_ptr(), sx.data_ptr(), ws[i % copies].data_ptr(),
                                        sw.data_ptr(), M, N, K, fmt, y.data_ptr(), s))

                for i in range(max(args.warmup, 3)):
                    quant(i)
                    gemm(i)
                def lin(i, s=sh):
                    c.check(L.w8a8_linear(x.data_ptr(), ws[i % copies].data_ptr(), sw.data_ptr(), M, N, K, fmt,
                                          xq.data_ptr(), sx.data_ptr(), y.data_ptr(), s))

                R = 3 * copies
                q_us = _graph_mean_s(c, quant, R) * 1e6
                g_us = _graph_mean_s(c, gemm, R) * 1e6
                l_us = _graph_mean_s(c, lin, R) * 1e6
                ge_us = _launch_mean_s(c, gemm, R) * 1e6
                byt = N * K + M * K + 2 * M * N + 4 * (M + N)
                flops = 2.0 * M * N * K
                attain = min(FP8_PEAK_TFLOPS, flops / byt * HBM_PEAK_GBPS / 1e3)   # TFLOP/s
                cases.append({"M": M, "N": N, "fmt": "fp8" if fmt == 0 else "int8",
                              "gemm_us": round(g_us, 2), "gemm_eager_us": round(ge_us, 2),
                              "quant_us": round(q_us, 2), "linear_us": round(l_us, 2),
                              "gemm_GBps": round(byt / g_us / 1e3, 1),
                              "gemm_tflops": round(flops / g_us / 1e6, 2),
                              "roofline_frac": round(flops / g_us / 1e6 / attain, 4)})
        del weights
        torch.cuda.empty_cache()
    hbm = [cs for cs in cases if cs["fmt"] == "fp8" and cs["M"] <= 128]
    tot_bytes = sum(cs["N"] * K + cs["M"] * K + 2 * cs["M"] * cs["N"] for cs in hbm)
    tot_us = sum(cs["gemm_us"] for cs in hbm)
    achieved = tot_bytes / tot_us / 1e3
    total_us = sum(cs["gemm_us"] + cs["quant_us"] for cs in cases)
    rec = _base_record(
        args, "W8A8 decode GEMM HBM GB/s (FP8, M<=128, K=4096, N in {4096,14336})", achieved,
        "GB/s", total_us / 1e3, "fp8_e4m3fn+int8",
        {"workload": "decode sweep M in {1,8,32,128,512}, K=4096, N in {4096,14336}; FP8 per-token "
                     "and SmoothQuant INT8 (alpha 0.5, smoothing folded offline); weights rotated "
                     "over >512 MB of copies", "K": K})
    rec["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                       "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None}
    rec["cases"] = cases
    rec["timing"] = ("per case: 3 x (weight copies) launches over rotating weights captured in one HIP graph "
                     "and replayed (gemm_us, quant_us; linear_us: w8a8_linear, the quantizer and the GEMM in one "
                     "call, one fused kernel for one token); gemm_eager_us: the same GEMM launches issued from "
                     "the host back to back")
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = decode_cpu_baseline()
    return rec


# ----------------------------------------------------------------------------- W4A16
def run_w4a16(args, c: Ctx):
    import numpy as np
    import synthetic
    torch, w8, L, sh, stream = c.torch, c.w8, c.L, c.sh, c.stream
    K = synthetic.DECODE_K
    xall = c.bf16(synthetic.decode_x())
    cases = []
    for N in synthetic.DECODE_NS:
        w = c.bf16(synthetic.decode_w(N))
        q, s = w8.quantize_int4(w)
        del w
        wbytes = N * K // 2 + N * (K // 128) * 2
        copies = max(2, math.ceil(600e6 / wbytes))
        qs = [q] + [q.clone() for _ in range(copies - 1)]
        ss = [s] + [s.clone() for _ in range(copies - 1)]
        torch.cuda.synchronize()
        for M in (1, 8, 32, 128):
            x = xall[:M]
            y = torch.empty((M, N), dtype=torch.bfloat16, device=c.dev)

            def launch(i, s=sh):
                c.check(L.w8a8_gemm_w4a16(x.data_ptr(), qs[i % copies].data_ptr(), ss[i % copies].data_ptr(),
                                          M, N, K, y.data_ptr(), s))

            for i in range(max(args.warmup, 3)):
                launch(i)
            g_us = _graph_mean_s(c, launch, 3 * copies) * 1e6
            ge_us = _launch_mean_s(c, launch, 3 * copies) * 1e6
            byt = wbytes + 2 * M * K + 2 * M * N
            flops = 2.0 * M * N * K
            cases.append({"M": M, "N": N, "gemm_us": round(g_us, 2), "gemm_eager_us": round(ge_us, 2),
                          "gemm_GBps": round(byt / g_us / 1e3, 1),
                          "gemm_tflops": round(flops / g_us / 1e6, 3),
                          "hbm_frac": round(byt / g_us / 1e3 / HBM_PEAK_GBPS, 4)})
        del qs, ss
        torch.cuda.empty_cache()
    tot_bytes = sum(cs["gemm_GBps"] * cs["gemm_us"] * 1e3 for cs in cases)
    tot_us = sum(cs["gemm_us"] for cs in cases)
    achieved = tot_bytes / tot_us / 1e3
    rec = _base_record(
        args, "W4A16 decode GEMM HBM GB/s (INT4 G=128 weights, bf16 activations, M<=128, K=4096, "
              "N in {4096,14336})", achieved, "GB/s", tot_us / 1e3, "int4+bf16 (bf16 MFMA)",
        {"workload": "weight-only INT4 decode sweep M in {1,8,32,128}, K=4096, N in {4096,14336}; "
                     "weights rotated over >512 MB of copies", "K": K})
    rec["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                       "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None}
    rec["cases"] = cases
    rec["timing"] = ("per case: 3 x (weight copies) launches over rotating weights captured in one HIP graph "
                     "and replayed (gemm_us); gemm_eager_us: the same launches issued from the host back to back")
    if not args.no_cpu_baseline:
        from oracle import w4a16 as W4
        wb = synthetic.decode_w(4096)
        oq, os_ = W4.quantize_int4_groups(wb)
        xb = synthetic.decode_x()[:32]
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 5.0:
            np.asarray(W4.gemm_w4a16_ref(xb, oq, os_)).sum()
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        byt = 4096 * K // 2 + 4096 * (K // 128) * 2 + 2 * 32 * K + 2 * 32 * 4096
        rec["cpu_baseline"] = {"value": round(byt / dt / 1e9, 3), "unit": "GB/s", "cores": _threads(),
                               "kind": "oracle",
                               "sample": f"M=32, N=4096, K={K} (dequantize + fp64 product), weights "
                                         f"pre-quantized; {reps} runs of {dt:.2f} s"}
    return rec


# ----------------------------------------------------------------------------- block-scaled
def _timed_pair(args, c: Ctx, first, second):
    """Warm up, then time `steps` of first() + second() (nothing else on the stream); then
    each of the two kernels alone, launched back to back. Returns seconds per step and the
    two kernels' mean durations."""
    for _ in range(args.warmup):
        first()
        second()
    c.torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        first()
        second()
    c.torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    a = _launch_mean_s(c, lambda i: first(), args.steps)
    b = _launch_mean_s(c, lambda i: second(), args.steps)
    return wall, a, b


def run_blockscaled(args, c: Ctx):
    import numpy as np
    import synthetic
    torch, w8, L, sh = c.torch, c.w8, c.L, c.sh
    M, K, N = synthetic.BLOCKSCALED_SHAPE
    xb, wb = synthetic.blockscaled()
    x = c.bf16(xb)
    w = c.bf16(wb)
    wq, sw = w8.quantize_weight_block(w)
    del w
    xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=c.dev)
    sx = torch.empty((M, K // 128), dtype=torch.float32, device=c.dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=c.dev)
    torch.cuda.synchronize()
    wall, q_s, g_s = _timed_pair(
        args, c,
        lambda: c.check(L.w8a8_quantize_per_token_group(x.data_ptr(), M, K, xq.data_ptr(), sx.data_ptr(), sh)),
        lambda: c.check(L.w8a8_gemm_blockscaled(xq.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(),
                                                M, N, K, y.data_ptr(), sh)))
    flops = 2.0 * M * N * K
    achieved = flops / g_s / 1e12
    rec = _base_record(args, "Block-scaled FP8 GEMM TFLOP/s (group quant + GEMM), % of FP8 MFMA peak",
                       flops / wall / 1e12, "TFLOP/s", wall * 1e3, "fp8_e4m3fn",
                       {"workload": "1x128 activation groups, 128x128 weight blocks, fp32 promotion "
                                    "per 128-K group", "M": M, "K": K, "N": N})
    rec["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": None}
    f, f_xcd = sclk_during(c, lambda i: c.check(L.w8a8_gemm_blockscaled(
        xq.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(), M, N, K, y.data_ptr(), sh)),
        4 + math.ceil(25e-3 / g_s))
    rec["sclk"] = {"gemm_pass_GHz": round(f, 3), "gemm_pass_per_xcd_GHz": f_xcd, "spec_GHz": SPEC_SCLK_GHZ}
    rec["gemm_frac_at_measured_clock"] = round(achieved / (FP8_PEAK_TFLOPS * f / SPEC_SCLK_GHZ), 4)
    q_bytes = 3.0 * M * K + 4.0 * M * (K // 128)
    rec["kernels"] = {"gemm_us": round(g_s * 1e6, 1), "group_quant_us": round(q_s * 1e6, 1),
                      "group_quant_GBps": round(q_bytes / q_s / 1e9, 1)}
    if not args.no_cpu_baseline:
        from oracle import gemm as G
        from oracle import quant as Q
        rows, cols = 64, 2048
        owq, osw = Q.quantize_weight_block_fp8(wb[:cols])
        t0 = time.perf_counter()
        oxq, osx = Q.quantize_per_token_group_fp8(xb[:rows])
        np.asarray(G.gemm_blockscaled_ref(oxq, osx, owq, osw)).sum()
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(2.0 * rows * cols * K / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": _threads(), "kind": "oracle",
                               "sample": f"{rows} tokens x {cols} outputs x K={K} (group quantize + "
                                         f"per-group fp64 contraction), weights pre-quantized; {dt:.1f} s"}
    return rec


# ----------------------------------------------------------------------------- MXFP4
def run_mxfp4(args, c: Ctx):
    import numpy as np
    import synthetic
    torch, w8, L, sh = c.torch, c.w8, c.L, c.sh
    M, K, N = synthetic.MXFP4_SHAPE
    xb, wb = synthetic.mxfp4()
    x = c.bf16(xb)
    w = c.bf16(wb)
    wq, sw = w8.quantize_mxfp4(w)
    del w
    xq = torch.empty((M, K // 2), dtype=torch.uint8, device=c.dev)
    sx = torch.empty((M, K // 32), dtype=torch.uint8, device=c.dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=c.dev)
    torch.cuda.synchronize()
    wall, q_s, g_s = _timed_pair(
        args, c,
        lambda: c.check(L.w8a8_quantize_mxfp4(x.data_ptr(), M, K, xq.data_ptr(), sx.data_ptr(), sh)),
        lambda: c.check(L.w8a8_gemm_mxfp4(xq.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(),
                                          M, N, K, y.data_ptr(), sh)))
    flops = 2.0 * M * N * K
    achieved = flops / g_s / 1e12
    rec = _base_record(args, "MXFP4 GEMM TFLOP/s (MX quantize + FP4 GEMM), % of FP4 MFMA peak",
                       flops / wall / 1e12, "TFLOP/s", wall * 1e3, "fp4_e2m1+e8m0",
                       {"workload": "OCP MXFP4 operands (E2M1, E8M0 per 32 along K)", "M": M, "K": K, "N": N})
    rec["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP4_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(achieved / FP4_PEAK_TFLOPS, 4), "traffic": None}
    f, f_xcd = sclk_during(c, lambda i: c.check(L.w8a8_gemm_mxfp4(
        xq.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(), M, N, K, y.data_ptr(), sh)),
        4 + math.ceil(25e-3 / g_s))
    rec["sclk"] = {"gemm_pass_GHz": round(f, 3), "gemm_pass_per_xcd_GHz": f_xcd, "spec_GHz": SPEC_SCLK_GHZ}
    rec["gemm_frac_at_measured_clock"] = round(achieved / (FP4_PEAK_TFLOPS * f / SPEC_SCLK_GHZ), 4)
    q_bytes = 2.5 * M * K + M * K / 32
    rec["kernels"] = {"gemm_us": round(g_s * 1e6, 1), "mx_quant_us": round(q_s * 1e6, 1),
                      "mx_quant_GBps": round(q_bytes / q_s / 1e9, 1)}
    if not args.no_cpu_baseline:
        from oracle import gemm as G
        from oracle import quant as Q
        rows, cols = 64, 2048
        owq, osw = Q.quantize_mxfp4(wb[:cols])
        t0 = time.perf_counter()
        oxq, osx = Q.quantize_mxfp4(xb[:rows])
        np.asarray(G.gemm_mxfp4_ref(oxq, osx, owq, osw)).sum()
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(2.0 * rows * cols * K / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": _threads(), "kind": "oracle",
                               "sample": f"{rows} tokens x {cols} outputs x K={K} (MX quantize + fp64 "
                                         f"contraction of decoded blocks), weights pre-quantized; {dt:.1f} s"}
    return rec


# ----------------------------------------------------------------------------- NVFP4
def run_nvfp4(args, c: Ctx):
    import numpy as np
    import synthetic
    torch, w8, L, sh = c.torch, c.w8, c.L, c.sh
    M, K, N = synthetic.MXFP4_SHAPE
    xb, wb = synthetic.mxfp4()
    x = c.bf16(xb)
    w = c.bf16(wb)
    wq, sw, gw = w8.quantize_nvfp4(w)
    del w
    xq = torch.empty((M, K // 2), dtype=torch.uint8, device=c.dev)
    sx = torch.empty((M, K // 16), dtype=torch.uint8, device=c.dev)
    gx = torch.empty((1,), dtype=torch.float32, device=c.dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=c.dev)
    torch.cuda.synchronize()
    wall, q_s, g_s = _timed_pair(
        args, c,
        lambda: c.check(L.w8a8_quantize_nvfp4(x.data_ptr(), M, K, 0, xq.data_ptr(), sx.data_ptr(),
                                              gx.data_ptr(), sh)),
        lambda: c.check(L.w8a8_gemm_nvfp4(xq.data_ptr(), sx.data_ptr(), gx.data_ptr(), wq.data_ptr(),
                                          sw.data_ptr(), gw.data_ptr(), M, N, K, y.data_ptr(), sh)))
    flops = 2.0 * M * N * K
    achieved = flops / g_s / 1e12
    rec = _base_record(args, "NVFP4 GEMM TFLOP/s (tensor-scale + NVFP4 quantize + GEMM), % of fp16 MFMA peak",
                       flops / wall / 1e12, "TFLOP/s", wall * 1e3, "fp4_e2m1+e4m3 (fp16 MFMA)",
                       {"workload": "NVFP4 operands (E2M1, E4M3 scale per 16 along K, fp32 tensor scale), "
                                    "dequantized to fp16 per workgroup", "M": M, "K": K, "N": N})
    rec["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(achieved / FP16_PEAK_TFLOPS, 4), "traffic": None}
    q_bytes = 4.5 * M * K + M * K / 16
    rec["kernels"] = {"gemm_us": round(g_s * 1e6, 1), "nv_quant_us": round(q_s * 1e6, 1),
                      "nv_quant_GBps": round(q_bytes / q_s / 1e9, 1)}
    if not args.no_cpu_baseline:
        from oracle import nvfp4 as NV
        rows, cols = 64, 2048
        gxo = NV.tensor_scale(xb)
        owq, osw, ogw = NV.quantize_nvfp4(wb[:cols])
        t0 = time.perf_counter()
        oxq, osx, _ = NV.quantize_nvfp4(xb[:rows], g=gxo)
        np.asarray(NV.gemm_nvfp4_ref(oxq, osx, gxo, owq, osw, ogw)).sum()
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(2.0 * rows * cols * K / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": _threads(), "kind": "oracle",
                               "sample": f"{rows} tokens x {cols} outputs x K={K} (NVFP4 quantize with the "
                                         f"full tensor's scale + fp64 contraction), weights pre-quantized; "
                                         f"{dt:.1f} s"}
    return rec


def main():
    args = _parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path: the method shards along tokens or output channels with no "
              "exchange, so the per-GPU kernel is what is measured.", file=sys.stderr)
        sys.exit(2)

    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.mfma_summary:
        mfma_summary(args)
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy * 2**20
        src = torch.ones((n,), dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n}), flush=True)
        return
    c = Ctx()
    runs = {"prefill": run_prefill, "msweep": run_msweep, "qsweep": run_qsweep, "decode": run_decode,
            "blockscaled": run_blockscaled,
            "epilogue": run_epilogue, "static": run_static,
            "mxfp4": run_mxfp4, "nvfp4": run_nvfp4, "w4a16": run_w4a16}
    names = list(runs) if args.workload == "all" else [args.workload]
    for name in names:
        rec = runs[name](args, c)
        print(json.dumps(rec), flush=True)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
