"""Benchmark: W8A8 FP8 linear layers at 8B-model prefill shapes on one MI355X.

One step = the four prefill linears of an 8B model at M = 2048 tokens (QKV 4096->6144,
O 4096->4096, gate+up 4096->28672, down 14336->4096), each as dynamic per-token E4M3FN
quantization of its bf16 activations followed by the FP8 GEMM with the fused
diag(s_x) . diag(s_w) epilogue writing bf16. Weights are quantized per output channel
once, before timing (static weights). Inputs are seeded synthetic draws (module
`synthetic`), resident in HBM before the timed region.

Prints one JSON line: throughput in TFLOP/s (2MNK per GEMM, quantize time included), the
GEMM kernel's roofline position (per-launch duration from HIP events on the launch
stream), per-kernel figures, and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fp8_gemm_prefill_8b_traffic.txt")
GEMM_SOURCES = [os.path.join(ROOT, "fp4_w8a8_quantized_amd", "csrc", f)
                for f in ("gemm.hip", "common.h")]


def _parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--cpu-rows", type=int, default=256,
                   help="tokens per linear in the oracle sample (rows are independent)")
    return p.parse_args()


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


def cpu_baseline(layers, rows: int):
    """The oracle as it stands on a sample of the same step: `rows` tokens of each linear
    (per-token work is row-independent), weights quantized beforehand (untimed, like the
    GPU path). Returns the record for the JSON line."""
    import numpy as np
    from oracle import gemm as G
    from oracle import quant as Q

    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
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
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of 2048 tokens of each of the 4 prefill linears (quantize + fp64 "
                      f"contraction + scales), weights pre-quantized untimed; {dt:.1f} s"}


def main():
    args = _parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path: the method shards along tokens or output channels with no "
              "exchange, so the per-GPU kernel is what is measured.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_w8a8_quantized_amd as w8
    import synthetic

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs (host generation, then resident in HBM)
    layers = [synthetic.prefill(i) for i in range(len(synthetic.PREFILL_SHAPES))]
    dl = []
    for name, xb, wb in layers:
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        w = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(dev)
        wq, sw = w8.quantize_weight_per_channel(w)             # offline: static weights
        del w
        M, K = x.shape
        N = wq.shape[0]
        xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
        sx = torch.empty((M,), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        dl.append(dict(name=name, x=x, xq=xq, sx=sx, wq=wq, sw=sw, y=y, M=M, N=N, K=K))
    torch.cuda.synchronize()

    L = w8.lib()
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def launch_layer(d):
        st = L.w8a8_quantize_per_token(d["x"].data_ptr(), d["M"], d["K"], 0, d["xq"].data_ptr(),
                                       d["sx"].data_ptr(), sh)
        assert st == 0, w8.status_string(st)
        st = L.w8a8_gemm(d["xq"].data_ptr(), d["sx"].data_ptr(), d["wq"].data_ptr(),
                         d["sw"].data_ptr(), d["M"], d["N"], d["K"], 0, d["y"].data_ptr(), sh)
        assert st == 0, w8.status_string(st)

    def step():
        for d in dl:
            launch_layer(d)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps, with HIP events around every launch on the launch stream
    nl = len(dl)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(nl)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for li, d in enumerate(dl):
            e0, e1, e2 = ev[s][li]
            e0.record(stream)
            st = L.w8a8_quantize_per_token(d["x"].data_ptr(), d["M"], d["K"], 0, d["xq"].data_ptr(),
                                           d["sx"].data_ptr(), sh)
            assert st == 0
            e1.record(stream)
            st = L.w8a8_gemm(d["xq"].data_ptr(), d["sx"].data_ptr(), d["wq"].data_ptr(),
                             d["sw"].data_ptr(), d["M"], d["N"], d["K"], 0, d["y"].data_ptr(), sh)
            assert st == 0
            e2.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    flops_step = sum(2.0 * d["M"] * d["N"] * d["K"] for d in dl)
    value = flops_step * args.steps / elapsed / 1e12
    ms_per_step = elapsed / args.steps * 1e3

    q_ms = np.zeros(nl)
    g_ms = np.zeros(nl)
    for s in range(args.steps):
        for li in range(nl):
            e0, e1, e2 = ev[s][li]
            q_ms[li] += e0.elapsed_time(e1)
            g_ms[li] += e1.elapsed_time(e2)
    q_ms /= args.steps
    g_ms /= args.steps

    # dominant kernel: the FP8 GEMM (algorithmic 2MNK per launch over its mean duration)
    gemm_flops = np.array([2.0 * d["M"] * d["N"] * d["K"] for d in dl])
    achieved = float(gemm_flops.mean() / (g_ms.mean() * 1e-3) / 1e12)
    traffic = measured_traffic()
    # quantize kernel: 2 B read + 1 B written per element + 4 B per row scale
    q_bytes = np.array([3.0 * d["M"] * d["K"] + 4.0 * d["M"] for d in dl])
    q_gbps = float(q_bytes.mean() / (q_ms.mean() * 1e-3) / 1e9)

    per_layer = {d["name"]: {"M": d["M"], "N": d["N"], "K": d["K"],
                             "gemm_us": round(g_ms[i] * 1e3, 2),
                             "gemm_tflops": round(gemm_flops[i] / (g_ms[i] * 1e-3) / 1e12, 1),
                             "quant_us": round(q_ms[i] * 1e3, 2),
                             "quant_GBps": round(q_bytes[i] / (q_ms[i] * 1e-3) / 1e9, 1)}
                 for i, d in enumerate(dl)}

    rec = {
        "metric": "W8A8 FP8 GEMM TFLOP/s (quant+GEMM+epilogue) at 8B shapes; % of FP8 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn",
        "data": "synthetic",
        "config": {"workload": "8B-style prefill FP8 W8A8 linears, M=2048 tokens, "
                               "(K,N) in {(4096,6144),(4096,4096),(4096,28672),(14336,4096)}, "
                               "per-token/per-channel scales, bf16 out",
                   "tokens": 2048, "shapes_KN": [[d["K"], d["N"]] for d in dl]},
        "pct_of_fp8_peak": round(100.0 * value / FP8_PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": traffic},
        "kernels": {"gemm_fp8_mean_us": round(float(g_ms.mean()) * 1e3, 2),
                    "quantize_fp8_mean_us": round(float(q_ms.mean()) * 1e3, 2),
                    "quantize_fp8_GBps": round(q_gbps, 1),
                    "quantize_fp8_hbm_frac": round(q_gbps / HBM_PEAK_GBPS, 4),
                    "per_layer": per_layer,
                    "gemm_source_sha256_16": gemm_source_hash()},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(layers, args.cpu_rows)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
