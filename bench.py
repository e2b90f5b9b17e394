"""Benchmark of the UFP4 hot path on one MI355X.

One step = one linear layer's worth of the path on the dense workload
(X 8192x2048 bf16 with 0.5% outlier channels x50, W 8192x2048, dY 8192x8192):
six fused RHT + 4-bit quantizations (X, W, dY row-wise; W, dY, X column-wise;
RTNE on X/W, stochastic rounding on dY; n = 16, 1 x 16 fp32-scale blocks,
E1M2 grid by default) followed by the three block-scaled 4-bit GEMMs
FPROP Y = X W^T, DGRAD dX = dY W, WGRAD dW = dY^T X.

Inputs are synthetic (seeded), resident in HBM before the timed region.
Prints ONE JSON line.  --gpus N > 1 is not supported (one GPU only).
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA (the family the GEMM issues)
FP4_PEAK_TFLOPS = 10100.0     # dense fp4/fp6 MFMA, context only


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--grid", default="e1m2", choices=["e1m2", "int4", "e2m1"])
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--sets", type=int, default=3,
                   help="input buffer sets rotated across steps (defeats the 256 MB MALL)")
    return p.parse_args()


def build_step(U, wl, grid, device):
    X, W, dY = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY"]
    sf, sd, sw = wl.meta["sign_seeds"]
    sr = wl.meta["sr_seed"]
    mk = lambda seed, rnd, stream=0: U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, 16, 16,  # noqa: E731
                                                  sign_seed=seed, sr_seed=sr, sr_stream=stream)
    cfg = {
        "x_row": mk(sf, U.UFP4_RTNE), "w_row": mk(sf, U.UFP4_RTNE),
        "dy_row": mk(sd, U.UFP4_SR, 0), "w_col": mk(sd, U.UFP4_RTNE),
        "dy_col": mk(sw, U.UFP4_SR, 1), "x_col": mk(sw, U.UFP4_RTNE),
    }
    M, K = X.shape
    N = W.shape[0]

    def alloc(P, Kd):
        return (torch.empty((P, Kd // 2), dtype=torch.uint8, device=device),
                torch.empty((P, Kd // 16), dtype=torch.float32, device=device))

    bufs = {"x_row": alloc(M, K), "w_row": alloc(N, K), "dy_row": alloc(M, N),
            "w_col": alloc(K, N), "dy_col": alloc(N, M), "x_col": alloc(K, M)}
    Y = torch.empty((M, N), dtype=torch.float32, device=device)
    dX = torch.empty((M, K), dtype=torch.float32, device=device)
    dW = torch.empty((N, K), dtype=torch.float32, device=device)
    src = {"x_row": (X, 0), "w_row": (W, 0), "dy_row": (dY, 0), "w_col": (W, 1),
           "dy_col": (dY, 1), "x_col": (X, 1)}
    q = {}

    def quant(name, inputs):
        t, along = inputs[name]
        c, s = bufs[name]
        q[name], _ = U.ufp4_rht_quant(t, along, cfg[name], codes=c, scales=s)

    order = ["x_row", "w_row", "dy_row", "w_col", "dy_col", "x_col"]

    def step(inputs, timer=None):
        for name in order:
            if timer:
                timer.begin("quant_" + name)
            quant(name, inputs)
            if timer:
                timer.end("quant_" + name)
        for name, fn, a, b, out in (("fprop", U.ufp4_gemm_fprop, "x_row", "w_row", Y),
                                    ("dgrad", U.ufp4_gemm_dgrad, "dy_row", "w_col", dX),
                                    ("wgrad", U.ufp4_gemm_wgrad, "dy_col", "x_col", dW)):
            if timer:
                timer.begin(name)
            fn(q[a], q[b], out)
            if timer:
                timer.end(name)

    sizes = {"M": M, "K": K, "N": N}
    quant_elems = {"x_row": M * K, "w_row": N * K, "dy_row": M * N, "w_col": N * K,
                   "dy_col": M * N, "x_col": M * K}
    return step, src, sizes, quant_elems


class EventTimer:
    """HIP events on torch's current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = {}
        self.samples = {}

    def begin(self, name):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pending[name] = e

    def end(self, name):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.samples.setdefault(name, []).append((self.pending.pop(name), e))

    def mean_ms(self):
        self.torch.cuda.synchronize()
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.samples.items()}


def cpu_oracle_baseline(grid):
    """The oracle as it stands on a bounded sample of the same workload: the
    dense step restricted to M' = 256 tokens and N' = 256 output features
    (full K = 2048): six quantizations and three fp64 GEMMs."""
    import numpy as np

    import oracle as O
    import workloads
    gi = {"e1m2": 0, "int4": 1, "e2m1": 2}[grid]
    Mp, Np, K = 256, 256, 2048
    wl = workloads.config2("cpu", M=Mp, K=K, N=Np)
    X, W, dY = (workloads.bits(wl.tensors[k]) for k in ("X", "W", "dY"))
    sf, sd, sw = wl.meta["sign_seeds"]
    sr = wl.meta["sr_seed"]
    spec = lambda seed, rnd, st=0: O.QuantSpec(gi, rnd, 0, 1, 16, 16, seed, sr, st)  # noqa: E731
    t0 = time.perf_counter()
    qx = O.quantize(X, 0, spec(sf, 0))
    qw = O.quantize(W, 0, spec(sf, 0))
    qdy = O.quantize(dY, 0, spec(sd, 1, 0))
    qwt = O.quantize(W, 1, spec(sd, 0))
    qdyt = O.quantize(dY, 1, spec(sw, 1, 1))
    qxt = O.quantize(X, 1, spec(sw, 0))
    tq = time.perf_counter() - t0
    deq = lambda r, s: O.dequant(r["codes"], r["scales"], s, r["P"], r["K"])[1]  # noqa: E731
    O.gemm_ref(deq(qx, spec(sf, 0)), deq(qw, spec(sf, 0)))
    O.gemm_ref(deq(qdy, spec(sd, 1)), deq(qwt, spec(sd, 0)))
    O.gemm_ref(deq(qdyt, spec(sw, 1)), deq(qxt, spec(sw, 0)))
    t = time.perf_counter() - t0
    flops = 3 * 2.0 * Mp * Np * K
    qbytes = 2.75 * (2 * Mp * K + 2 * Np * K + 2 * Mp * Np)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"dense step at M'={Mp}, N'={Np}, K={K} (6 quantizations + 3 fp64 GEMMs), "
                      f"{t:.2f} s; quantizer part {qbytes / tq / 1e9:.4f} GB/s on 1 core",
            "quant_GBps": round(qbytes / tq / 1e9, 6), "seconds": round(t, 3),
            "cpu": platform.processor() or platform.machine()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no collectives; see the design notes on sharding)", file=sys.stderr)
        sys.exit(2)
    global torch
    import torch

    import rht_bit_block_amd as U
    import workloads

    device = "cuda"
    grid = {"e1m2": U.UFP4_E1M2, "int4": U.UFP4_INT4, "e2m1": U.UFP4_E2M1}[args.grid]
    sets = []
    for i in range(max(1, args.sets)):
        wl = workloads.config2(device)
        if i:   # distinct buffers with the same contents (defeats cache reuse across steps)
            wl.tensors = {k: v.clone() for k, v in wl.tensors.items()}
        sets.append(wl)
    step, _, sz, quant_elems = build_step(U, sets[0], grid, device)
    inputs = [{"x_row": (s.tensors["X"], 0), "w_row": (s.tensors["W"], 0),
               "dy_row": (s.tensors["dY"], 0), "w_col": (s.tensors["W"], 1),
               "dy_col": (s.tensors["dY"], 1), "x_col": (s.tensors["X"], 1)} for s in sets]
    torch.cuda.synchronize()

    for i in range(args.warmup):
        step(inputs[i % len(inputs)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(inputs[i % len(inputs)])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps

    # per-kernel averages (separate pass, events around every launch)
    timer = EventTimer(torch)
    for i in range(max(5, args.steps // 2)):
        step(inputs[i % len(inputs)], timer)
    per = timer.mean_ms()

    M, K, N = sz["M"], sz["K"], sz["N"]
    gemm_flops = {"fprop": 2.0 * M * N * K, "dgrad": 2.0 * M * K * N, "wgrad": 2.0 * N * K * M}
    total_flops = sum(gemm_flops.values())
    qbytes = {k: 2.75 * v for k, v in quant_elems.items()}  # 2 B in + 0.5 B codes + 0.25 B scales
    gemm_ms = sum(per[k] for k in gemm_flops)
    quant_ms = sum(per["quant_" + k] for k in qbytes)
    kernels = {}
    for k, f in gemm_flops.items():
        kernels[k] = {"ms": round(per[k], 4), "TFLOP/s": round(f / per[k] / 1e9, 2),
                      "frac_bf16_peak": round(f / per[k] / 1e9 / BF16_PEAK_TFLOPS, 4)}
    for k, b in qbytes.items():
        kernels["quant_" + k] = {"ms": round(per["quant_" + k], 4),
                                 "GB/s": round(b / per["quant_" + k] / 1e6, 1),
                                 "frac_hbm_peak": round(b / per["quant_" + k] / 1e6 / HBM_PEAK_GBPS, 4)}
    # dominant kernel: the one with the largest share of the step
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    if dom in gemm_flops:
        ach = gemm_flops[dom] / per[dom] / 1e9
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        ach = qbytes[dom[6:]] / per[dom] / 1e6
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None}
    quant_gbps = sum(qbytes.values()) / quant_ms / 1e6
    value = total_flops / (ms_step * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu:
        try:
            cpu = cpu_oracle_baseline(args.grid)
        except Exception as e:  # report, never fake
            cpu = {"error": repr(e)}

    line = {
        "metric": "fused RHT+4b-quant GB/s and 4-bit GEMM TFLOP/s, % of MI355X roofline",
        "value": round(value, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.grid,
        "dtype_detail": "bf16 in; fp32 rotate/scale/round; 4-bit codes; split-bf16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded torch generators; dense linear-layer tensors)",
        "config": {"workload": f"dense linear layer M={M} K={K} N={N}: 6 fused RHT(n=16)+1x16 "
                               f"{args.grid} quantizations (SR on dY) + FPROP/DGRAD/WGRAD",
                   "global_batch": M, "seq_len": None, "parallelism": "single GPU"},
        "roofline": roof,
        "quant": {"GB/s": round(quant_gbps, 1), "frac_hbm_peak": round(quant_gbps / HBM_PEAK_GBPS, 4),
                  "ms": round(quant_ms, 4), "bytes_per_elem": 2.75},
        "gemm": {"TFLOP/s": round(total_flops / gemm_ms / 1e9, 2),
                 "frac_bf16_peak": round(total_flops / gemm_ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                 "frac_fp4_peak": round(total_flops / gemm_ms / 1e9 / FP4_PEAK_TFLOPS, 4),
                 "ms": round(gemm_ms, 4)},
        "kernels": kernels,
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
