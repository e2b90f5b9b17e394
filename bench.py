"""Benchmark of the UFP4 hot path on one MI355X.

One step = one MoE layer of the large-MoE single-GPU share: 16 local
experts, hidden 5120, expert FFN 1536, 32768 tokens routed top-8 uniformly
(262144 token rows, each expert padded to a multiple of 128), INT4 grid,
RHT n = 128 along every GEMM's shared dimension, 1 x 16 fp32-scale blocks,
RTNE on X / W and stochastic rounding on dY.  The step is six library
calls: three dual-axis fused RHT + 4-bit quantizations (one read each of
X_perm, W and dY_perm gives its row-wise copy and its per-expert column-wise
copy: W^T per expert, dY_perm^T and X_perm^T per expert segment -- six
quantized operands) and the three grouped GEMMs FPROP Y_e = X_e W_e^T, DGRAD
dX_e = dY_e W_e and WGRAD dW_e = dY_e^T X_e.

Inputs are synthetic (seeded), resident in HBM before the timed region and
rotated over buffer sets, so no step reads inputs cached by the one before.
Library calls go through the C ABI with prebuilt ctypes arguments (the
binding's allocation and marshalling stay outside the timed region).  Kernel
times are HIP events on the stream the kernels run on (torch's current
stream); per-kernel averages come from back-to-back launches of that call.

Context sections (not the step): the dense linear layer (X 8192x2048, W
8192x2048, dY 8192x8192, n = 16, 1 x 16) in E1M2, INT4 and E2M1; the
FPROP-only 256^3 case (launch-bound); the 64-expert Zipf-routed MoE layer;
the 2D square-block workload (32 x 32 power-of-two blocks on the scaled
matrix cores, its quantizations and transposes); the RHT's cost on one large
tensor (the same quantization with n = 1 and n = 16 ... 128) beside a plain
device copy; quantization diagnostics; and the CPU oracle on a bounded
sample of the step.

Prints ONE JSON line.  --gpus N > 1 is not supported (one GPU only).
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0      # dense fp8 MFMA (the level products of the fp32-scale GEMM)
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA (its scale products)
FP4_PEAK_TFLOPS = 10100.0     # dense fp4 / fp6 MFMA
# What the fp32-scale GEMM can reach at most: per 16-wide K step and 32 x 32
# output tile it needs 16 fp32 fmas (64 VALU cycles at 16 lanes per cycle)
# beside two MFMAs (64 matrix-core cycles), i.e. 16384 MACs per 64 cycles per
# SIMD = 256 x 4 SIMDs x 256 CUs x 2.4 GHz x 2 flops.
RD_CEILING_TFLOPS = 256 * 4 * 256 * 2.4e9 * 2 / 1e12

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per
# dispatch, one counter per run) on the step of this file, scaled by what the
# same counters read for a plain 1 GiB device copy (bench.py --calibrate-copy).
# A figure holds only for the kernel sources it was taken on: their hash is
# recorded and a mismatch reports null.
FETCH_SCALE, WRITE_SCALE = 1048576 / 524299.5, 1048576 / 1048576.0
_GEMM_SRC = ("gemm_rd.hip", "gemm_epilogue.h", "ufp4_internal.h")
_QUANT_SRC = ("quant_core.h", "ufp4_internal.h")
MEASURED_TRAFFIC = {
    # (workload, kernel): (sources, sha256[:16] of them, FETCH_SIZE KiB, WRITE_SIZE KiB)
    ("moe16", "fprop"): (_GEMM_SRC, "7ae132ace46eff1f", 1564996.9, 1590543.6),
    ("moe16", "dgrad"): (_GEMM_SRC, "7ae132ace46eff1f", 717470.9, 5258969.6),
    ("moe16", "wgrad"): (_GEMM_SRC, "7ae132ace46eff1f", 1228766.4, 524362.9),
    ("moe16", "quant_x"): (_QUANT_SRC, "1db68f7e106e33ee", 1314699.2, 2077052.7),
    ("moe16", "quant_w"): (_QUANT_SRC, "1db68f7e106e33ee", 123024.7, 185821.2),
    ("moe16", "quant_dy"): (_QUANT_SRC, "1db68f7e106e33ee", 394842.9, 592626.8),
}


def _src_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "rht_bit_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` as last counted, or None when the
    counters were not taken for it or its sources have changed since."""
    ent = MEASURED_TRAFFIC.get((workload, kernel))
    if ent is None:
        return None
    files, digest, fetch_kib, write_kib = ent
    if _src_hash(files) != digest:
        return None
    return int(round((fetch_kib * FETCH_SCALE + write_kib * WRITE_SCALE) * 1024))


def _timed(torch, fn, reps, stream=None):
    """Average time of fn() over reps back-to-back calls, HIP events on the
    launch stream (after two untimed calls)."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st = stream if stream is not None else torch.cuda.current_stream()
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _raw(U, name, fn, args):
    """A raw C-ABI call that raises on a non-zero status."""
    def call():
        st = fn(*args)
        if st:
            raise RuntimeError(f"{name} failed: {U.ufp4_status_string(st)}")
    return call


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--sets", type=int, default=2,
                   help="input buffer sets rotated across steps (each > the 256 MB MALL)")
    p.add_argument("--only-step", action="store_true",
                   help="time the step and its kernels only (no context sections, no CPU oracle)")
    p.add_argument("--overlap", action="store_true",
                   help="run WGRAD on a second stream beside FPROP and DGRAD (default: the "
                        "step's calls in order on one stream)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-context", action="store_true", help="skip every context section")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain device-to-device copy of 1 GiB five times (known "
                        "bytes, to scale the profiler's FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


class MoELayer:
    """One MoE layer (six quantizations + three grouped GEMMs) as raw C-ABI
    calls with prebuilt ctypes arguments, for each input buffer set.  Used for
    the 16-expert share (the step) and the 64-expert Zipf layer (context)."""

    def __init__(self, U, torch, wl, grid, n, b, nsets=1, dual=True, overlap=False):
        import workloads
        self.U, self.torch = U, torch
        self.stream = torch.cuda.current_stream()
        cs = ctypes.c_void_p(self.stream.cuda_stream)
        # WGRAD needs only the quantized copies, so with overlap it runs on a
        # second stream (default priority) beside FPROP and DGRAD, and the
        # workgroups of each fill the others' partly empty last rounds.  Off by
        # default: the GEMMs split their own half-empty last rounds, and with
        # that the one-stream order measured as fast or faster
        self.side = torch.cuda.Stream() if overlap else None
        ss = ctypes.c_void_p(self.side.cuda_stream) if overlap else None
        self.side_calls = []
        X, W, dYp = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY_perm"]
        self.off = [int(v) for v in wl.meta["offsets"].tolist()]
        self.counts = [int(c) for c in wl.meta["counts"]]
        E, H, F = wl.meta["experts"], wl.meta["hidden"], wl.meta["ffn"]
        self.E, self.H, self.F = E, H, F
        Xp = workloads.gather_rows(X, wl.meta["gather"].to(X.device))
        del X
        base = {"X": Xp, "W": W, "dY": dYp}
        self.sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        T = Xp.shape[0]
        self.T = T
        sf, sd, sw = wl.meta["sign_seeds"]
        sr = wl.meta["sr_seed"]
        mk = lambda seed, rnd, st=0: U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, n,  # noqa: E731
                                                  sign_seed=seed, sr_seed=sr, sr_stream=st)
        woff = [g * F for g in range(E + 1)]
        # (name, tensor, segment offsets or None for row-wise, cfg)
        self.qcalls = [("x_row", "X", None, mk(sf, U.UFP4_RTNE)),
                       ("w_row", "W", None, mk(sf, U.UFP4_RTNE)),
                       ("dy_row", "dY", None, mk(sd, U.UFP4_SR, 0)),
                       ("w_col", "W", woff, mk(sd, U.UFP4_RTNE)),
                       ("dy_col", "dY", self.off, mk(sw, U.UFP4_SR, 1)),
                       ("x_col", "X", self.off, mk(sw, U.UFP4_RTNE))]
        lib = U.lib_handle()
        self.dual = dual
        self.q = {}
        for name, tn, seg, cfg in self.qcalls:
            rows, cols = base[tn].shape
            P, K = (rows, cols) if seg is None else (cols, rows)
            codes = torch.empty(P * K // 2, dtype=torch.uint8, device="cuda")
            scales = torch.empty(P * K // b, dtype=torch.float32, device="cuda")
            self.q[name] = U.QTensor(codes, scales, P, K, cfg)
        self.q["w_col_stacked"] = U.stacked(self.q["w_col"], E)
        self.out = {"fprop": torch.empty((T, F), dtype=torch.float32, device="cuda"),
                    "dgrad": torch.empty((T, H), dtype=torch.float32, device="cuda"),
                    "wgrad": torch.empty((E * F, H), dtype=torch.float32, device="cuda")}
        self._keep = []
        offs = {}
        for key, o in (("tok", self.off), ("w", woff)):
            arr = (ctypes.c_int64 * len(o))(*o)
            self._keep.append(arr)
            offs[key] = arr
        goff = offs["tok"]
        cfgs = {name: cfg for name, _, _, cfg in self.qcalls}
        self.calls = []
        for ts in self.sets:
            calls = []
            # dual: one read of each tensor for its row-wise copy and its
            # per-expert (segmented) column-wise copy
            for k, tn in ((("x", "X"), ("w", "W"), ("dy", "dY")) if dual else ()):
                t, qr, qc = ts[tn], self.q[k + "_row"], self.q[k + "_col"]
                rows, cols = t.shape
                arr = offs["w"] if k == "w" else offs["tok"]
                nseg = len(woff) - 1 if k == "w" else len(self.off) - 1
                args = (ctypes.c_void_p(t.data_ptr()), rows, cols, t.stride(0), arr, nseg,
                        ctypes.byref(cfgs[k + "_row"]), ctypes.byref(cfgs[k + "_col"]),
                        ctypes.c_void_p(qr.codes.data_ptr()), ctypes.c_void_p(qr.scales.data_ptr()),
                        ctypes.c_void_p(qc.codes.data_ptr()), ctypes.c_void_p(qc.scales.data_ptr()), cs)
                calls.append(("quant_" + k, _raw(U, k, lib.ufp4_rht_quant_dual, args)))
            for name, tn, seg, cfg in ([] if dual else self.qcalls):
                t, q = ts[tn], self.q[name]
                rows, cols = t.shape
                if seg is None:
                    args = (ctypes.c_void_p(t.data_ptr()), rows, cols, t.stride(0), 0,
                            ctypes.byref(cfg), ctypes.c_void_p(q.codes.data_ptr()),
                            ctypes.c_void_p(q.scales.data_ptr()), None, cs)
                    calls.append(("quant_" + name, _raw(U, name, lib.ufp4_rht_quant, args)))
                else:
                    arr = offs["w"] if seg is woff else offs["tok"]
                    args = (ctypes.c_void_p(t.data_ptr()), rows, cols, t.stride(0), arr,
                            len(seg) - 1, ctypes.byref(cfg), ctypes.c_void_p(q.codes.data_ptr()),
                            ctypes.c_void_p(q.scales.data_ptr()), cs)
                    calls.append(("quant_" + name,
                                  _raw(U, name, lib.ufp4_rht_quant_segmented, args)))
            for name, a, bq in (("fprop", "x_row", "w_row"), ("dgrad", "dy_row", "w_col_stacked"),
                                ("wgrad", "dy_col", "x_col")):
                qa, qb = self.q[a].c(), self.q[bq].c()
                self._keep += [qa, qb]
                out = self.out[name]
                args = (ctypes.byref(qa), ctypes.byref(qb), E, goff,
                        ctypes.c_void_p(out.data_ptr()), out.stride(0), cs)
                calls.append((name, _raw(U, name, getattr(lib, f"ufp4_gemm_{name}_grouped"), args)))
                if name == "wgrad" and overlap:
                    self.side_calls.append(_raw(U, name, lib.ufp4_gemm_wgrad_grouped, args[:-1] + (ss,)))
            self.calls.append(calls)
        if overlap:
            self.ev_fork, self.ev_join = torch.cuda.Event(), torch.cuda.Event()
        tokens = sum(self.counts)
        self.tokens = tokens
        f = 2.0 * tokens * F * H                 # unpadded token rows
        self.flops = {"fprop": f, "dgrad": f, "wgrad": f}
        if dual:   # bf16 read once, two code and scale sets written
            bpe = 2.0 + 2 * (0.5 + 4.0 / b)
            self.qbytes = {"quant_" + k: bpe * base[tn].numel()
                           for k, tn in (("x", "X"), ("w", "W"), ("dy", "dY"))}
        else:      # bf16 in, 4-bit code, fp32 scale per block
            bpe = 2.0 + 0.5 + 4.0 / b
            self.qbytes = {"quant_" + name: bpe * base[tn].numel() for name, tn, _, _ in self.qcalls}
        self.bpe = bpe

    def step(self, i):
        calls = self.calls[i % len(self.calls)]
        if self.side is None:
            for _, fn in calls:
                fn()
            return
        for name, fn in calls:
            if name == "fprop":   # every quantization is enqueued: fork WGRAD
                self.ev_fork.record(self.stream)
                self.side.wait_event(self.ev_fork)
                self.side_calls[i % len(self.side_calls)]()
            if name != "wgrad":
                fn()
        self.ev_join.record(self.side)
        self.stream.wait_event(self.ev_join)

    def names(self):
        return [c[0] for c in self.calls[0]]

    def time_call(self, idx, reps):
        """Average duration of call idx over reps back-to-back launches
        (rotating input sets), HIP events on the launch stream."""
        k = [0]

        def fn():
            self.calls[k[0] % len(self.calls)][idx][1]()
            k[0] += 1
        return _timed(self.torch, fn, reps, self.stream)


def time_steps(torch, layer, steps, warmup):
    """Warm-up steps, then `steps` steps between a synchronize and HIP events
    on the launch stream: ms per step and the wall time of the timed region."""
    for i in range(warmup):
        layer.step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(layer.stream)
    for i in range(steps):
        layer.step(i)
    e1.record(layer.stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


def kernel_table(layer, per, workload):
    """Per-kernel ms, TFLOP/s or GB/s, fractions of the peaks and HBM bytes
    per launch (as last counted; null if the kernel changed since)."""
    kernels = {}
    for k, f in layer.flops.items():
        tf = f / per[k] / 1e9
        kernels[k] = {"ms": round(per[k], 4), "TFLOP/s": round(tf, 2),
                      "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
                      "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                      "frac_fp4_peak": round(tf / FP4_PEAK_TFLOPS, 4),
                      "traffic_B": measured_traffic(workload, k)}
    for k, nb in layer.qbytes.items():
        gbps = nb / per[k] / 1e6
        kernels[k] = {"ms": round(per[k], 4), "GB/s": round(gbps, 1),
                      "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                      "traffic_B": measured_traffic(workload, k)}
    return kernels


class DenseLayer:
    """The dense linear layer's library calls (X 8192x2048 with 0.5 % outlier
    channels x50, W 8192x2048, dY 8192x8192; n = 16, 1 x 16 fp32 scales):
    three dual-axis quantizations (one read of X, W, dY each, both quantized
    copies; SR on dY) and FPROP / DGRAD / WGRAD, as raw C-ABI calls for each
    input buffer set."""

    def __init__(self, U, torch, grid, nsets):
        import workloads
        self.U, self.torch = U, torch
        self.stream = torch.cuda.current_stream()
        self.side = None   # every GEMM of this layer fills whole rounds of the CUs
        cs = ctypes.c_void_p(self.stream.cuda_stream)
        base = workloads.config2("cuda")
        self.sets = [base.tensors] + [{k: v.clone() for k, v in base.tensors.items()}
                                      for _ in range(nsets - 1)]
        X = base.tensors["X"]
        M, K = X.shape
        N = base.tensors["W"].shape[0]
        self.M, self.K, self.N = M, K, N
        sf, sd, sw = base.meta["sign_seeds"]
        sr = base.meta["sr_seed"]
        mk = lambda seed, rnd, st=0: U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, 16, 16,  # noqa: E731
                                                  sign_seed=seed, sr_seed=sr, sr_stream=st)
        # tensor: (row-wise cfg, column-wise cfg)
        self.cfgs = {"x": ("X", mk(sf, U.UFP4_RTNE), mk(sw, U.UFP4_RTNE)),
                     "w": ("W", mk(sf, U.UFP4_RTNE), mk(sd, U.UFP4_RTNE)),
                     "dy": ("dY", mk(sd, U.UFP4_SR, 0), mk(sw, U.UFP4_SR, 1))}
        lib = U.lib_handle()
        self.q = {}
        for k, (tn, cr, cc) in self.cfgs.items():
            rows, cols = base.tensors[tn].shape
            for side, (P, Kd, cfg) in (("row", (rows, cols, cr)), ("col", (cols, rows, cc))):
                self.q[f"{k}_{side}"] = U.QTensor(
                    torch.empty((P, Kd // 2), dtype=torch.uint8, device="cuda"),
                    torch.empty((P, Kd // 16), dtype=torch.float32, device="cuda"), P, Kd, cfg)
        self.out = {"fprop": torch.empty((M, N), dtype=torch.float32, device="cuda"),
                    "dgrad": torch.empty((M, K), dtype=torch.float32, device="cuda"),
                    "wgrad": torch.empty((N, K), dtype=torch.float32, device="cuda")}
        self._keep = []
        self.calls = []
        for ts in self.sets:
            calls = []
            for k, (tn, cr, cc) in self.cfgs.items():
                t = ts[tn]
                rows, cols = t.shape
                qr, qc = self.q[k + "_row"], self.q[k + "_col"]
                args = (ctypes.c_void_p(t.data_ptr()), rows, cols, t.stride(0), None, 1,
                        ctypes.byref(cr), ctypes.byref(cc), ctypes.c_void_p(qr.codes.data_ptr()),
                        ctypes.c_void_p(qr.scales.data_ptr()), ctypes.c_void_p(qc.codes.data_ptr()),
                        ctypes.c_void_p(qc.scales.data_ptr()), cs)
                calls.append(("quant_" + k, _raw(U, k, lib.ufp4_rht_quant_dual, args)))
            for name, a, b in (("fprop", "x_row", "w_row"), ("dgrad", "dy_row", "w_col"),
                               ("wgrad", "dy_col", "x_col")):
                qa, qb = self.q[a].c(), self.q[b].c()
                self._keep += [qa, qb]
                out = self.out[name]
                args = (ctypes.byref(qa), ctypes.byref(qb), ctypes.c_void_p(out.data_ptr()),
                        out.stride(0), cs)
                calls.append((name, _raw(U, name, getattr(lib, "ufp4_gemm_" + name), args)))
            self.calls.append(calls)
        self.flops = {"fprop": 2.0 * M * N * K, "dgrad": 2.0 * M * K * N, "wgrad": 2.0 * N * K * M}
        # a dual-axis call reads bf16 once and writes two code and scale sets
        self.bpe = 2.0 + 2 * (0.5 + 4.0 / 16)
        self.qbytes = {"quant_" + k: self.bpe * base.tensors[tn].numel()
                       for k, (tn, _, _) in self.cfgs.items()}

    step = MoELayer.step
    names = MoELayer.names
    time_call = MoELayer.time_call


def layer_report(torch, layer, steps, warmup, workload, reps=None):
    """Step time plus the per-kernel table of one layer."""
    ms, wall = time_steps(torch, layer, steps, warmup)
    per = {n: layer.time_call(i, reps or max(10, steps)) for i, n in enumerate(layer.names())}
    kernels = kernel_table(layer, per, workload)
    flops = sum(layer.flops.values())
    gemm_ms = sum(per[k] for k in layer.flops)
    quant_ms = sum(per[k] for k in layer.qbytes)
    qgbps = sum(layer.qbytes.values()) / quant_ms / 1e6
    return {"ms_per_step": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 2),
            "gemm": {"ms": round(gemm_ms, 4), "TFLOP/s": round(flops / gemm_ms / 1e9, 2),
                     "frac_fp8_peak": round(flops / gemm_ms / 1e9 / FP8_PEAK_TFLOPS, 4)},
            "quant": {"ms": round(quant_ms, 4), "GB/s": round(qgbps, 1),
                      "frac_hbm_peak": round(qgbps / HBM_PEAK_GBPS, 4),
                      "bytes_per_elem": layer.bpe},
            "kernels": kernels}, per, wall


def fprop_256(U, torch, reps=50):
    """FPROP only on X, W 256 x 256 (n = 16, 1 x 16, E1M2, RTNE): two fused
    quantizations and one GEMM.  Launch- and cache-bound (0.13M elements,
    3.4e7 flops): reported for completeness, not a roofline point."""
    import workloads
    wl = workloads.config1("cuda")
    X, W = wl.tensors["X"], wl.tensors["W"]
    lib = U.lib_handle()
    cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cfg = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=0)
    qx, _ = U.ufp4_rht_quant(X, 0, cfg)
    qw, _ = U.ufp4_rht_quant(W, 0, cfg)
    Y = torch.empty((256, 256), dtype=torch.float32, device="cuda")
    a, b = qx.c(), qw.c()
    calls = [_raw(U, "quant_x", lib.ufp4_rht_quant,
                  (ctypes.c_void_p(X.data_ptr()), 256, 256, 256, 0, ctypes.byref(cfg),
                   ctypes.c_void_p(qx.codes.data_ptr()), ctypes.c_void_p(qx.scales.data_ptr()), None, cs)),
             _raw(U, "quant_w", lib.ufp4_rht_quant,
                  (ctypes.c_void_p(W.data_ptr()), 256, 256, 256, 0, ctypes.byref(cfg),
                   ctypes.c_void_p(qw.codes.data_ptr()), ctypes.c_void_p(qw.scales.data_ptr()), None, cs)),
             _raw(U, "fprop", lib.ufp4_gemm_fprop,
                  (ctypes.byref(a), ctypes.byref(b), ctypes.c_void_p(Y.data_ptr()), 256, cs))]

    def step():
        for c in calls:
            c()
    ms = _timed(torch, step, reps)
    return {"ms_per_step": round(ms, 4), "TFLOP/s": round(2.0 * 256 ** 3 / ms / 1e9, 3),
            "per_call_ms": [round(_timed(torch, c, reps), 4) for c in calls],
            "note": "launch- and cache-bound (0.13M elements, 3.4e7 flops); not a roofline point"}


def rht_cost(U, torch, reps=10):
    """The RHT's cost inside the fused quantizer: one large bf16 tensor
    (32768 x 8192 N(0,1), seeded) quantized row-wise (RTNE, 1 x 16 fp32
    scales, INT4) with the Hadamard size n = 1 (no rotation) and n = 16, 32,
    64, 128, plus SR at n = 16 and 128, next to a plain 1 GiB device copy
    (torch's, and the library's streaming copy kernel) timed the same way.  GB/s count 2.75 B per element (the copy: 2 B per
    byte copied).  The pages say fusing the RHT into the FP4 quantizer adds
    only a modest overhead (no hardware named); ratio_vs_n1 is that overhead
    here."""
    lib = U.lib_handle()
    cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    g = torch.Generator(device="cuda")
    g.manual_seed(7001)
    rows, cols = 32768, 8192
    x = torch.randn((rows, cols), device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 16), dtype=torch.float32, device="cuda")
    out = {"shape": [rows, cols], "grid": "int4", "block": "1x16 fp32"}
    base = None
    for n, rnd in ((1, U.UFP4_RTNE), (16, U.UFP4_RTNE), (32, U.UFP4_RTNE), (64, U.UFP4_RTNE),
                   (128, U.UFP4_RTNE), (16, U.UFP4_SR), (128, U.UFP4_SR)):
        cfg = U.make_cfg(U.UFP4_INT4, rnd, U.UFP4_SCALE_F32, 1, 16, n, sign_seed=7002, sr_seed=7003)
        args = (ctypes.c_void_p(x.data_ptr()), rows, cols, x.stride(0), 0, ctypes.byref(cfg),
                ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), None, cs)
        ms = _timed(torch, _raw(U, "rht_quant", lib.ufp4_rht_quant, args), reps)
        gbps = 2.75 * rows * cols / ms / 1e6
        name = f"row_{'sr' if rnd else 'rtne'}_n{n}"
        if n == 1:
            base = ms
        out[name] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                     "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                     "ratio_vs_n1": round(ms / base, 3)}
    del x, codes, scales
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = _timed(torch, lambda: dst.copy_(src), reps)
    gbps = 2.0 * n / ms / 1e6
    out["device_copy_1GiB"] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                               "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    args = (ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, cs)
    ms = _timed(torch, _raw(U, "stream_copy", lib.ufp4_stream_copy, args), reps)
    gbps = 2.0 * n / ms / 1e6
    out["stream_copy_1GiB"] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                               "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                               "kernel": "the library's streaming copy (ufp4_stream_copy)"}
    del src, dst
    torch.cuda.empty_cache()
    return out


def square_blocks(U, torch, reps=10):
    """The 2D square-block workload (X 16384x4096, W 4096x4096, dY 16384x4096;
    32 x 32 blocks with power-of-two E8M0 scales, SR, no rotation), E2M1 and
    E1M2: each tensor quantized once (GB/s at 2 B in + 0.5 B codes + 1 B per
    1024 elements), the transposes that give the reused operands, and the
    three GEMMs on the scaled matrix cores.  Also the dense layer's FPROP with
    1 x 32 E8M0 blocks, and in MXFP8 (E4M3 elements) with its quantization."""
    import workloads
    out = {}
    cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = U.lib_handle()

    def gemm_call(name, a, b, c):
        qa, qb = a.c(), b.c()
        keep.extend([qa, qb])
        return _raw(U, name, getattr(lib, "ufp4_gemm_" + name),
                    (ctypes.byref(qa), ctypes.byref(qb), ctypes.c_void_p(c.data_ptr()), c.stride(0), cs))

    def gemm_ws_call(op, a, b, c):
        qa, qb = a.c(), b.c()
        need = U.ufp4_gemm_workspace_bytes(op, a, b)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        keep.extend([qa, qb, ws])
        return _raw(U, "gemm_ws", lib.ufp4_gemm_ws,
                    (op, ctypes.byref(qa), ctypes.byref(qb), 0, None, ctypes.c_void_p(c.data_ptr()),
                     c.stride(0), ctypes.c_void_p(ws.data_ptr()), need, cs))

    keep = []
    wl = workloads.config5("cuda")
    X, W, dY = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY"]
    M, K = X.shape
    N = W.shape[0]
    qbpe = 2.0 + 0.5 + 1.0 / 1024
    for gname, grid in (("e2m1", U.UFP4_E2M1), ("e1m2", U.UFP4_E1M2)):
        mk = lambda st: U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, 32, 32, 1,  # noqa: E731
                                   sr_seed=wl.meta["sr_seed"], sr_stream=st)
        qs = {}
        for tn, t, st in (("x", X, 0), ("w", W, 1), ("dy", dY, 2)):
            cfg = mk(st)
            q, _ = U.ufp4_rht_quant(t, 0, cfg)
            qs[tn] = q
            rows, cols = t.shape
            args = (ctypes.c_void_p(t.data_ptr()), rows, cols, t.stride(0), 0, ctypes.byref(cfg),
                    ctypes.c_void_p(q.codes.data_ptr()), ctypes.c_void_p(q.scales.data_ptr()), None, cs)
            keep.append(cfg)
            ms = _timed(torch, _raw(U, "quant_2d", lib.ufp4_rht_quant, args), reps)
            gbps = qbpe * t.numel() / ms / 1e6
            out[f"quant_2d_{gname}_{tn}_{rows}x{cols}"] = {
                "ms": round(ms, 4), "GB/s": round(gbps, 1),
                "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes_per_elem": round(qbpe, 5)}
        qwt, qxt, qdyt = (U.ufp4_transpose_qtensor(qs[k]) for k in ("w", "x", "dy"))
        for tn, src, dst in (("w", qs["w"], qwt), ("dy", qs["dy"], qdyt)):
            qd = src.c()
            keep.append(qd)
            ms = _timed(torch, _raw(U, "transpose", lib.ufp4_transpose_qtensor,
                                    (ctypes.byref(qd), ctypes.c_void_p(dst.codes.data_ptr()),
                                     ctypes.c_void_p(dst.scales.data_ptr()), cs)), reps)
            nbytes = 2 * (src.codes.numel() + src.scales.numel())
            out[f"transpose_2d_{gname}_{tn}"] = {"ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                                                 "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4)}
        peak = FP4_PEAK_TFLOPS if grid == U.UFP4_E2M1 else FP8_PEAK_TFLOPS
        for name, a, b, shp in (("fprop", qs["x"], qs["w"], (M, N)), ("dgrad", qs["dy"], qwt, (M, K)),
                                ("wgrad", qdyt, qxt, (N, K))):
            c = torch.empty(shp, dtype=torch.float32, device="cuda")
            ms = _timed(torch, gemm_call(name, a, b, c), reps)
            tf = 2.0 * M * N * K / ms / 1e9
            out[f"gemm_2d_{M}x{K}x{N}_{gname}_{name}"] = {
                "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "peak": peak,
                "frac": round(tf / peak, 4),
                "mfma": "v_mfma_scale_f32_32x32x64_f8f6f4 (" + ("FP4" if grid == U.UFP4_E2M1 else "FP8 E4M3") + ")"}
            if grid != U.UFP4_E2M1:   # the same GEMM as FP6 operands (workspace entry point)
                op = {"fprop": U.UFP4_GEMM_FPROP, "dgrad": U.UFP4_GEMM_DGRAD,
                      "wgrad": U.UFP4_GEMM_WGRAD}[name]
                ms = _timed(torch, gemm_ws_call(op, a, b, c), reps)
                tf = 2.0 * M * N * K / ms / 1e9
                out[f"gemm_2d_{M}x{K}x{N}_{gname}_{name}_fp6"] = {
                    "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "peak": FP4_PEAK_TFLOPS,
                    "frac": round(tf / FP4_PEAK_TFLOPS, 4),
                    "mfma": "v_mfma_scale_f32_32x32x64_f8f6f4 (FP6 E2M3; ms includes the "
                            "expansion of both operands into the workspace)"}
            del c
        del qs, qwt, qxt, qdyt
    # 16 x 16 square blocks (E2M1, SR): the quantization of X and FPROP, which
    # runs on the general kernel (the scaled matrix cores take 32-element blocks)
    c16 = U.make_cfg(U.UFP4_E2M1, U.UFP4_SR, U.UFP4_SCALE_POW2, 16, 16, 1,
                     sr_seed=wl.meta["sr_seed"], sr_stream=0)
    keep.append(c16)
    q16 = {}
    for tn, t in (("x", X), ("w", W)):
        q, _ = U.ufp4_rht_quant(t, 0, c16)
        q16[tn] = q
    rows, cols = X.shape
    args = (ctypes.c_void_p(X.data_ptr()), rows, cols, X.stride(0), 0, ctypes.byref(c16),
            ctypes.c_void_p(q16["x"].codes.data_ptr()), ctypes.c_void_p(q16["x"].scales.data_ptr()),
            None, cs)
    ms = _timed(torch, _raw(U, "quant_2d_16", lib.ufp4_rht_quant, args), reps)
    bpe16 = 2.0 + 0.5 + 1.0 / 256
    out[f"quant_2d_16x16_e2m1_x_{rows}x{cols}"] = {
        "ms": round(ms, 4), "GB/s": round(bpe16 * X.numel() / ms / 1e6, 1),
        "frac_hbm_peak": round(bpe16 * X.numel() / ms / 1e6 / HBM_PEAK_GBPS, 4),
        "bytes_per_elem": round(bpe16, 5)}
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ms = _timed(torch, gemm_call("fprop", q16["x"], q16["w"], c), reps)
    tf = 2.0 * M * N * K / ms / 1e9
    out[f"gemm_2d_16x16_{M}x{K}x{N}_e2m1_fprop"] = {
        "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "peak": FP8_PEAK_TFLOPS,
        "frac": round(tf / FP8_PEAK_TFLOPS, 4),
        "mfma": "general kernel: split-bf16 operands on v_mfma_f32_32x32x16_bf16"}
    del c, q16
    del wl, X, W, dY
    torch.cuda.empty_cache()
    wl2 = workloads.config2("cuda")
    X2, W2 = wl2.tensors["X"], wl2.tensors["W"]
    M2, K2 = X2.shape
    N2 = W2.shape[0]
    for gname, grid in (("e2m1", U.UFP4_E2M1), ("e1m2", U.UFP4_E1M2)):
        cfg = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 32, sign_seed=wl2.meta["sign_seeds"][0])
        qx, _ = U.ufp4_rht_quant(X2, 0, cfg)
        qw, _ = U.ufp4_rht_quant(W2, 0, cfg)
        c = torch.empty((M2, N2), dtype=torch.float32, device="cuda")
        ms = _timed(torch, gemm_call("fprop", qx, qw, c), reps)
        tf = 2.0 * M2 * N2 * K2 / ms / 1e9
        peak = FP4_PEAK_TFLOPS if grid == U.UFP4_E2M1 else FP8_PEAK_TFLOPS
        out[f"dense_1x32_e8m0_{M2}x{K2}x{N2}_{gname}_fprop"] = {
            "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "peak": peak, "frac": round(tf / peak, 4)}
        if grid != U.UFP4_E2M1:
            ms = _timed(torch, gemm_ws_call(U.UFP4_GEMM_FPROP, qx, qw, c), reps)
            tf = 2.0 * M2 * N2 * K2 / ms / 1e9
            out[f"dense_1x32_e8m0_{M2}x{K2}x{N2}_{gname}_fprop_fp6"] = {
                "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "peak": FP4_PEAK_TFLOPS,
                "frac": round(tf / FP4_PEAK_TFLOPS, 4)}
    cfg = U.make_cfg(U.UFP4_E4M3, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1)
    qx, _ = U.ufp4_rht_quant(X2, 0, cfg)
    qw, _ = U.ufp4_rht_quant(W2, 0, cfg)
    c = torch.empty((M2, N2), dtype=torch.float32, device="cuda")
    ms = _timed(torch, gemm_call("fprop", qx, qw, c), reps)
    tf = 2.0 * M2 * N2 * K2 / ms / 1e9
    out[f"mxfp8_{M2}x{K2}x{N2}_fprop"] = {
        "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "peak": FP8_PEAK_TFLOPS,
        "frac": round(tf / FP8_PEAK_TFLOPS, 4), "mfma": "v_mfma_scale_f32_32x32x64_f8f6f4 (FP8 E4M3)"}
    qargs = (ctypes.c_void_p(X2.data_ptr()), M2, K2, K2, 0, ctypes.byref(cfg),
             ctypes.c_void_p(qx.codes.data_ptr()), ctypes.c_void_p(qx.scales.data_ptr()), None, cs)
    ms = _timed(torch, _raw(U, "mxfp8 quant", lib.ufp4_rht_quant, qargs), reps)
    nbytes = M2 * K2 * (2 + 1 + 1 / 32)
    out[f"mxfp8_quant_rows_{M2}x{K2}"] = {"ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                                          "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                          "bytes_per_elem": round(2 + 1 + 1 / 32, 4)}
    del wl2, X2, W2, qx, qw, c
    torch.cuda.empty_cache()
    return out


def diagnostics(U, torch, reps=10):
    """Quantization diagnostics on the dense layer's X (context; not part of
    the step): for E2M1 / E1M2 / INT4, without and with the RHT (n = 1, 16),
    RTNE with 1 x 16 fp32 scales -- the fraction of elements on each
    magnitude level, the mean rounding error E[rho(t) - t] per level in grid
    units (bin-asymmetry equation), and FPROP's relative Frobenius error
    against the fp32 product of the unquantized bf16 inputs.  Also the
    level-statistics kernel's time (reads 2 B per element, writes nothing)."""
    import numpy as np
    import workloads
    wl = workloads.config2("cuda")
    X, W = wl.tensors["X"], wl.tensors["W"]
    M, K = X.shape
    ref = X.float() @ W.float().t()
    ref_norm = torch.linalg.vector_norm(ref).item()
    cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = U.lib_handle()
    out = {}
    names = (("e2m1", U.UFP4_E2M1), ("e1m2", U.UFP4_E1M2), ("int4", U.UFP4_INT4))
    stats = torch.empty(16, dtype=torch.int64, device="cuda")
    for gname, grid in names:
        for n in (1, 16):
            cfg = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, n,
                             sign_seed=wl.meta["sign_seeds"][0])
            U.ufp4_quant_diag(X, cfg, stats=stats)
            st = stats.cpu().numpy()
            cnt = st[:8].astype(np.float64)
            util = (cnt / cnt.sum()).round(5).tolist()
            mean = [round(float(st[8 + k]) * 2.0 ** -28 / cnt[k], 6) if cnt[k] else None
                    for k in range(8)]
            qx, _ = U.ufp4_rht_quant(X, 0, cfg)
            qw, _ = U.ufp4_rht_quant(W, 0, cfg)
            y = U.ufp4_gemm_fprop(qx, qw)
            err = torch.linalg.vector_norm(y - ref).item() / ref_norm
            out[f"X_{gname}_n{n}"] = {"level_util": util, "level_mean_err": mean,
                                      "fprop_rel_err_vs_bf16": round(err, 6)}
            del qx, qw, y
    cfg = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=1)
    ws = torch.empty(U.DIAG_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    args = (ctypes.c_void_p(X.data_ptr()), M, K, K, ctypes.byref(cfg),
            ctypes.c_void_p(stats.data_ptr()), ctypes.c_void_p(ws.data_ptr()), cs)
    ms = _timed(torch, _raw(U, "diag", lib.ufp4_quant_diag, args), reps)
    gbps = 2.0 * M * K / ms / 1e6
    out["kernel_e1m2_n16"] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                              "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                              "bytes_per_elem": 2.0}
    del wl, X, W, ref
    torch.cuda.empty_cache()
    return out


def _cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    return model, affinity, blas


def cpu_oracle_baseline():
    """The oracle as it stands on a bounded sample of the step: expert 0 of
    the 16-expert layer restricted to its first 4096 token rows (its own
    operands: X_e 4096 x 5120, W_e 1536 x 5120, dY_e 4096 x 1536), the same
    six quantizations (INT4, n = 128, 1 x 16; SR on dY), six
    dequantizations and the three fp64 GEMMs.  The quantizer is single-
    threaded numpy; the GEMMs use numpy's BLAS thread pool.  value = the
    sample's GEMM flops over its whole time (TFLOP/s, the step's unit)."""
    import oracle as O
    import workloads
    wl = workloads.config4("cpu")
    off = wl.meta["offsets"].tolist()
    L = 4096
    g0 = wl.meta["gather"][off[0]:off[0] + L]
    Xe = workloads.bits(workloads.gather_rows(wl.tensors["X"], g0))
    We = workloads.bits(wl.tensors["W"][:wl.meta["ffn"]])
    dYe = workloads.bits(wl.tensors["dY_perm"][off[0]:off[0] + L])
    del wl
    sf, sd, sw = 4101, 4102, 4103
    sr = 4201
    spec = lambda seed, rnd, st=0: O.QuantSpec(1, rnd, 0, 1, 16, 128, seed, sr, st)  # noqa: E731
    t0 = time.perf_counter()
    qx = O.quantize(Xe, 0, spec(sf, 0))
    qw = O.quantize(We, 0, spec(sf, 0))
    qdy = O.quantize(dYe, 0, spec(sd, 1, 0))
    qwt = O.quantize(We, 1, spec(sd, 0))
    qdyt = O.quantize(dYe, 1, spec(sw, 1, 1))
    qxt = O.quantize(Xe, 1, spec(sw, 0))
    tq = time.perf_counter() - t0
    deq = lambda r, s: O.dequant(r["codes"], r["scales"], s, r["P"], r["K"])[1]  # noqa: E731
    O.gemm_ref(deq(qx, spec(sf, 0)), deq(qw, spec(sf, 0)))
    O.gemm_ref(deq(qdy, spec(sd, 1)), deq(qwt, spec(sd, 0)))
    O.gemm_ref(deq(qdyt, spec(sw, 1)), deq(qxt, spec(sw, 0)))
    t = time.perf_counter() - t0
    H, F = Xe.shape[1], We.shape[0]
    flops = 3 * 2.0 * L * F * H
    qbytes = 2.75 * 2 * (Xe.size + We.size + dYe.size)
    model, affinity, blas = _cpu_info()
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": blas or affinity,
            "kind": "oracle",
            "sample": f"expert 0 of the 16-expert layer, first {L} of its token rows (X_e {L}x{H}, "
                      f"W_e {F}x{H}, dY_e {L}x{F}): 6 quantizations + 6 dequantizations + 3 fp64 "
                      f"GEMMs in {t:.2f} s; the quantizer part ran at {qbytes / tq / 1e9:.4f} GB/s "
                      "(numpy, one thread); value is the sample's GEMM flops over its whole time",
            "seconds": round(t, 3), "quant_seconds": round(tq, 3),
            "quant_GBps": round(qbytes / tq / 1e9, 6),
            "cpu_model": model, "cores_source": "numpy BLAS thread pool (threadpoolctl)"
            if blas else "len(os.sched_getaffinity(0))",
            "sched_getaffinity": affinity}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no collectives; the design notes describe how it would shard)",
              file=sys.stderr)
        sys.exit(2)
    global torch
    import torch

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)
        return

    import rht_bit_block_amd as U
    import workloads

    # ---- the step: the 16-expert MoE layer --------------------------------
    wl = workloads.config4("cuda")
    layer = MoELayer(U, torch, wl, U.UFP4_INT4, 128, 16, nsets=max(1, args.sets),
                     overlap=args.overlap)
    del wl
    torch.cuda.synchronize()
    print(f"[bench] step: 16-expert layer, {layer.T} padded token rows, "
          f"{args.warmup} warm-up + {args.steps} timed steps", file=sys.stderr, flush=True)
    ms_step, wall = time_steps(torch, layer, args.steps, args.warmup)
    per = {n: layer.time_call(i, max(10, args.steps)) for i, n in enumerate(layer.names())}
    kernels = kernel_table(layer, per, "moe16")
    total_flops = sum(layer.flops.values())
    value = total_flops / (ms_step * 1e-3) / 1e12
    gemm_ms = sum(per[k] for k in layer.flops)
    quant_ms = sum(per[k] for k in layer.qbytes)
    quant_gbps = sum(layer.qbytes.values()) / quant_ms / 1e6
    dom = max(layer.flops, key=lambda k: per[k])          # the GEMMs dominate the step
    ach = layer.flops[dom] / per[dom] / 1e9
    roof = {"kernel": dom, "kernel_symbol": "k_gemm_rd<1,16> (grouped along "
            + ("K" if dom == "wgrad" else "rows") + ")",
            "bound": "mfma", "achieved": round(ach, 2), "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / FP8_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("moe16", dom),
            "peak_basis": "FP8 dense MFMA: the level products run on v_mfma_f32_32x32x16_fp8_fp8",
            "frac_bf16_peak": round(ach / BF16_PEAK_TFLOPS, 4),
            "frac_fp4_peak": round(ach / FP4_PEAK_TFLOPS, 4),
            "scheme_ceiling_tflops": round(RD_CEILING_TFLOPS, 1),
            "frac_scheme_ceiling": round(ach / RD_CEILING_TFLOPS, 4)}
    layer_bpe = layer.bpe
    step_info = {"ms_per_step": round(ms_step, 4), "tokens_x_topk": layer.tokens,
                 "padded_rows": layer.T, "experts": layer.E}
    del layer
    torch.cuda.empty_cache()
    print(f"[bench] step {ms_step:.3f} ms, {value:.1f} TFLOP/s", file=sys.stderr, flush=True)

    context = {}
    if not (args.only_step or args.no_context):
        sections = [
            ("dense_layer", lambda: {g: layer_report(torch, DenseLayer(U, torch, gi, 3), 20, 5, "dense")[0]
                                     for g, gi in (("e1m2", U.UFP4_E1M2), ("int4", U.UFP4_INT4),
                                                   ("e2m1", U.UFP4_E2M1))}),
            ("fprop_256", lambda: fprop_256(U, torch)),
            ("moe64_zipf_e1m2_1x32_n32", lambda: layer_report(
                torch, MoELayer(U, torch, workloads.config3("cuda"), U.UFP4_E1M2, 32, 32, nsets=2,
                                overlap=args.overlap),
                10, 3, "moe64")[0]),
            ("square_blocks", lambda: square_blocks(U, torch)),
            ("rht_cost", lambda: rht_cost(U, torch)),
            ("diagnostics", lambda: diagnostics(U, torch)),
        ]
        for name, fn in sections:
            print(f"[bench] context: {name}", file=sys.stderr, flush=True)
            context[name] = fn()
            torch.cuda.empty_cache()

    cpu = None
    if not (args.no_cpu or args.only_step):
        print("[bench] CPU oracle sample", file=sys.stderr, flush=True)
        try:
            cpu = cpu_oracle_baseline()
        except Exception as e:  # report, never fake
            cpu = {"error": repr(e)}

    line = {
        "metric": "fused RHT+4b-quant GB/s and 4-bit GEMM TFLOP/s, % of MI355X roofline",
        "value": round(value, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4",
        "dtype_detail": "bf16 in; fp32 rotate / scale / round; INT4 codes with fp32 block scales; "
                        "GEMM: exact level products (fp8 MFMA) times bf16-piece scale products "
                        "(bf16 MFMA), fp32 fma accumulate",
        "data": "synthetic (seeded torch generators; MoE layer tensors: X N(0,1) with 0.1% entries "
                "x100, W N(0,0.02), dY N(0,1e-3); uniform top-8 routing)",
        "config": {"workload": "large-MoE single-GPU share: 16 experts, hidden 5120, FFN 1536, 32768 "
                               "tokens top-8 (262144 token rows, padded per expert to 128); 3 dual-axis "
                               "fused RHT(n=128)+1x16 INT4 quantizations (6 quantized operands, SR on "
                               "dY) + grouped FPROP/DGRAD/WGRAD",
                   "global_batch": 32768, "seq_len": None, "parallelism": "single GPU",
                   "experts": step_info["experts"], "tokens_x_topk": step_info["tokens_x_topk"],
                   "padded_rows": step_info["padded_rows"], "input_sets": max(1, args.sets),
                   "schedule": ("quantizations, then WGRAD on a second stream beside FPROP and "
                                "DGRAD; the step ends when both streams are done" if args.overlap
                                else "one stream, calls in order")},
        "roofline": roof,
        "quant": {"GB/s": round(quant_gbps, 1), "frac_hbm_peak": round(quant_gbps / HBM_PEAK_GBPS, 4),
                  "ms": round(quant_ms, 4), "bytes_per_elem": round(layer_bpe, 4)},
        "gemm": {"TFLOP/s": round(total_flops / gemm_ms / 1e9, 2),
                 "frac_fp8_peak": round(total_flops / gemm_ms / 1e9 / FP8_PEAK_TFLOPS, 4),
                 "frac_bf16_peak": round(total_flops / gemm_ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                 "frac_fp4_peak": round(total_flops / gemm_ms / 1e9 / FP4_PEAK_TFLOPS, 4),
                 "ms": round(gemm_ms, 4)},
        "kernels": kernels,
        "cpu_baseline": cpu,
        "context": context,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
