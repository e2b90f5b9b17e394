"""Benchmark of the UFP4 hot path on one MI355X.

One step = one linear layer's worth of the path on the dense workload
(X 8192x2048 bf16 with 0.5% outlier channels x50, W 8192x2048, dY 8192x8192):
six fused RHT + 4-bit quantizations (X, W, dY row-wise; W, dY, X column-wise;
RTNE on X/W, stochastic rounding on dY; n = 16, 1 x 16 fp32-scale blocks,
E1M2 grid by default) followed by the three block-scaled 4-bit GEMMs
FPROP Y = X W^T, DGRAD dX = dY W, WGRAD dW = dY^T X.

Inputs are synthetic (seeded), resident in HBM before the timed region, and
rotated over several buffer sets (> the 256 MB last-level cache) so no step
reads inputs cached by the previous one.  Library calls go through the C ABI
with prebuilt ctypes arguments (the Python binding's allocation and
marshalling stay outside the timed region).  Kernel times are HIP events on
the stream the kernels run on (torch's current stream); per-kernel averages
come from back-to-back launches of that call alone.

Prints ONE JSON line.  --gpus N > 1 is not supported (one GPU only).
"""
import argparse
import ctypes
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA (the family the GEMM issues)
FP4_PEAK_TFLOPS = 10100.0     # dense fp4/fp6 MFMA
FP8_PEAK_TFLOPS = 5000.0      # dense fp8 MFMA
QBYTES_PER_ELEM = 2.75        # bf16 in (2) + 4-bit code (0.5) + fp32 scale / 16 (0.25)

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per
# dispatch, one counter per run) on this workload with the E1M2 grid, scaled by
# what the same counters read for a plain 1 GiB device copy (bench.py
# --calibrate-copy).  A figure holds only for the kernel source it was taken
# on: the sources' hash is recorded and a mismatch reports null.
FETCH_SCALE, WRITE_SCALE = 1048576 / 524299.5, 1048576 / 1048576.0
_GEMM_SRC = ("gemm_rd.hip", "gemm_epilogue.h", "ufp4_internal.h")
_QUANT_SRC = ("quant_core.h", "ufp4_internal.h")
MEASURED_TRAFFIC = {
    # kernel: (sources, sha256[:16] of them, FETCH_SIZE KiB, WRITE_SIZE KiB)
    "fprop": (_GEMM_SRC, "03dfb9abdd189341", 68166.2, 262342.5),
    "dgrad": (_GEMM_SRC, "03dfb9abdd189341", 73808.0, 65543.4),
    "wgrad": (_GEMM_SRC, "03dfb9abdd189341", 73808.0, 65543.4),
    "quant_x": (_QUANT_SRC, "85ffe19635535d1d", 16527.7, 31031.3),
    "quant_w": (_QUANT_SRC, "85ffe19635535d1d", 16527.7, 31031.3),
    "quant_dy": (_QUANT_SRC, "85ffe19635535d1d", 65818.6, 126899.7),
}


def measured_traffic(kernel, grid):
    """HBM bytes per launch of `kernel` as last counted, or None when the
    counters were not taken for it or its source has changed since."""
    import hashlib
    ent = MEASURED_TRAFFIC.get(kernel)
    if ent is None or grid != "e1m2":
        return None
    files, digest, fetch_kib, write_kib = ent
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "rht_bit_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != digest:
        return None
    return int(round((fetch_kib * FETCH_SCALE + write_kib * WRITE_SCALE) * 1024))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--grid", default="e1m2", choices=["e1m2", "int4", "e2m1"])
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-mx", action="store_true",
                   help="skip the power-of-two (scaled matrix core) GEMM figures")
    p.add_argument("--streams", type=int, default=1, choices=[1, 2],
                   help="2: run the quantizations FPROP does not need on a second stream")
    p.add_argument("--dual", type=int, default=1, choices=[0, 1],
                   help="1 (default): each of X, W, dY quantized along both axes by one fused "
                        "call; 0: six single-axis calls (bit-identical outputs)")
    p.add_argument("--no-moe", action="store_true",
                   help="skip the grouped (MoE) layer figures")
    p.add_argument("--no-diag", action="store_true",
                   help="skip the quantization diagnostics (level statistics) figures")
    p.add_argument("--no-stream", action="store_true",
                   help="skip the large-tensor streaming quantizer figures and the device-copy reference")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain device-to-device copy of 1 GiB five times (known "
                        "bytes, to scale the profiler's FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--sets", type=int, default=3,
                   help="input buffer sets rotated across steps (defeats the 256 MB MALL)")
    return p.parse_args()


class Workload:
    """The dense layer's 9 library calls, as raw C-ABI calls with prebuilt
    ctypes arguments, for each input buffer set."""

    # With two streams, the quantizations that FPROP does not need (dY row-wise,
    # W, dY and X column-wise) run on a second stream beside X/W row-wise and
    # FPROP; DGRAD waits for them.  Same calls, same bytes, one GPU.
    AUX = ("quant_dy_row", "quant_w_col", "quant_dy_col", "quant_x_col")

    def __init__(self, U, torch, grid, nsets, streams=1, dual=False):
        import workloads
        self.U, self.torch = U, torch
        self.streams = streams
        self.dual = dual
        self.main = torch.cuda.current_stream()
        self.aux = torch.cuda.Stream() if streams == 2 else self.main   # default priority
        base = workloads.config2("cuda")
        self.sets = [base.tensors] + [{k: v.clone() for k, v in base.tensors.items()}
                                      for _ in range(nsets - 1)]
        X = base.tensors["X"]
        self.M, self.K = X.shape
        self.N = base.tensors["W"].shape[0]
        sf, sd, sw = base.meta["sign_seeds"]
        sr = base.meta["sr_seed"]
        mk = lambda seed, rnd, st=0: U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, 16, 16,  # noqa: E731
                                                  sign_seed=seed, sr_seed=sr, sr_stream=st)
        # (name, tensor, along, cfg)
        self.qcalls = [("x_row", "X", 0, mk(sf, U.UFP4_RTNE)), ("w_row", "W", 0, mk(sf, U.UFP4_RTNE)),
                       ("dy_row", "dY", 0, mk(sd, U.UFP4_SR, 0)), ("w_col", "W", 1, mk(sd, U.UFP4_RTNE)),
                       ("dy_col", "dY", 1, mk(sw, U.UFP4_SR, 1)), ("x_col", "X", 1, mk(sw, U.UFP4_RTNE))]
        self.lib = U.lib_handle()
        self.stream = ctypes.c_void_p(self.main.cuda_stream)
        self.aux_stream = ctypes.c_void_p(self.aux.cuda_stream)
        dev = "cuda"
        self.q = {}
        for name, tn, along, cfg in self.qcalls:
            rows, cols = base.tensors[tn].shape
            P, Kd = (cols, rows) if along else (rows, cols)
            codes = torch.empty((P, Kd // 2), dtype=torch.uint8, device=dev)
            scales = torch.empty((P, Kd // 16), dtype=torch.float32, device=dev)
            self.q[name] = U.QTensor(codes, scales, P, Kd, cfg)
        M, K, N = self.M, self.K, self.N
        self.out = {"fprop": torch.empty((M, N), dtype=torch.float32, device=dev),
                    "dgrad": torch.empty((M, K), dtype=torch.float32, device=dev),
                    "wgrad": torch.empty((N, K), dtype=torch.float32, device=dev)}
        self.gcalls = [("fprop", "x_row", "w_row"), ("dgrad", "dy_row", "w_col"),
                       ("wgrad", "dy_col", "x_col")]
        self._keep = []
        self.calls = [self._build_calls(s) for s in self.sets]
        if dual:   # one fused dual-axis call per tensor: bf16 read once, two code sets
            self.elems = {"x": X.numel(), "w": base.tensors["W"].numel(),
                          "dy": base.tensors["dY"].numel()}
            self.qbpe = {k: 2.0 + 2 * (QBYTES_PER_ELEM - 2.0) for k in self.elems}
        else:
            self.elems = {name: base.tensors[tn].numel() for name, tn, _, _ in self.qcalls}
            self.qbpe = {k: QBYTES_PER_ELEM for k in self.elems}
        self.flops = {"fprop": 2.0 * M * N * K, "dgrad": 2.0 * M * K * N, "wgrad": 2.0 * N * K * M}

    def _build_calls(self, tensors):
        lib, calls = self.lib, []
        if self.dual:
            cfgs = {name: cfg for name, _, _, cfg in self.qcalls}
            for name, tn in (("x", "X"), ("w", "W"), ("dy", "dY")):
                t = tensors[tn]
                rows, cols = t.shape
                qr, qc = self.q[name + "_row"], self.q[name + "_col"]
                args = (ctypes.c_void_p(t.data_ptr()), rows, cols, t.stride(0), None, 1,
                        ctypes.byref(cfgs[name + "_row"]), ctypes.byref(cfgs[name + "_col"]),
                        ctypes.c_void_p(qr.codes.data_ptr()), ctypes.c_void_p(qr.scales.data_ptr()),
                        ctypes.c_void_p(qc.codes.data_ptr()), ctypes.c_void_p(qc.scales.data_ptr()),
                        self.stream)
                calls.append(("quant_" + name, lib.ufp4_rht_quant_dual, args))
        for name, tn, along, cfg in ([] if self.dual else self.qcalls):
            t = tensors[tn]
            rows, cols = t.shape
            q = self.q[name]
            st = self.aux_stream if "quant_" + name in self.AUX else self.stream
            args = (ctypes.c_void_p(t.data_ptr()), rows, cols, t.stride(0), along,
                    ctypes.byref(cfg), ctypes.c_void_p(q.codes.data_ptr()),
                    ctypes.c_void_p(q.scales.data_ptr()), None, st)
            calls.append(("quant_" + name, lib.ufp4_rht_quant, args))
        for name, a, b in self.gcalls:
            qa, qb = self.q[a].c(), self.q[b].c()
            self._keep += [qa, qb]
            out = self.out[name]
            fn = getattr(lib, "ufp4_gemm_" + name)
            calls.append((name, fn, (ctypes.byref(qa), ctypes.byref(qb),
                                     ctypes.c_void_p(out.data_ptr()), out.stride(0), self.stream)))
        return calls

    def step(self, i):
        calls = self.calls[i % len(self.calls)]
        if self.streams == 2:
            ev0 = self.torch.cuda.Event()
            ev0.record(self.main)
            self.aux.wait_event(ev0)      # buffers of earlier steps are done with
        for name, fn, args in calls:
            if self.streams == 2 and name == "dgrad":
                ev1 = self.torch.cuda.Event()
                ev1.record(self.aux)
                self.main.wait_event(ev1)
            st = fn(*args)
            if st:
                raise RuntimeError(f"{name} failed: {self.U.ufp4_status_string(st)}")

    def time_call(self, idx, reps):
        """Average duration of call idx over reps back-to-back launches
        (rotating input sets), HIP events on the launch stream."""
        torch = self.torch
        for i in range(2):
            _, fn, args = self.calls[i % len(self.calls)][idx]
            fn(*args)
        torch.cuda.synchronize()
        name = self.calls[0][idx][0]
        st = self.aux if name in self.AUX else self.main   # events on the launch stream
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(reps):
            _, fn, args = self.calls[i % len(self.calls)][idx]
            fn(*args)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps


def single_axis(U, torch, wl, reps=20):
    """The dense layer's six quantizations as single-axis fused calls
    (context; the step uses the dual-axis call): each timed over back-to-back
    launches on the step's rotating input sets, with prebuilt C-ABI
    arguments; GB/s count 2.75 B per element (bf16 in, code, fp32 scale)."""
    lib = U.lib_handle()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    for name, tn, along, cfg in wl.qcalls:
        q = wl.q[name]
        calls = []
        for t in (ts[tn] for ts in wl.sets):
            rows, cols = t.shape
            calls.append((ctypes.c_void_p(t.data_ptr()), rows, cols, t.stride(0), along,
                          ctypes.byref(cfg), ctypes.c_void_p(q.codes.data_ptr()),
                          ctypes.c_void_p(q.scales.data_ptr()), None, stream))
        for a in calls:
            lib.ufp4_rht_quant(*a)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            st = lib.ufp4_rht_quant(*calls[i % len(calls)])
            if st:
                raise RuntimeError(f"{name} failed: {U.ufp4_status_string(st)}")
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbps = QBYTES_PER_ELEM * wl.sets[0][tn].numel() / ms / 1e6
        rnd = "sr" if cfg.rounding == U.UFP4_SR else "rtne"
        out[f"{name}_{rnd}"] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                                "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    return out


def quant_stream(U, torch, reps=10):
    """The row-wise fused quantizer on one large bf16 tensor (32768 x 8192,
    N(0,1) from a seeded generator; n = 16, 1 x 16 fp32 scales, E1M2), RTNE
    and SR, next to a plain 1 GiB device-to-device copy timed the same way:
    what the streaming kernel reaches against what the memory system gives a
    copy on this machine (context; GB/s count 2.75 B per element, the copy 2 B
    per byte copied)."""
    lib = U.lib_handle()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    g = torch.Generator(device="cuda")
    g.manual_seed(7001)
    rows, cols = 32768, 8192
    x = torch.randn((rows, cols), device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 16), dtype=torch.float32, device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {"shape": [rows, cols]}
    for name, rnd in (("row_rtne_n16", U.UFP4_RTNE), ("row_sr_n16", U.UFP4_SR)):
        cfg = U.make_cfg(U.UFP4_E1M2, rnd, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=7002, sr_seed=7003)
        args = (ctypes.c_void_p(x.data_ptr()), rows, cols, x.stride(0), 0, ctypes.byref(cfg),
                ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), None, stream)

        def call(a=args):
            st = lib.ufp4_rht_quant(*a)
            if st:
                raise RuntimeError(f"{name} failed: {U.ufp4_status_string(st)}")
        ms = timed(call)
        gbps = QBYTES_PER_ELEM * rows * cols / ms / 1e6
        out[name] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                     "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    del x, codes, scales
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src))
    gbps = 2.0 * n / ms / 1e6
    out["device_copy_1GiB"] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                               "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    del src, dst
    torch.cuda.empty_cache()
    return out


def mx_gemms(U, torch, reps=10):
    """The GEMMs of the power-of-two configurations on the scaled matrix
    cores, each timed over back-to-back launches (context; not part of the
    step): the square-block layer M=16384 K=4096 N=4096 (32 x 32 E8M0 blocks,
    W quantized once and reused transposed, SR, no rotation) with E2M1 and
    E1M2 codes, FPROP of the dense layer with 1 x 32 E8M0 blocks, and the
    dense layer in MXFP8 (E4M3 elements): its FPROP and X's quantization."""
    import workloads
    out = {}
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = U.lib_handle()

    def timed(fn, a, b, c):
        qa, qb = a.c(), b.c()
        return timed_args(fn, (ctypes.byref(qa), ctypes.byref(qb), ctypes.c_void_p(c.data_ptr()),
                               c.stride(0), stream))

    def timed_args(fn, args):
        for _ in range(2):
            fn(*args)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn(*args)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    wl = workloads.config5("cuda")
    X, W, dY = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY"]
    M, K = X.shape
    N = W.shape[0]
    for gname, grid in (("e2m1", U.UFP4_E2M1), ("e1m2", U.UFP4_E1M2)):
        mk = lambda st: U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, 32, 32, 1,  # noqa: E731
                                   sr_seed=wl.meta["sr_seed"], sr_stream=st)
        qx, _ = U.ufp4_rht_quant(X, 0, mk(0))
        qw, _ = U.ufp4_rht_quant(W, 0, mk(1))
        qdy, _ = U.ufp4_rht_quant(dY, 0, mk(2))
        qwt, qxt, qdyt = (U.ufp4_transpose_qtensor(q) for q in (qw, qx, qdy))
        if grid == U.UFP4_E2M1:   # the transpose that reuses dY for WGRAD
            qd = qdy.c()
            ms = timed_args(lib.ufp4_transpose_qtensor,
                            (ctypes.byref(qd), ctypes.c_void_p(qdyt.codes.data_ptr()),
                             ctypes.c_void_p(qdyt.scales.data_ptr()), stream))
            nbytes = 2 * (qdy.codes.numel() + qdy.scales.numel() * qdy.scales.element_size())
            out[f"transpose_square_blocks_{M}x{N}_codes_scales"] = {
                "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4)}
        peak = FP4_PEAK_TFLOPS if grid == U.UFP4_E2M1 else FP8_PEAK_TFLOPS
        for name, a, b, shp in (("fprop", qx, qw, (M, N)), ("dgrad", qdy, qwt, (M, K)),
                                ("wgrad", qdyt, qxt, (N, K))):
            c = torch.empty(shp, dtype=torch.float32, device="cuda")
            ms = timed(getattr(lib, "ufp4_gemm_" + name), a, b, c)
            tf = 2.0 * M * N * K / ms / 1e9
            out[f"square_blocks_{M}x{K}x{N}_{gname}_{name}"] = {
                "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "peak": peak,
                "frac": round(tf / peak, 4),
                "mfma": "v_mfma_scale_f32_32x32x64_f8f6f4 (" + ("FP4" if grid == U.UFP4_E2M1 else "FP8 E4M3") + ")"}
        del qx, qw, qdy, qwt, qxt, qdyt
    # dense layer FPROP with 1 x 32 E8M0 blocks, n = 32 rotation
    wl2 = workloads.config2("cuda")
    X2, W2 = wl2.tensors["X"], wl2.tensors["W"]
    M2, K2 = X2.shape
    N2 = W2.shape[0]
    for gname, grid in (("e2m1", U.UFP4_E2M1), ("e1m2", U.UFP4_E1M2)):
        cfg = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 32, sign_seed=wl2.meta["sign_seeds"][0])
        qx, _ = U.ufp4_rht_quant(X2, 0, cfg)
        qw, _ = U.ufp4_rht_quant(W2, 0, cfg)
        c = torch.empty((M2, N2), dtype=torch.float32, device="cuda")
        ms = timed(lib.ufp4_gemm_fprop, qx, qw, c)
        tf = 2.0 * M2 * N2 * K2 / ms / 1e9
        peak = FP4_PEAK_TFLOPS if grid == U.UFP4_E2M1 else FP8_PEAK_TFLOPS
        out[f"dense_1x32_e8m0_{M2}x{K2}x{N2}_{gname}_fprop"] = {
            "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "peak": peak, "frac": round(tf / peak, 4)}
    # MXFP8 (E4M3, 1 x 32 E8M0): the dense layer's FPROP and X's quantization
    cfg = U.make_cfg(U.UFP4_E4M3, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1)
    qx, _ = U.ufp4_rht_quant(X2, 0, cfg)
    qw, _ = U.ufp4_rht_quant(W2, 0, cfg)
    c = torch.empty((M2, N2), dtype=torch.float32, device="cuda")
    ms = timed(lib.ufp4_gemm_fprop, qx, qw, c)
    tf = 2.0 * M2 * N2 * K2 / ms / 1e9
    out[f"mxfp8_{M2}x{K2}x{N2}_fprop"] = {
        "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "peak": FP8_PEAK_TFLOPS,
        "frac": round(tf / FP8_PEAK_TFLOPS, 4),
        "mfma": "v_mfma_scale_f32_32x32x64_f8f6f4 (FP8 E4M3)"}
    qargs = (ctypes.c_void_p(X2.data_ptr()), M2, K2, K2, 0, ctypes.byref(cfg),
             ctypes.c_void_p(qx.codes.data_ptr()), ctypes.c_void_p(qx.scales.data_ptr()), None,
             stream)
    ms = timed_args(lib.ufp4_rht_quant, qargs)
    nbytes = M2 * K2 * (2 + 1 + 1 / 32)
    out[f"mxfp8_quant_rows_{M2}x{K2}"] = {"ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                                          "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                          "bytes_per_elem": round(2 + 1 + 1 / 32, 4)}
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
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
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
    args = (ctypes.c_void_p(X.data_ptr()), M, K, K, ctypes.byref(cfg),
            ctypes.c_void_p(stats.data_ptr()), stream)
    for _ in range(2):
        lib.ufp4_quant_diag(*args)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        lib.ufp4_quant_diag(*args)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbps = 2.0 * M * K / ms / 1e6
    out["kernel_e1m2_n16"] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                              "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                              "bytes_per_elem": 2.0}
    return out


def moe_layers(U, torch, reps=5):
    """The MoE layers of the grouped configurations (context; not part of the
    step): 64 experts (Zipf routing, top-6; E1M2, n = 32, 1 x 32 fp32 scales)
    and 16 experts (uniform top-8; INT4, n = 128, 1 x 16), each as its six
    quantizations (X_perm, W, dY_perm row-wise; W^T per expert, dY_perm^T and
    X_perm^T per expert segment) and its three grouped GEMMs.  TFLOP/s count
    the unpadded token rows; back-to-back launches timed with HIP events."""
    import workloads
    out = {}
    cases = (("moe64_zipf_e1m2_1x32_n32", workloads.config3, U.UFP4_E1M2, 32, 32),
             ("moe16_share_int4_1x16_n128", workloads.config4, U.UFP4_INT4, 128, 16))
    for name, mkwl, grid, n, b in cases:
        wl = mkwl("cuda")
        X, W, dYp = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY_perm"]
        off = wl.meta["offsets"].tolist()
        counts = wl.meta["counts"]
        E, H, F = wl.meta["experts"], wl.meta["hidden"], wl.meta["ffn"]
        Xp = workloads.gather_rows(X, wl.meta["gather"].to(X.device))
        del X
        sf, sd, sw = wl.meta["sign_seeds"]
        sr = wl.meta["sr_seed"]
        mk = lambda seed, rnd, st=0: U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, n,  # noqa: E731
                                                  sign_seed=seed, sr_seed=sr, sr_stream=st)
        woff = [g * F for g in range(E + 1)]
        q = {}
        quant = {
            "quant_x_row": (lambda: U.ufp4_rht_quant(Xp, 0, mk(sf, U.UFP4_RTNE))[0], Xp.numel()),
            "quant_w_row": (lambda: U.ufp4_rht_quant(W, 0, mk(sf, U.UFP4_RTNE))[0], W.numel()),
            "quant_dy_row": (lambda: U.ufp4_rht_quant(dYp, 0, mk(sd, U.UFP4_SR, 0))[0], dYp.numel()),
            "quant_w_col": (lambda: U.ufp4_rht_quant_segmented(W, woff, mk(sd, U.UFP4_RTNE)), W.numel()),
            "quant_dy_col": (lambda: U.ufp4_rht_quant_segmented(dYp, off, mk(sw, U.UFP4_SR, 1)), dYp.numel()),
            "quant_x_col": (lambda: U.ufp4_rht_quant_segmented(Xp, off, mk(sw, U.UFP4_RTNE)), Xp.numel()),
        }
        res = {}
        bpe = 2.0 + 0.5 + 4.0 / b

        def timed(fn):
            r = fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                r = fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps, r

        for k, (fn, elems) in quant.items():
            ms, q[k] = timed(fn)
            res[k] = {"ms": round(ms, 4), "GB/s": round(bpe * elems / ms / 1e6, 1)}
        tokens = int(sum(int(c) for c in counts))
        flops = 2.0 * tokens * F * H
        gemms = {
            "fprop": lambda: U.ufp4_gemm_fprop_grouped(q["quant_x_row"], q["quant_w_row"], off),
            "dgrad": lambda: U.ufp4_gemm_dgrad_grouped(q["quant_dy_row"], U.stacked(q["quant_w_col"], E), off),
            "wgrad": lambda: U.ufp4_gemm_wgrad_grouped(q["quant_dy_col"], q["quant_x_col"], off),
        }
        for k, fn in gemms.items():
            ms, r = timed(fn)
            del r
            tf = flops / ms / 1e9
            res[k] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                      "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
        res["tokens_x_topk"] = tokens
        res["padded_rows"] = int(off[-1])
        out[name] = res
        del wl, Xp, W, dYp, q
        torch.cuda.empty_cache()
    return out


def cpu_oracle_baseline(grid):
    """The oracle as it stands on a bounded sample of the same workload: the
    dense step restricted to M' = 6144 tokens and N' = 6144 output features
    (full K = 2048): six quantizations, six dequantizations and three fp64
    GEMMs.  The quantizer is single-threaded numpy; the GEMMs use numpy's
    BLAS thread pool, whose size is reported as the cores used."""
    import oracle as O
    import workloads
    gi = {"e1m2": 0, "int4": 1, "e2m1": 2}[grid]
    Mp, Np, K = 6144, 6144, 2048
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
    qbytes = QBYTES_PER_ELEM * (2 * Mp * K + 2 * Np * K + 2 * Mp * Np)
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"dense step at M'={Mp}, N'={Np}, K={K} (6 quantizations + 3 fp64 "
                      f"GEMMs) in {t:.2f} s; its quantizer part ran at "
                      f"{qbytes / tq / 1e9:.4f} GB/s (numpy, single-threaded); "
                      "value is the sample's GEMM flops over its whole time",
            "quant_GBps": round(qbytes / tq / 1e9, 6), "seconds": round(t, 3),
            "cpu": platform.processor() or platform.machine()}


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

    grid = {"e1m2": U.UFP4_E1M2, "int4": U.UFP4_INT4, "e2m1": U.UFP4_E2M1}[args.grid]
    wl = Workload(U, torch, grid, max(1, args.sets), streams=args.streams, dual=args.dual)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        wl.step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        wl.step(i)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps

    # per-kernel averages: each call alone, back to back
    names = [c[0] for c in wl.calls[0]]
    per = {n: wl.time_call(i, max(10, args.steps)) for i, n in enumerate(names)}

    kernels = {}
    for k, f in wl.flops.items():
        kernels[k] = {"ms": round(per[k], 4), "TFLOP/s": round(f / per[k] / 1e9, 2),
                      "frac_bf16_peak": round(f / per[k] / 1e9 / BF16_PEAK_TFLOPS, 4)}
    qbytes = {k: wl.qbpe[k] * v for k, v in wl.elems.items()}
    for k, b in qbytes.items():
        kernels["quant_" + k] = {"ms": round(per["quant_" + k], 4),
                                 "GB/s": round(b / per["quant_" + k] / 1e6, 1),
                                 "frac_hbm_peak": round(b / per["quant_" + k] / 1e6 / HBM_PEAK_GBPS, 4)}
    for k in kernels:   # HBM bytes per launch as last counted (null if the kernel changed)
        kernels[k]["traffic_B"] = measured_traffic(k, args.grid)
    gemm_ms = sum(per[k] for k in wl.flops)
    quant_ms = sum(per["quant_" + k] for k in qbytes)
    total_flops = sum(wl.flops.values())
    # dominant kernel: the one with the largest share of the step
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    if dom in wl.flops:
        ach = wl.flops[dom] / per[dom] / 1e9
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(dom, args.grid), "traffic_unit": "B/launch"}
    else:
        ach = qbytes[dom[6:]] / per[dom] / 1e6
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dom, args.grid), "traffic_unit": "B/launch"}
    quant_gbps = sum(qbytes.values()) / quant_ms / 1e6
    value = total_flops / (ms_step * 1e-3) / 1e12

    single = single_axis(U, torch, wl)
    wl_m, wl_k, wl_n = wl.M, wl.K, wl.N
    qbpe = next(iter(wl.qbpe.values()))
    stream_q = None
    if not args.no_stream:
        wl = None   # free the step's buffers first
        torch.cuda.empty_cache()
        stream_q = quant_stream(U, torch)
    mx = None
    if not args.no_mx:
        wl = None   # free the step's buffers first
        torch.cuda.empty_cache()
        mx = mx_gemms(U, torch)
    moe = None
    if not args.no_moe:
        if args.no_mx:
            wl = None
            torch.cuda.empty_cache()
        moe = moe_layers(U, torch)
    diag = None
    if not args.no_diag:
        wl = None
        torch.cuda.empty_cache()
        diag = diagnostics(U, torch)

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
        "dtype_detail": "bf16 in; fp32 rotate/scale/round; 4-bit codes; GEMM: exact E4M3 level products (fp8 MFMA) x bf16 scale products (bf16 MFMA), fp32 fma accumulate",
        "data": "synthetic (seeded torch generators; dense linear-layer tensors)",
        "config": {"workload": f"dense linear layer M={wl_m} K={wl_k} N={wl_n}: "
                               + ("3 dual-axis fused RHT(n=16)+1x16 " if args.dual else "6 fused RHT(n=16)+1x16 ")
                               + f"{args.grid} quantizations (6 quantized copies, SR on dY) + FPROP/DGRAD/WGRAD",
                   "global_batch": wl_m, "seq_len": None, "parallelism": "single GPU",
                   "streams": args.streams, "dual_axis_quant": bool(args.dual)},
        "roofline": roof,
        "quant": {"GB/s": round(quant_gbps, 1), "frac_hbm_peak": round(quant_gbps / HBM_PEAK_GBPS, 4),
                  "ms": round(quant_ms, 4), "bytes_per_elem": qbpe},
        "gemm": {"TFLOP/s": round(total_flops / gemm_ms / 1e9, 2),
                 "frac_bf16_peak": round(total_flops / gemm_ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                 "frac_fp4_peak": round(total_flops / gemm_ms / 1e9 / FP4_PEAK_TFLOPS, 4),
                 "ms": round(gemm_ms, 4)},
        "kernels": kernels,
        "quant_single_axis": single,
        "quant_stream": stream_q,
        "cpu_baseline": cpu,
        "mx_gemms": mx,
        "moe_layers": moe,
        "diagnostics": diag,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
