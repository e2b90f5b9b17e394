"""Parity at the full sizes of the five workloads, in the launch
configuration bench.py times: every quantization call and GEMM of the
workload runs on the GPU at full size; the oracle recomputes seeded samples
(rows / columns / 32-row block groups) one by one.  Quantization samples must
match bit for bit (codes, scales; stochastic-rounding draws are indexed by
the element's position in the full operand); GEMM samples (a block of output
rows x columns) must be within 1e-4 relative Frobenius error of the oracle's
fp64 product of its own dequantized samples."""
import numpy as np
import pytest
import torch

import oracle as O
import rht_bit_block_amd as U
import workloads
from gpu_helpers import GEMM_TOL, host_bits, spec_of

pytestmark = pytest.mark.gpu


def _case(*a):
    print("case:", *a, flush=True)


def pick(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=min(k, n), replace=False))


def rows_bits(t, idx):
    return host_bits(t[torch.as_tensor(idx, device=t.device)])


def cols_bits(t, idx):
    return host_bits(t[:, torch.as_tensor(idx, device=t.device)])


def assert_quant_rows(codes, scales, ref, idx, what):
    """codes/scales: full GPU outputs of a K-contiguous operand (2-D)."""
    got_c = codes[torch.as_tensor(idx, device=codes.device)].cpu().numpy()
    got_s = scales[torch.as_tensor(idx, device=scales.device)].cpu().numpy()
    assert np.array_equal(got_c, ref["codes"]), f"{what}: codes differ"
    assert np.array_equal(got_s.view(np.uint32), ref["scales"].view(np.uint32)), f"{what}: scales differ"


def deq(ref, cfg):
    return O.dequant(ref["codes"], ref["scales"], spec_of(cfg), ref["P"], ref["K"])[1]


def assert_gemm(C, ridx, cidx, A64, B64, what):
    got = C[torch.as_tensor(ridx, device=C.device)][:, torch.as_tensor(cidx, device=C.device)]
    err = O.rel_fro(got.cpu().numpy(), O.gemm_ref(A64, B64))
    assert err <= GEMM_TOL, f"{what}: rel_fro {err:.3e}"
    return err


# ---------------------------------------------------------------------------
def test_config1_fprop_full():
    _case("config1")
    wl = workloads.config1("cuda")
    X, W = wl.tensors["X"], wl.tensors["W"]
    cfg = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=0)
    qx, rx = U.ufp4_rht_quant(X, 0, cfg, rotated=True)
    qw, _ = U.ufp4_rht_quant(W, 0, cfg)
    Y = U.ufp4_gemm_fprop(qx, qw)
    ox = O.quantize(host_bits(X), 0, spec_of(cfg))
    ow = O.quantize(host_bits(W), 0, spec_of(cfg))
    assert np.array_equal(rx.cpu().numpy().view(np.uint32), ox["rotated"].view(np.uint32))
    assert_quant_rows(qx.codes, qx.scales, ox, np.arange(256), "X")
    assert_quant_rows(qw.codes, qw.scales, ow, np.arange(256), "W")
    assert_gemm(Y, np.arange(256), np.arange(256), deq(ox, cfg), deq(ow, cfg), "fprop")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("grid", [U.UFP4_E1M2, U.UFP4_INT4, U.UFP4_E2M1])
def test_config2_dense_layer(grid):
    _case("config2", grid)
    wl = workloads.config2("cuda")
    X, W, dY = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY"]
    M, K = X.shape
    N = W.shape[0]
    sf, sd, sw = wl.meta["sign_seeds"]
    sr = wl.meta["sr_seed"]
    mk = lambda seed, rnd, st=0: U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, 16, 16,  # noqa: E731
                                              sign_seed=seed, sr_seed=sr, sr_stream=st)
    c_xr, c_wr, c_dyr = mk(sf, U.UFP4_RTNE), mk(sf, U.UFP4_RTNE), mk(sd, U.UFP4_SR, 0)
    c_wc, c_dyc, c_xc = mk(sd, U.UFP4_RTNE), mk(sw, U.UFP4_SR, 1), mk(sw, U.UFP4_RTNE)
    qxr, _ = U.ufp4_rht_quant(X, 0, c_xr)
    qwr, _ = U.ufp4_rht_quant(W, 0, c_wr)
    qdyr, _ = U.ufp4_rht_quant(dY, 0, c_dyr)
    qwc, _ = U.ufp4_rht_quant(W, 1, c_wc)
    qdyc, _ = U.ufp4_rht_quant(dY, 1, c_dyc)
    qxc, _ = U.ufp4_rht_quant(X, 1, c_xc)
    Y = U.ufp4_gemm_fprop(qxr, qwr)
    dX = U.ufp4_gemm_dgrad(qdyr, qwc)
    dW = U.ufp4_gemm_wgrad(qdyc, qxc)
    torch.cuda.synchronize()
    rM, rN, rK = pick(M, 24, 1), pick(N, 24, 2), pick(K, 24, 3)
    ox = O.quantize(rows_bits(X, rM), 0, spec_of(c_xr), row_index=rM)
    ow = O.quantize(rows_bits(W, rN), 0, spec_of(c_wr), row_index=rN)
    ody = O.quantize(rows_bits(dY, rM), 0, spec_of(c_dyr), row_index=rM)
    owt = O.quantize(cols_bits(W, rK), 1, spec_of(c_wc), row_index=rK)
    odyt = O.quantize(cols_bits(dY, rN), 1, spec_of(c_dyc), row_index=rN)
    oxt = O.quantize(cols_bits(X, rK), 1, spec_of(c_xc), row_index=rK)
    assert_quant_rows(qxr.codes, qxr.scales, ox, rM, "X row")
    assert_quant_rows(qwr.codes, qwr.scales, ow, rN, "W row")
    assert_quant_rows(qdyr.codes, qdyr.scales, ody, rM, "dY row (SR)")
    assert_quant_rows(qwc.codes, qwc.scales, owt, rK, "W col")
    assert_quant_rows(qdyc.codes, qdyc.scales, odyt, rN, "dY col (SR)")
    assert_quant_rows(qxc.codes, qxc.scales, oxt, rK, "X col")
    assert_gemm(Y, rM, rN, deq(ox, c_xr), deq(ow, c_wr), "fprop")
    assert_gemm(dX, rM, rK, deq(ody, c_dyr), deq(owt, c_wc), "dgrad")
    assert_gemm(dW, rN, rK, deq(odyt, c_dyc), deq(oxt, c_xc), "wgrad")


@pytest.mark.parametrize("grid", [U.UFP4_E1M2, U.UFP4_E2M1])
@pytest.mark.parametrize("n", [1, 16])
def test_config2_diag(grid, n):
    """Level statistics of config 2's X at full size: counts cover every
    element and equal the level histogram of the quantizer's own codes; a
    64-row slice quantized as its own operand matches the oracle exactly."""
    _case("config2 diag", grid, n)
    wl = workloads.config2("cuda")
    X = wl.tensors["X"]
    M, K = X.shape
    cfg = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, n, sign_seed=wl.meta["sign_seeds"][0])
    st = U.ufp4_quant_diag(X, cfg).cpu().numpy()
    assert st[:8].sum() == M * K
    q, _ = U.ufp4_rht_quant(X, 0, cfg)
    codes = q.codes
    nib = torch.stack([codes & 15, codes >> 4], dim=-1).reshape(-1).long()
    if grid == U.UFP4_INT4:
        mag = torch.where(nib >= 8, 16 - nib, nib)
    else:
        mag = nib & 7
    assert np.array_equal(torch.bincount(mag, minlength=8).cpu().numpy(), st[:8])
    r0 = int(pick(M // 64, 1, 7)[0]) * 64
    Xs = X[r0:r0 + 64].contiguous()
    got = U.ufp4_quant_diag(Xs, cfg).cpu().numpy()
    want = O.level_stats(O.quantize(host_bits(Xs), 0, spec_of(cfg)), grid)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
def _seg_codes(q, C, off, g, L, p_idx):
    """Rows p_idx of segment g of a segmented column-wise quantization."""
    base_c = C * off[g] // 2
    base_s = C * off[g] // q.cfg.block_cols
    nb = L // q.cfg.block_cols
    codes = q.codes.view(-1)[base_c: base_c + C * L // 2].view(C, L // 2)
    scales = q.scales.view(-1)[base_s: base_s + C * nb].view(C, nb)
    return codes, scales


def _moe(wl, grid, n, b):
    X, W, dYp = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY_perm"]
    gather, off, counts = wl.meta["gather"], wl.meta["offsets"].tolist(), wl.meta["counts"]
    E, H, F = wl.meta["experts"], wl.meta["hidden"], wl.meta["ffn"]
    Xp = workloads.gather_rows(X, gather.to(X.device))
    sf, sd, sw = wl.meta["sign_seeds"]
    sr = wl.meta["sr_seed"]
    mk = lambda seed, rnd, st=0: U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, n,  # noqa: E731
                                              sign_seed=seed, sr_seed=sr, sr_stream=st)
    c_xr, c_wr, c_dyr = mk(sf, U.UFP4_RTNE), mk(sf, U.UFP4_RTNE), mk(sd, U.UFP4_SR, 0)
    c_wc, c_dyc, c_xc = mk(sd, U.UFP4_RTNE), mk(sw, U.UFP4_SR, 1), mk(sw, U.UFP4_RTNE)
    qxr, _ = U.ufp4_rht_quant(Xp, 0, c_xr)
    qwr, _ = U.ufp4_rht_quant(W, 0, c_wr)
    qdyr, _ = U.ufp4_rht_quant(dYp, 0, c_dyr)
    woff = [g * F for g in range(E + 1)]
    qwc = U.ufp4_rht_quant_segmented(W, woff, c_wc)
    qdyc = U.ufp4_rht_quant_segmented(dYp, off, c_dyc)
    qxc = U.ufp4_rht_quant_segmented(Xp, off, c_xc)
    Y = U.ufp4_gemm_fprop_grouped(qxr, qwr, off)
    dX = U.ufp4_gemm_dgrad_grouped(qdyr, U.stacked(qwc, E), off)
    dW = U.ufp4_gemm_wgrad_grouped(qdyc, qxc, off)
    torch.cuda.synchronize()
    # the dual-axis calls bench.py times (one read per tensor, per-expert
    # column-wise side) give the same bits as the single-axis calls, which
    # are checked against the oracle below
    for t, cr, cc, o, (qr, qc), what in ((Xp, c_xr, c_xc, off, (qxr, qxc), "X_perm"),
                                         (W, c_wr, c_wc, woff, (qwr, qwc), "W"),
                                         (dYp, c_dyr, c_dyc, off, (qdyr, qdyc), "dY_perm")):
        dr, dc = U.ufp4_rht_quant_dual(t, cr, cc, row_offsets=o)
        assert torch.equal(dr.codes.view(-1), qr.codes.view(-1)), f"{what}: dual row codes"
        assert torch.equal(dr.scales.view(-1), qr.scales.view(-1)), f"{what}: dual row scales"
        assert torch.equal(dc.codes.view(-1), qc.codes.view(-1)), f"{what}: dual column codes"
        assert torch.equal(dc.scales.view(-1), qc.scales.view(-1)), f"{what}: dual column scales"
        del dr, dc
    # experts to sample: the largest, a median one and the smallest non-empty
    nz = [g for g in range(E) if off[g + 1] > off[g]]
    sizes = sorted(nz, key=lambda g: off[g + 1] - off[g])
    experts = sorted({sizes[-1], sizes[len(sizes) // 2], sizes[0]})
    for g in experts:
        o0, o1 = off[g], off[g + 1]
        L = o1 - o0
        rows = o0 + pick(L, 16, 10 + g)             # tokens of expert g (padding included)
        rF, rH = pick(F, 16, 20 + g), pick(H, 16, 30 + g)
        _case("expert", g, "tokens", int(counts[g]), "padded", L)
        ox = O.quantize(rows_bits(Xp, rows), 0, spec_of(c_xr), row_index=rows)
        ow = O.quantize(rows_bits(W, g * F + rF), 0, spec_of(c_wr), row_index=g * F + rF)
        ody = O.quantize(rows_bits(dYp, rows), 0, spec_of(c_dyr), row_index=rows)
        Wg = W[g * F:(g + 1) * F]
        owt = O.quantize(cols_bits(Wg, rH), 1, spec_of(c_wc), row_index=rH, elem_base=H * g * F)
        seg_dy, seg_x = dYp[o0:o1], Xp[o0:o1]
        odyt = O.quantize(cols_bits(seg_dy, rF), 1, spec_of(c_dyc), row_index=rF, elem_base=F * o0)
        oxt = O.quantize(cols_bits(seg_x, rH), 1, spec_of(c_xc), row_index=rH, elem_base=H * o0)
        assert_quant_rows(qxr.codes, qxr.scales, ox, rows, "X_perm row")
        assert_quant_rows(qwr.codes, qwr.scales, ow, g * F + rF, "W row")
        assert_quant_rows(qdyr.codes, qdyr.scales, ody, rows, "dY_perm row (SR)")
        wc_c, wc_s = _seg_codes(qwc, H, woff, g, F, rH)
        assert_quant_rows(wc_c, wc_s, owt, rH, "W^T segment")
        dy_c, dy_s = _seg_codes(qdyc, F, off, g, L, rF)
        assert_quant_rows(dy_c, dy_s, odyt, rF, "dY^T segment (SR)")
        x_c, x_s = _seg_codes(qxc, H, off, g, L, rH)
        assert_quant_rows(x_c, x_s, oxt, rH, "X^T segment")
        assert_gemm(Y, rows, rF, deq(ox, c_xr), deq(ow, c_wr), f"fprop e{g}")
        assert_gemm(dX, rows, rH, deq(ody, c_dyr), deq(owt, c_wc), f"dgrad e{g}")
        assert_gemm(dW, g * F + rF, rH, deq(odyt, c_dyc), deq(oxt, c_xc), f"wgrad e{g}")
    empty = [g for g in range(E) if off[g + 1] == off[g]]
    for g in empty:   # an expert without tokens has a zero weight gradient
        assert torch.count_nonzero(dW[g * F:(g + 1) * F]).item() == 0


def test_config3_moe64_zipf():
    _case("config3")
    wl = workloads.config3("cuda")
    _moe(wl, U.UFP4_E1M2, 32, 32)


def test_config4_moe16_share():
    _case("config4")
    wl = workloads.config4("cuda")
    _moe(wl, U.UFP4_INT4, 128, 16)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("grid", [U.UFP4_E2M1, U.UFP4_E1M2])
def test_config5_square_blocks(grid):
    _case("config5", grid)
    wl = workloads.config5("cuda")
    X, W, dY = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY"]
    M, K = X.shape
    N = W.shape[0]
    sr = wl.meta["sr_seed"]
    mk = lambda st: U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, 32, 32, 1,  # noqa: E731
                               sr_seed=sr, sr_stream=st)
    cx, cw, cdy = mk(0), mk(1), mk(2)
    qx, _ = U.ufp4_rht_quant(X, 0, cx)
    qw, _ = U.ufp4_rht_quant(W, 0, cw)
    qdy, _ = U.ufp4_rht_quant(dY, 0, cdy)
    # quantize once, reuse transposed: S(B) = S(B^T) on square blocks
    qwt, qdyt, qxt = (U.ufp4_transpose_qtensor(q) for q in (qw, qdy, qx))
    Y = U.ufp4_gemm_fprop(qx, qw)
    dX = U.ufp4_gemm_dgrad(qdy, qwt)
    dW = U.ufp4_gemm_wgrad(qdyt, qxt)
    # quantizing W^T directly gives exactly the transposed scale grid
    qw_direct, _ = U.ufp4_rht_quant(W.t().contiguous(), 0, cw)
    assert torch.equal(qw_direct.scales, qw.scales.t().contiguous())
    assert torch.equal(qwt.scales, qw.scales.t().contiguous())
    torch.cuda.synchronize()
    # samples: whole 32-row block groups (the 2D block is the unit)
    bx, bw, bdy = pick(M // 32, 2, 1), pick(N // 32, 2, 2), pick(M // 32, 2, 3)
    rx = np.concatenate([32 * b + np.arange(32) for b in bx])
    rw = np.concatenate([32 * b + np.arange(32) for b in bw])
    rdy = np.concatenate([32 * b + np.arange(32) for b in bdy])
    ox = O.quantize(rows_bits(X, rx), 0, spec_of(cx), row_index=rx)
    ow = O.quantize(rows_bits(W, rw), 0, spec_of(cw), row_index=rw)
    ody = O.quantize(rows_bits(dY, rdy), 0, spec_of(cdy), row_index=rdy)
    for q, ref, r, bs, what in ((qx, ox, rx, bx, "X"), (qw, ow, rw, bw, "W"), (qdy, ody, rdy, bdy, "dY")):
        got_c = q.codes[torch.as_tensor(r, device="cuda")].cpu().numpy()
        assert np.array_equal(got_c, ref["codes"]), what
        got_s = q.scales[torch.as_tensor(bs, device="cuda")].cpu().numpy()
        assert np.array_equal(got_s, ref["scales"]), what
    assert_gemm(Y, rx, rw, deq(ox, cx), deq(ow, cw), "fprop")
    # DGRAD samples dX[rdy, c] need W's columns c: the oracle quantizes the
    # 32-wide block column strips of W that hold them (full height)
    cstrip = pick(K // 32, 1, 4)[0]
    ccols = 32 * cstrip + np.arange(32)
    ow_strip = O.quantize(host_bits(W[:, 32 * cstrip:32 * cstrip + 32]), 0, spec_of(cw),
                          col_index=ccols, K_total=K)
    assert np.array_equal(qwt.codes[torch.as_tensor(ccols, device="cuda")].cpu().numpy(),
                          O.pack_nibbles(O.unpack_nibbles(ow_strip["codes"]).T))
    assert_gemm(dX, rdy, ccols, deq(ody, cdy), deq(ow_strip, cw).T, "dgrad")
    # WGRAD samples dW[r, c]: dY's block column of r and X's block column of c
    rstrip = pick(N // 32, 1, 5)[0]
    rrows = 32 * rstrip + np.arange(32)
    ody_strip = O.quantize(host_bits(dY[:, 32 * rstrip:32 * rstrip + 32]), 0, spec_of(cdy),
                           col_index=rrows, K_total=N)
    ox_strip = O.quantize(host_bits(X[:, 32 * cstrip:32 * cstrip + 32]), 0, spec_of(cx),
                          col_index=ccols, K_total=K)
    assert_gemm(dW, rrows, ccols, deq(ody_strip, cdy).T, deq(ox_strip, cx).T, "wgrad")


# ---------------------------------------------------------------------------
def test_config2_mxfp8():
    """The dense layer's FPROP in MXFP8 (E4M3, 1 x 32 E8M0) at full size:
    sampled rows of both operands bit-exact, sampled outputs within 1e-4."""
    _case("config2 mxfp8")
    wl = workloads.config2("cuda")
    X, W = wl.tensors["X"], wl.tensors["W"]
    M, K = X.shape
    N = W.shape[0]
    cfg = U.make_cfg(U.UFP4_E4M3, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 16,
                     sign_seed=wl.meta["sign_seeds"][0])
    qx, _ = U.ufp4_rht_quant(X, 0, cfg)
    qw, _ = U.ufp4_rht_quant(W, 0, cfg)
    Y = U.ufp4_gemm_fprop(qx, qw)
    torch.cuda.synchronize()
    rM, rN = pick(M, 24, 41), pick(N, 24, 42)
    ox = O.quantize(rows_bits(X, rM), 0, spec_of(cfg), row_index=rM)
    ow = O.quantize(rows_bits(W, rN), 0, spec_of(cfg), row_index=rN)
    assert_quant_rows(qx.codes, qx.scales, ox, rM, "X row (MXFP8)")
    assert_quant_rows(qw.codes, qw.scales, ow, rN, "W row (MXFP8)")
    assert_gemm(Y, rM, rN, deq(ox, cfg), deq(ow, cfg), "fprop (MXFP8)")


# ---------------------------------------------------------------------------
# The dense layer's quantizations exactly as bench.py's step makes them: one
# dual-axis call per tensor (X, W row- and column-wise RTNE; dY with SR on
# streams 0 / 1).  Sampled rows of the row-wise outputs and sampled columns
# of the column-wise ones are bit-exact against the oracle; every output is
# also identical to the corresponding single-axis call's.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("grid", [U.UFP4_E1M2, U.UFP4_INT4, U.UFP4_E2M1])
def test_config2_dual_calls(grid):
    _case("config2 dual", grid)
    wl = workloads.config2("cuda")
    sf, sd, sw = wl.meta["sign_seeds"]
    sr = wl.meta["sr_seed"]
    mk = lambda seed, rnd, st=0: U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, 16, 16,  # noqa: E731
                                              sign_seed=seed, sr_seed=sr, sr_stream=st)
    calls = (("X", mk(sf, U.UFP4_RTNE), mk(sw, U.UFP4_RTNE)),
             ("W", mk(sf, U.UFP4_RTNE), mk(sd, U.UFP4_RTNE)),
             ("dY", mk(sd, U.UFP4_SR, 0), mk(sw, U.UFP4_SR, 1)))
    for i, (name, cr, cc) in enumerate(calls):
        t = wl.tensors[name]
        R, C = t.shape
        qr, qc = U.ufp4_rht_quant_dual(t, cr, cc)
        torch.cuda.synchronize()
        rr, rc = pick(R, 24, 100 + i), pick(C, 24, 200 + i)
        o_r = O.quantize(rows_bits(t, rr), 0, spec_of(cr), row_index=rr)
        o_c = O.quantize(cols_bits(t, rc), 1, spec_of(cc), row_index=rc)
        assert_quant_rows(qr.codes.view(R, C // 2), qr.scales.view(R, C // 16), o_r, rr,
                          f"{name} dual row")
        assert_quant_rows(qc.codes.view(C, R // 2), qc.scales.view(C, R // 16), o_c, rc,
                          f"{name} dual col")
        sr_, _ = U.ufp4_rht_quant(t, 0, cr)
        sc_, _ = U.ufp4_rht_quant(t, 1, cc)
        assert torch.equal(qr.codes.view(R, C // 2), sr_.codes), f"{name}: row codes vs single-axis"
        assert torch.equal(qr.scales.view(R, C // 16), sr_.scales), f"{name}: row scales"
        assert torch.equal(qc.codes.view(C, R // 2), sc_.codes), f"{name}: col codes vs single-axis"
        assert torch.equal(qc.scales.view(C, R // 16), sc_.scales), f"{name}: col scales"
        del qr, qc, sr_, sc_


# ---------------------------------------------------------------------------
# Every element of the dense layer's FPROP (E1M2, 8192 x 8192 x 2048, the
# XCD-grouped tile order over all 1024 tiles) against the oracle's fp64
# product of its own full quantizations of X and W.
# ---------------------------------------------------------------------------
def test_config2_fprop_full_output():
    _case("config2 full fprop")
    wl = workloads.config2("cuda")
    X, W = wl.tensors["X"], wl.tensors["W"]
    sf = wl.meta["sign_seeds"][0]
    cfg = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=sf)
    qx, _ = U.ufp4_rht_quant(X, 0, cfg)
    qw, _ = U.ufp4_rht_quant(W, 0, cfg)
    Y = U.ufp4_gemm_fprop(qx, qw).cpu().numpy()
    ox = O.quantize(host_bits(X), 0, spec_of(cfg))
    ow = O.quantize(host_bits(W), 0, spec_of(cfg))
    assert np.array_equal(qx.codes.cpu().numpy(), ox["codes"])
    assert np.array_equal(qw.codes.cpu().numpy(), ow["codes"])
    ref = O.gemm_ref(deq(ox, cfg), deq(ow, cfg))
    err = O.rel_fro(Y, ref)
    # every 256 x 256 tile on its own, so a misplaced or skipped tile shows
    tiles = Y.shape[0] // 256, Y.shape[1] // 256
    worst = max(O.rel_fro(Y[256 * i:256 * i + 256, 256 * j:256 * j + 256],
                          ref[256 * i:256 * i + 256, 256 * j:256 * j + 256])
                for i in range(tiles[0]) for j in range(tiles[1]))
    print(f"  rel. Frobenius error {err:.3e}, worst tile {worst:.3e}", flush=True)
    assert err <= GEMM_TOL and worst <= GEMM_TOL
