"""GPU parity at the full sizes of the benchmarked workloads, through the
same C-ABI calls and launch shapes that bench.py times.

The oracle cannot redo a whole workload in seconds, so every check here is
on sampled outputs that the oracle computes one by one from the original
bf16 inputs:

* a row-mode pack of row r depends only on row r, and a column-mode pack of
  column c only on column c (32-row blocks of one column), so the oracle
  packs just the sampled rows / columns and the GPU's packed tensors must
  match them byte for byte;
* a GEMM output C[m, n] depends only on row m of the A operand and row n of
  the B operand, so the oracle packs those operand rows itself and computes
  C on a sampled grid of m and n in binary64.

Bars as in the small parity tests: packed codes, scales and column sums
bit-exact; bf16 outputs within 2e-3 * max|ref| + half a bf16 ulp of the
unrounded binary64 oracle value.  Prologue packs take the GPU's own bf16
intermediates (h, da, H, dz) as oracle input, as the fused path's contract
is to pack exactly the tensor it stored."""
import os
import sys

import numpy as np
import pytest
import torch

from microscaling_block_scaled_mx_amd import inputs as I
from packed_layout import unblocked, untiled
from parity_checks import bf16_close, bf16_rel_err

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu

NS = 64  # sampled rows / columns per checked tensor (a multiple of 32)


@pytest.fixture(scope="module")
def mxl():
    from microscaling_block_scaled_mx_amd import mx
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert mx.device_supported(0), "GPU tests need a gfx950 device"
    return mx


def dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def host(t):
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    return a.view(np.uint16) if t.dtype == torch.int16 else a


def pick(rng, n, k=NS, lo=0):
    """k sorted distinct indices in [lo, n), always including both ends."""
    mid = rng.choice(np.arange(lo + 1, n - 1), size=k - 2, replace=False)
    return np.sort(np.concatenate([[lo, n - 1], mid])).astype(np.int64)


def gpu_plain(p, K, bits, batch=None):
    """The GPU's packed operand (codes, scales) in the oracle's plain layout:
    codes [rows][K*bits/8], scales [rows][K/32] (per expert when batched)."""
    return untiled(host(p[0]), K, bits), unblocked(host(p[1]), K // 32)


def orc_rows(orc, x, idx, fmt, mode, had, pro=0, aux=None):
    """Oracle row-mode pack of rows idx of x (whole rows: K = x's columns)."""
    from oracle import oracle as O
    xs = np.ascontiguousarray(x[idx])
    a = None if aux is None else np.ascontiguousarray(aux[idx])
    C = xs.shape[1] // 2 if pro == O.PRO_SWIGLU else (xs.shape[1] * 2 if pro == O.PRO_DSWIGLU else xs.shape[1])
    q = orc.quantize(xs, len(idx), C, fmt, mode, had, pro=pro, aux=a, row=True)
    return q["row_codes"], q["row_scales"]


def orc_cols(orc, x, idx, fmt, mode, had, pro=0, aux=None, F=None, colsum=False):
    """Oracle column-mode pack of output columns idx of x (each column packed
    along all of x's rows).  For the GLU prologues the input columns that
    feed the sampled output columns are gathered: SwiGLU reads gate column f
    and up column F+f of x = H; dSwiGLU writes d_gate f and d_up F+f from
    dz column f and H columns f, F+f (idx then names f < F only, and the
    result rows are [d_gate(idx) | d_up(idx)])."""
    from oracle import oracle as O
    R = x.shape[0]
    if pro == O.PRO_SWIGLU:
        xs, a, C = np.concatenate([x[:, idx], x[:, F + idx]], 1), None, len(idx)
    elif pro == O.PRO_DSWIGLU:
        xs, a, C = x[:, idx], np.concatenate([aux[:, idx], aux[:, F + idx]], 1), 2 * len(idx)
    else:
        xs, a, C = x[:, idx], None if aux is None else aux[:, idx], len(idx)
    q = orc.quantize(np.ascontiguousarray(xs), R, C, fmt, mode, had, pro=pro,
                     aux=None if a is None else np.ascontiguousarray(a), row=False, col=True, colsum=colsum)
    return q


def assert_rows_equal(got, want, what):
    for g, w, part in zip(got, want, ("codes", "scales")):
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            raise AssertionError(f"{what} {part}: {len(bad)} mismatching bytes, first at {bad[:4].tolist()}")


def assert_close(got_bf16, ref64, what):
    assert bf16_close(got_bf16, ref64), f"{what}: outside the bound, worst {bf16_rel_err(got_bf16, ref64):.3g}"


def gemm_grid(orc, a, b, K, fmt, bias=None):
    """Oracle C = A . B^T for operand rows a = (codes, scales) [m] and
    b = (codes, scales) [n]: the sampled [m, n] grid, binary64."""
    return orc.gemm(a[0], a[1], b[0], b[1], a[0].shape[0], b[0].shape[0], K, fmt, bias=bias)


# ------------------------------------------------------------------ linear step (MXFP6 headline, MXFP4 sweep)
def check_linear_step(mxl, orc, step, rng, full_packs):
    """One bench.py LinearStep on input copy 0: packs (X, W, dY; row + column)
    and the fwd / dgrad / wgrad GEMMs."""
    from bench import Timer
    M, N, K, fmt, mode, had = step.M, step.N, step.K, step.fmt, step.mode, step.had
    bits = mxl.BITS[fmt]
    step.run(0, Timer())
    torch.cuda.synchronize()
    X, W, dY = step.host
    g = {n: gpu_plain(p, k, bits) for n, p, k in (("Xr", step.Xr, K), ("Xc", step.Xc, M), ("Wr", step.Wr, K),
                                                  ("Wc", step.Wc, N), ("dYr", step.dYr, N), ("dYc", step.dYc, M))}
    if full_packs:  # every byte of the six packed operands
        for name, x, R, C in (("X", X, M, K), ("W", W, N, K), ("dY", dY, M, N)):
            q = orc.quantize(x, R, C, fmt, mode, had, row=True, col=True)
            assert_rows_equal(g[name + "r"], (q["row_codes"], q["row_scales"]), name + " row pack")
            assert_rows_equal(g[name + "c"], (q["col_codes"], q["col_scales"]), name + " col pack")
    m, n, k = pick(rng, M), pick(rng, N), pick(rng, K)
    # operand rows the sampled outputs need, packed by the oracle from the bf16 inputs
    Xr, Wr, dYr = orc_rows(orc, X, m, fmt, mode, had), orc_rows(orc, W, n, fmt, mode, had), \
        orc_rows(orc, dY, m, fmt, mode, had)
    qWc, qdYc, qXc = orc_cols(orc, W, k, fmt, mode, had), orc_cols(orc, dY, n, fmt, mode, had), \
        orc_cols(orc, X, k, fmt, mode, had)
    Wc, dYc, Xc = ((q["col_codes"], q["col_scales"]) for q in (qWc, qdYc, qXc))
    for name, got, want in (("X row", g["Xr"], Xr), ("W row", g["Wr"], Wr), ("dY row", g["dYr"], dYr),
                            ("W col", g["Wc"], Wc), ("dY col", g["dYc"], dYc), ("X col", g["Xc"], Xc)):
        idx = {"X row": m, "W row": n, "dY row": m, "W col": k, "dY col": n, "X col": k}[name]
        assert_rows_equal((got[0][idx], got[1][idx]), want, name + " pack (sampled)")
    Y, dX, dW = host(step.Y), host(step.dX), host(step.dW)
    assert_close(Y[np.ix_(m, n)], gemm_grid(orc, Xr, Wr, K, fmt), "Y = X W^T")
    assert_close(dX[np.ix_(m, k)], gemm_grid(orc, dYr, Wc, N, fmt), "dX = dY W")
    assert_close(dW[np.ix_(n, k)], gemm_grid(orc, dYc, Xc, M, fmt), "dW = dY^T X")


def test_linear_mxfp6_flux_attention_projection_full_size(mxl, orc):
    # the headline step: MXFP6 + Hadamard-32, X [4096,3072], W [3072,3072],
    # dY [4096,3072]; every packed byte, and 64 x 64 outputs of each GEMM
    from bench import LinearStep
    step = LinearStep(mxl, 4096, 3072, 3072, mxl.E2M3, mxl.FLOOR, True, 201, copies=1)
    check_linear_step(mxl, orc, step, np.random.default_rng(11), full_packs=True)


@pytest.mark.parametrize("i", range(len(I.FLUX_LINEARS)), ids=[n for n, _, _ in I.FLUX_LINEARS])
def test_linear_mxfp4_flux_sweep_full_size(mxl, orc, i):
    # the MXFP4 sweep at M = 16384 tokens; sampled packs and GEMM outputs
    from bench import LinearStep
    name, K, N = I.FLUX_LINEARS[i]
    step = LinearStep(mxl, 16384, N, K, mxl.E2M1, mxl.FLOOR, False, 401 + i, copies=1)
    check_linear_step(mxl, orc, step, np.random.default_rng(20 + i), full_packs=False)
    del step
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_tuned_splitk_plan_at_512_tokens(mxl, orc, fmt):
    # the adaLN dgrad at 512 tokens (M = 512, N = 3072, K = 18432): the tuned
    # table splits K (few output tiles, long K); through mx_gemm_plan and
    # mx_gemm_splitk as bench.py times it, sampled outputs against the oracle
    M, N, K = 512, 3072, 18432
    mode = mxl.RCEIL if fmt == mxl.E4M3 else mxl.FLOOR
    had = fmt == mxl.E2M3
    tile, split, ws_bytes = mxl.gemm_plan(M, N, K, fmt)
    assert split > 1 and ws_bytes == split * M * N * 4
    rng = np.random.default_rng(600 + fmt)
    A = I.bf16_normal(rng, (M, K), 1.0)
    B = I.bf16_normal(rng, (N, K), 0.02)
    pa, pb = mxl.alloc_packed(M, K, fmt), mxl.alloc_packed(N, K, fmt)
    mxl.quantize(dev(A), M, K, fmt, mode, had, row=pa)
    mxl.quantize(dev(B), N, K, fmt, mode, had, row=pb)
    C = torch.empty((M, N), dtype=torch.int16, device="cuda")
    mxl.gemm_planned(pa, pb, M, N, K, fmt, C)
    m, n = pick(rng, M), pick(rng, N)
    ref = gemm_grid(orc, orc_rows(orc, A, m, fmt, mode, had), orc_rows(orc, B, n, fmt, mode, had), K, fmt)
    assert_close(host(C)[np.ix_(m, n)], ref, f"split-K {split} C = A B^T")


# ------------------------------------------------------------------ fused MXFP6 MLP, M = 8192
def test_fused_mlp_mxfp6_flux_full_size(mxl, orc):
    from oracle import oracle as O
    M, D, F = 8192, 3072, 12288
    fmt, mode, had = mxl.E2M3, mxl.FLOOR, True
    bits = 6
    X, W1, b1, W2, dY = I.mlp(301, M, D, F)
    P = lambda r, k: mxl.alloc_packed(r, k, fmt)
    e16 = lambda *s: torch.empty(s, dtype=torch.int16, device="cuda")
    t = dict(X=dev(X), W1=dev(W1), b1=dev(b1), W2=dev(W2), dY=dev(dY), h=e16(M, F), Y=e16(M, D), Xr=P(M, D),
             Xc=P(D, M), W1r=P(F, D), W1c=P(D, F), W2r=P(D, F), W2c=P(F, D), ar=P(M, F), ac=P(F, M),
             da=e16(M, F), dX=e16(M, D), dW1=e16(F, D), dW2=e16(D, F),
             db1=torch.empty(F, dtype=torch.float32, device="cuda"),
             part=torch.empty((M // 32, F), dtype=torch.float32, device="cuda"), dYr=P(M, D), dYc=P(D, M),
             dhr=P(M, F), dhc=P(F, M))
    # the calls bench.py times
    mxl.fused_mlp_fwd(M, D, F, t["X"], t["W1"], t["b1"], t["W2"], t["h"], t["Y"], t["Xr"], t["Xc"], t["W1r"],
                      t["W1c"], t["W2r"], t["W2c"], t["ar"], t["ac"])
    mxl.fused_mlp_bwd(M, D, F, t["dY"], t["h"], t["Xc"], t["W1c"], t["W2c"], t["ac"], t["da"], t["dX"], t["dW1"],
                      t["dW2"], t["db1"], t["part"], t["dYr"], t["dYc"], t["dhr"], t["dhc"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    m, d, f = pick(rng, M), pick(rng, D), pick(rng, F)
    h, da = host(t["h"]), host(t["da"])
    G = lambda name, k: gpu_plain(t[name], k, bits)
    cols = lambda q: (q["col_codes"], q["col_scales"])
    # weight and input packs
    Xr, W1r, W2r = orc_rows(orc, X, m, fmt, mode, had), orc_rows(orc, W1, f, fmt, mode, had), \
        orc_rows(orc, W2, d, fmt, mode, had)
    Xc, W1c, W2c = cols(orc_cols(orc, X, d, fmt, mode, had)), cols(orc_cols(orc, W1, d, fmt, mode, had)), \
        cols(orc_cols(orc, W2, f, fmt, mode, had))
    dYr, dYc = orc_rows(orc, dY, m, fmt, mode, had), cols(orc_cols(orc, dY, d, fmt, mode, had))
    for name, k, idx, want in (("Xr", D, m, Xr), ("W1r", D, f, W1r), ("W2r", F, d, W2r), ("Xc", M, d, Xc),
                               ("W1c", F, d, W1c), ("W2c", D, f, W2c), ("dYr", D, m, dYr), ("dYc", M, d, dYc)):
        got = G(name, k)
        assert_rows_equal((got[0][idx], got[1][idx]), want, name + " pack (sampled)")
    # fc1 + bias -> h
    assert_close(h[np.ix_(m, f)], gemm_grid(orc, Xr, W1r, D, fmt, bias=np.ascontiguousarray(b1[f])), "h")
    # GELU-prologue packs of a from the GPU's h, then fc2 -> Y
    ar, ac = orc_rows(orc, h, m, fmt, mode, had, pro=O.PRO_GELU), cols(orc_cols(orc, h, f, fmt, mode, had,
                                                                             pro=O.PRO_GELU))
    got = G("ar", F)
    assert_rows_equal((got[0][m], got[1][m]), ar, "a row pack (sampled)")
    got = G("ac", M)
    assert_rows_equal((got[0][f], got[1][f]), ac, "a col pack (sampled)")
    assert_close(host(t["Y"])[np.ix_(m, d)], gemm_grid(orc, ar, W2r, F, fmt), "Y")
    # fc2 dgrad -> da
    assert_close(da[np.ix_(m, f)], gemm_grid(orc, dYr, W2c, D, fmt), "da")
    # dGELU-prologue packs of dh and the bias-gradient column sum from the GPU's da and h
    dhr = orc_rows(orc, da, m, fmt, mode, had, pro=O.PRO_DGELU, aux=h)
    qdhc = orc_cols(orc, da, f, fmt, mode, had, pro=O.PRO_DGELU, aux=h, colsum=True)
    got = G("dhr", F)
    assert_rows_equal((got[0][m], got[1][m]), dhr, "dh row pack (sampled)")
    got = G("dhc", M)
    assert_rows_equal((got[0][f], got[1][f]), cols(qdhc), "dh col pack (sampled)")
    assert np.array_equal(host(t["part"])[:, f].view(np.uint32), qdhc["colsum_partials"].view(np.uint32))
    assert np.array_equal(host(t["db1"])[f].view(np.uint32), qdhc["colsum"].view(np.uint32))
    # fc1 dgrad, fc1 wgrad, fc2 wgrad
    assert_close(host(t["dX"])[np.ix_(m, d)], gemm_grid(orc, dhr, W1c, F, fmt), "dX")
    assert_close(host(t["dW1"])[np.ix_(f, d)], gemm_grid(orc, cols(qdhc), Xc, M, fmt), "dW1")
    assert_close(host(t["dW2"])[np.ix_(d, f)], gemm_grid(orc, dYc, ac, M, fmt), "dW2")


# ------------------------------------------------------------------ grouped MXFP8 SwiGLU MLP
def test_grouped_mxfp8_swiglu_full_size(mxl, orc):
    from oracle import oracle as O
    R, D, F, G = 32768, 2048, 768, 8
    counts, offsets, X, W1, W2, dY = I.grouped_mlp(501, R, D, F, G)
    fmt, mode, had, bits = mxl.E4M3, mxl.RCEIL, False, 8
    P = lambda r, k, b=None: mxl.alloc_packed(r, k, fmt, batch=b)
    e16 = lambda *s: torch.empty(s, dtype=torch.int16, device="cuda")
    t = dict(X=dev(X), W1=dev(W1), W2=dev(W2), dY=dev(dY), off=dev(offsets.astype(np.int32)), Xr=P(R, D),
             Xc=P(D, R), W1r=P(2 * F, D, G), W1c=P(D, 2 * F, G), W2r=P(D, F, G), W2c=P(F, D, G), H=e16(R, 2 * F),
             zr=P(R, F), zc=P(F, R), Y=e16(R, D), dYr=P(R, D), dYc=P(D, R), dHr=P(R, 2 * F), dHc=P(2 * F, R),
             dX=e16(R, D), dW1=e16(G, 2 * F, D), dW2=e16(G, D, F))
    # the calls bench.py times, in its order
    mxl.quantize(t["X"], R, D, fmt, mode, row=t["Xr"], col=t["Xc"])
    mxl.quantize(t["W1"], 2 * F, D, fmt, mode, row=t["W1r"], col=t["W1c"], batch=G)
    mxl.quantize(t["W2"], D, F, fmt, mode, row=t["W2r"], col=t["W2c"], batch=G)
    mxl.grouped_gemm(mxl.RAGGED_M, G, R, t["off"], t["Xr"], t["W1r"], t["H"], epilogue=mxl.EPI_SWIGLU, N=2 * F,
                     K=D, out_row=t["zr"], out_col=t["zc"])
    mxl.grouped_gemm(mxl.RAGGED_M, G, R, t["off"], t["zr"], t["W2r"], t["Y"], N=D, K=F)
    mxl.quantize(t["dY"], R, D, fmt, mode, row=t["dYr"], col=t["dYc"])
    mxl.grouped_gemm(mxl.RAGGED_M, G, R, t["off"], t["dYr"], t["W2c"], None, epilogue=mxl.EPI_DSWIGLU, N=F, K=D,
                     aux=t["H"], out_row=t["dHr"], out_col=t["dHc"])
    mxl.grouped_gemm(mxl.RAGGED_M, G, R, t["off"], t["dHr"], t["W1c"], t["dX"], N=D, K=2 * F)
    mxl.grouped_gemm(mxl.RAGGED_K, G, R, t["off"], t["dYc"], t["zc"], t["dW2"], M=D, N=F)
    mxl.grouped_gemm(mxl.RAGGED_K, G, R, t["off"], t["dHc"], t["Xc"], t["dW1"], M=2 * F, N=D)
    torch.cuda.synchronize()
    # the same dgrad again with the debug store of dz (the epilogue's bf16
    # product before dSwiGLU): the packs must not change, and dz feeds the
    # oracle's dSwiGLU packs
    dz_t = e16(R, F)
    dHr2, dHc2 = P(R, 2 * F), P(2 * F, R)
    mxl.grouped_gemm(mxl.RAGGED_M, G, R, t["off"], t["dYr"], t["W2c"], dz_t, epilogue=mxl.EPI_DSWIGLU, N=F, K=D,
                     aux=t["H"], out_row=dHr2, out_col=dHc2)
    for a, b in ((t["dHr"], dHr2), (t["dHc"], dHc2)):
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    H, dz = host(t["H"]), host(dz_t)
    rng = np.random.default_rng(51)
    ranges = O.grouped_ranges(offsets)
    live = [g for g, (s, e) in enumerate(ranges) if e > s]
    assert counts[3] == 0 and len(live) == G - 1
    d, f2, f = pick(rng, D), pick(rng, 2 * F), pick(rng, F)
    cols = lambda q: (q["col_codes"], q["col_scales"])
    gp = lambda name, k, b=None: gpu_plain(t[name], k, bits, b)
    gXr, gXc, gzr, gzc = gp("Xr", D), gp("Xc", R), gp("zr", F), gp("zc", R)
    gdYr, gdYc, gdHr, gdHc = gp("dYr", D), gp("dYc", R), gp("dHr", 2 * F), gp("dHc", R)
    gW1r, gW1c, gW2r, gW2c = gp("W1r", D, G), gp("W1c", 2 * F, G), gp("W2r", F, G), gp("W2c", D, G)
    Hh, Yh, dXh = H, host(t["Y"]), host(t["dX"])
    dW1h, dW2h = host(t["dW1"]), host(t["dW2"])
    assert not np.any(dW1h[3]) and not np.any(dW2h[3]), "the empty expert's weight gradients must be zeros"
    for g in live:
        s, e = ranges[g]
        m = pick(rng, e, 32, lo=s)  # sampled token rows of expert g
        W1r, W2r = orc_rows(orc, W1[g], f2, fmt, mode, had), orc_rows(orc, W2[g], d, fmt, mode, had)
        W1c, W2c = cols(orc_cols(orc, W1[g], d, fmt, mode, had)), cols(orc_cols(orc, W2[g], f, fmt, mode, had))
        for name, got, idx, want in (("W1r", gW1r, f2, W1r), ("W2r", gW2r, d, W2r), ("W1c", gW1c, d, W1c),
                                     ("W2c", gW2c, f, W2c)):
            assert_rows_equal((got[0][g][idx], got[1][g][idx]), want, f"{name}[{g}] pack (sampled)")
        Xr, dYr = orc_rows(orc, X, m, fmt, mode, had), orc_rows(orc, dY, m, fmt, mode, had)
        assert_rows_equal((gXr[0][m], gXr[1][m]), Xr, f"X row pack, expert {g}")
        assert_rows_equal((gdYr[0][m], gdYr[1][m]), dYr, f"dY row pack, expert {g}")
        # FC1 -> H (gate | up), SwiGLU packs of z from the GPU's H, FC2 -> Y
        assert_close(Hh[np.ix_(m, f2)], gemm_grid(orc, Xr, W1r, D, fmt), f"H, expert {g}")
        zr = orc_rows(orc, Hh, m, fmt, mode, had, pro=O.PRO_SWIGLU)
        assert_rows_equal((gzr[0][m], gzr[1][m]), zr, f"z row pack, expert {g}")
        assert_close(Yh[np.ix_(m, d)], gemm_grid(orc, zr, W2r, F, fmt), f"Y, expert {g}")
        # FC2 dgrad -> dz (debug store), dSwiGLU packs of dH, FC1 dgrad -> dX
        assert_close(dz[np.ix_(m, f)], gemm_grid(orc, dYr, W2c, D, fmt), f"dz, expert {g}")
        dHr = orc_rows(orc, dz, m, fmt, mode, had, pro=O.PRO_DSWIGLU, aux=Hh)
        assert_rows_equal((gdHr[0][m], gdHr[1][m]), dHr, f"dH row pack, expert {g}")
        assert_close(dXh[np.ix_(m, d)], gemm_grid(orc, dHr, W1c, 2 * F, fmt), f"dX, expert {g}")
        # ragged-K weight gradients over the expert's token range [s, e)
        seg = slice(s, e)
        dYc_g = cols(orc_cols(orc, dY[seg], d, fmt, mode, had))
        zc_g = cols(orc_cols(orc, Hh[seg], f, fmt, mode, had, pro=O.PRO_SWIGLU, F=F))
        dHc_g = cols(orc_cols(orc, dz[seg], f, fmt, mode, had, pro=O.PRO_DSWIGLU, aux=Hh[seg], F=F))
        Xc_g = cols(orc_cols(orc, X[seg], d, fmt, mode, had))
        kb = slice(s * bits // 8, e * bits // 8)
        ks = slice(s // 32, e // 32)
        jj = np.concatenate([f, F + f])  # dH columns [d_gate(f) | d_up(f)]
        for name, got, idx, want in (("dY col", gdYc, d, dYc_g), ("z col", gzc, f, zc_g),
                                     ("dH col", gdHc, jj, dHc_g), ("X col", gXc, d, Xc_g)):
            assert_rows_equal((got[0][idx][:, kb], got[1][idx][:, ks]), want, f"{name} pack, expert {g}")
        assert_close(dW2h[g][np.ix_(d, f)], gemm_grid(orc, dYc_g, zc_g, e - s, fmt), f"dW2, expert {g}")
        assert_close(dW1h[g][np.ix_(jj, d)], gemm_grid(orc, dHc_g, Xc_g, e - s, fmt), f"dW1, expert {g}")
