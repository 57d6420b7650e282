"""Python face of the CPU oracle (mx_oracle.c) plus the composite chains.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only importers; the GPU library and
its Python binding never import this module, and this module never imports
them.  Arrays are numpy; bf16 tensors travel as ``uint16`` bit patterns.

Page citations use the titles listed at the top of mx_oracle.c:
[P1] the MXFP6 Flux linears / fused MLP pull request, [P3] the MXFP4 Flux
training guide, [P4] the MXFP8 grouped SwiGLU MLP pull request.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle_mx.so")

E2M1, E2M3, E4M3 = 1, 2, 3
FLOOR, RCEIL = 0, 1
PRO_IDENTITY, PRO_GELU, PRO_DGELU, PRO_SWIGLU, PRO_DSWIGLU = 0, 1, 2, 3, 4
BITS = {E2M1: 4, E2M3: 6, E4M3: 8}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import build as _b  # local build script, gcc only
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        L.orc_decode.restype = ctypes.c_double
        L.orc_decode.argtypes = [ctypes.c_int, ctypes.c_uint]
        L.orc_encode.restype = ctypes.c_uint
        L.orc_encode.argtypes = [ctypes.c_int, ctypes.c_double]
        L.orc_scale_floor.restype = ctypes.c_uint
        L.orc_scale_floor.argtypes = [ctypes.c_int, ctypes.c_float]
        L.orc_scale_rceil.restype = ctypes.c_uint
        L.orc_scale_rceil.argtypes = [ctypes.c_float]
        L.orc_exp.restype = ctypes.c_float
        L.orc_exp.argtypes = [ctypes.c_float]
        L.orc_one_plus_tanh.restype = ctypes.c_float
        L.orc_one_plus_tanh.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_gelu_bf16.restype = ctypes.c_uint16
        L.orc_gelu_bf16.argtypes = [ctypes.c_uint16]
        L.orc_dgelu_bf16.restype = ctypes.c_uint16
        L.orc_dgelu_bf16.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        L.orc_swiglu_bf16.restype = ctypes.c_uint16
        L.orc_swiglu_bf16.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        L.orc_dswiglu_bf16.restype = None
        L.orc_dswiglu_bf16.argtypes = [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_uint16, u16p, u16p]
        L.orc_hadamard_c.restype = ctypes.c_float
        L.orc_hadamard_c.argtypes = []
        L.orc_hadamard32.restype = None
        L.orc_hadamard32.argtypes = [f32p, f32p]
        L.orc_prologue.restype = None
        L.orc_prologue.argtypes = [u16p, u16p, i64, i64, ctypes.c_int, u16p]
        L.orc_quantize.restype = ctypes.c_int
        L.orc_quantize.argtypes = [u16p, u16p, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, u8p, u8p, u8p, u8p, f32p, f32p]
        L.orc_gemm.restype = ctypes.c_int
        L.orc_gemm.argtypes = [u8p, u8p, u8p, u8p, i64, i64, i64, ctypes.c_int, u16p, i64p, i64, f64p]
        L.orc_get_code.restype = ctypes.c_uint
        L.orc_get_code.argtypes = [u8p, ctypes.c_int, i64]
        u32p = ctypes.POINTER(ctypes.c_uint32)
        L.orc_philox4x32_10.restype = None
        L.orc_philox4x32_10.argtypes = [u32p, u32p, u32p]
        L.orc_sr_word.restype = ctypes.c_uint32
        L.orc_sr_word.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_uint64]
        L.orc_encode_e2m1_sr.restype = ctypes.c_uint
        L.orc_encode_e2m1_sr.argtypes = [ctypes.c_double, ctypes.c_uint32]
        L.orc_quantize_sr.restype = ctypes.c_int
        L.orc_quantize_sr.argtypes = [u16p, i64, i64, ctypes.c_uint64, ctypes.c_uint64, u8p, u8p, u8p, u8p]
        _lib = L
    return _lib


def _p(a, ct):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ct))


# ---------------------------------------------------------------- scalars
def decode(fmt: int, code: int) -> float:
    return lib().orc_decode(fmt, code)


def encode(fmt: int, v: float) -> int:
    return lib().orc_encode(fmt, float(v))


def scale_floor(fmt: int, amax: float) -> int:
    return lib().orc_scale_floor(fmt, amax)


def scale_rceil(amax: float) -> int:
    return lib().orc_scale_rceil(amax)


def exp(x: float) -> float:
    return lib().orc_exp(x)


def one_plus_tanh(x: float) -> float:
    return lib().orc_one_plus_tanh(x)


def f32_to_bf16(x: float) -> int:
    return lib().orc_f32_to_bf16(x)


def gelu_bf16(h: int) -> int:
    return lib().orc_gelu_bf16(h)


def dgelu_bf16(da: int, h: int) -> int:
    return lib().orc_dgelu_bf16(da, h)


def swiglu_bf16(g: int, u: int) -> int:
    return lib().orc_swiglu_bf16(g, u)


def dswiglu_bf16(dz: int, g: int, u: int):
    a = ctypes.c_uint16()
    b = ctypes.c_uint16()
    lib().orc_dswiglu_bf16(dz, g, u, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def hadamard_c() -> float:
    return lib().orc_hadamard_c()


def hadamard32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (32,)
    r = np.empty(32, np.float32)
    lib().orc_hadamard32(_p(x, ctypes.c_float), _p(r, ctypes.c_float))
    return r


# ---------------------------------------------------------------- tensors
def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32)


def row_bytes(fmt: int, k: int) -> int:
    return k * BITS[fmt] // 8


def prologue(x: np.ndarray, aux, R: int, C: int, pro: int) -> np.ndarray:
    v = np.empty((R, C), np.uint16)
    lib().orc_prologue(_p(x, ctypes.c_uint16), _p(aux, ctypes.c_uint16), R, C, pro, _p(v, ctypes.c_uint16))
    return v


def quantize(x: np.ndarray, R: int, C: int, fmt: int, mode: int, hadamard: bool = False,
             pro: int = PRO_IDENTITY, aux=None, row: bool = True, col: bool = False,
             colsum: bool = False) -> dict:
    """Pack the bf16 tensor [R][C] (after the prologue) -- see orc_quantize."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    aux = None if aux is None else np.ascontiguousarray(aux, dtype=np.uint16)
    out = {}
    rc = rs = cc = cs = cp = csum = None
    if row:
        rc = np.zeros((R, row_bytes(fmt, C)), np.uint8)
        rs = np.zeros((R, C // 32), np.uint8)
    if col:
        cc = np.zeros((C, row_bytes(fmt, R)), np.uint8)
        cs = np.zeros((C, R // 32), np.uint8)
    if colsum:
        cp = np.zeros((R // 32, C), np.float32)
        csum = np.zeros((C,), np.float32)
    st = lib().orc_quantize(_p(x, ctypes.c_uint16), _p(aux, ctypes.c_uint16), R, C, fmt, mode,
                            int(hadamard), pro, _p(rc, ctypes.c_uint8), _p(rs, ctypes.c_uint8),
                            _p(cc, ctypes.c_uint8), _p(cs, ctypes.c_uint8), _p(cp, ctypes.c_float),
                            _p(csum, ctypes.c_float))
    if st != 0:
        raise ValueError(f"orc_quantize rejected the arguments (status {st})")
    if row:
        out["row_codes"], out["row_scales"] = rc, rs
    if col:
        out["col_codes"], out["col_scales"] = cc, cs
    if colsum:
        out["colsum_partials"], out["colsum"] = cp, csum
    return out


def philox4x32_10(ctr, key):
    """Philox4x32-10 (Salmon et al., SC 2011) of four counter words and two
    key words -> four output words."""
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib().orc_philox4x32_10(c, k, o)
    return list(o)


def sr_word(seed: int, axis: int, i: int) -> int:
    return lib().orc_sr_word(seed, axis, i)


def encode_e2m1_sr(v: float, r: int) -> int:
    return lib().orc_encode_e2m1_sr(float(v), r)


def quantize_sr(x: np.ndarray, R: int, C: int, seed: int, row: bool = True, col: bool = False,
                index_base: int = 0) -> dict:
    """MXFP4 (E2M1, FLOOR) pack with stochastic rounding of the elements
    [P3 Overview: SR of FP4 gradient quantization] -- see orc_quantize_sr."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    rc = rs = cc = cs = None
    if row:
        rc, rs = np.zeros((R, row_bytes(E2M1, C)), np.uint8), np.zeros((R, C // 32), np.uint8)
    if col:
        cc, cs = np.zeros((C, row_bytes(E2M1, R)), np.uint8), np.zeros((C, R // 32), np.uint8)
    st = lib().orc_quantize_sr(_p(x, ctypes.c_uint16), R, C, seed, index_base, _p(rc, ctypes.c_uint8),
                               _p(rs, ctypes.c_uint8), _p(cc, ctypes.c_uint8), _p(cs, ctypes.c_uint8))
    if st != 0:
        raise ValueError(f"orc_quantize_sr rejected the arguments (status {st})")
    out = {}
    if row:
        out["row_codes"], out["row_scales"] = rc, rs
    if col:
        out["col_codes"], out["col_scales"] = cc, cs
    return out


def gemm(a_codes, a_scales, b_codes, b_scales, M: int, N: int, K: int, fmt: int, bias=None,
         rows=None) -> np.ndarray:
    """C = A . B^T over dequantized operands, binary64 (see orc_gemm)."""
    a_codes = np.ascontiguousarray(a_codes, np.uint8)
    a_scales = np.ascontiguousarray(a_scales, np.uint8)
    b_codes = np.ascontiguousarray(b_codes, np.uint8)
    b_scales = np.ascontiguousarray(b_scales, np.uint8)
    assert a_codes.size == M * row_bytes(fmt, K) and b_codes.size == N * row_bytes(fmt, K)
    assert a_scales.size == M * (K // 32) and b_scales.size == N * (K // 32)
    ridx = None
    if rows is not None:
        ridx = np.ascontiguousarray(rows, np.int64)
    cnt = M if ridx is None else ridx.size
    out = np.empty((cnt, N), np.float64)
    if bias is not None:
        bias = np.ascontiguousarray(bias, np.uint16)
    st = lib().orc_gemm(_p(a_codes, ctypes.c_uint8), _p(a_scales, ctypes.c_uint8),
                        _p(b_codes, ctypes.c_uint8), _p(b_scales, ctypes.c_uint8), M, N, K, fmt,
                        _p(bias, ctypes.c_uint16), _p(ridx, ctypes.c_int64),
                        0 if ridx is None else ridx.size, _p(out, ctypes.c_double))
    if st != 0:
        raise ValueError(f"orc_gemm rejected the arguments (status {st})")
    return out


def gemm_accumulate(c_old, a_codes, a_scales, b_codes, b_scales, M: int, N: int, K: int, fmt: int,
                    bias=None) -> np.ndarray:
    """C_old + A . B^T (+ bias), binary64: the weight gradient added into a
    caller-owned main_grad ([P1] commit messages: the MXFP6 GEMM writes the
    weight gradient into main_grad itself instead of a separate add).
    ``c_old`` is bf16 bits (uint16) or float32, [M][N]; its values are exact
    in binary64.  The GPU rounds the sum once to c_old's dtype."""
    c_old = np.asarray(c_old)
    old = bf16_to_f32(c_old).astype(np.float64) if c_old.dtype == np.uint16 else c_old.astype(np.float64)
    assert old.shape == (M, N)
    return old + gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt, bias=bias)


def unpack_codes(codes: np.ndarray, fmt: int, k: int) -> np.ndarray:
    """Element codes [rows][k] from a packed [rows][k*bits/8] array."""
    codes = np.ascontiguousarray(codes, np.uint8)
    rows = codes.shape[0]
    out = np.empty((rows, k), np.uint8)
    L = lib()
    rb = row_bytes(fmt, k)
    for r in range(rows):
        rowp = codes[r].ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        for j in range(k):
            out[r, j] = L.orc_get_code(rowp, fmt, j)
    assert codes.shape[1] == rb
    return out


def round_bf16(x64: np.ndarray) -> np.ndarray:
    """Round a binary64 array to bf16 bits (binary64 -> binary32 -> bf16).

    Used only to shape oracle outputs for display; tolerance checks compare
    against the unrounded binary64 values."""
    f = np.asarray(x64, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


# ---------------------------------------------------------------- chains
def linear_ref(X, W, dY, fmt, mode, hadamard, M, N, K, rows=None):
    """MX linear Y = X.W^T, dX = dY.W, dW = dY^T.X on one set of bf16 inputs.

    [P1 description]: every MXFP6 GEMM needs M, N, K multiples of 256 because
    the backward GEMMs use K as an output dimension.  Operand mapping: fwd
    A = rows of X, B = rows of W (K = in features); dgrad A = rows of dY,
    B = columns of W (K = out features); wgrad A = columns of dY, B = columns
    of X (K = tokens)."""
    px = quantize(X, M, K, fmt, mode, hadamard, row=True, col=True)
    pw = quantize(W, N, K, fmt, mode, hadamard, row=True, col=True)
    pd = quantize(dY, M, N, fmt, mode, hadamard, row=True, col=True)
    out = {"X": px, "W": pw, "dY": pd}
    out["Y"] = gemm(px["row_codes"], px["row_scales"], pw["row_codes"], pw["row_scales"], M, N, K, fmt,
                    rows=rows)
    out["dX"] = gemm(pd["row_codes"], pd["row_scales"], pw["col_codes"], pw["col_scales"], M, K, N, fmt,
                     rows=rows)
    out["dW"] = gemm(pd["col_codes"], pd["col_scales"], px["col_codes"], px["col_scales"], N, K, M, fmt,
                     rows=None if rows is None else [r for r in rows if r < N])
    return out


def _kslice(codes, scales, fmt, k0, k1):
    """Columns [k0, k1) of a K-major packed operand (k0, k1 multiples of 32)."""
    b = BITS[fmt]
    return (np.ascontiguousarray(codes[:, k0 * b // 8:k1 * b // 8]),
            np.ascontiguousarray(scales[:, k0 // 32:k1 // 32]))


def mlp_fwd_ref(X, W1, b1, W2, M, D, F, h_in=None, rows=None, fmt=E2M3, mode=FLOOR, had=True):
    """Fused MLP forward [P1 description and Summary]: fc1 (+ bias in the
    accumulator), tanh-GELU taken by the packer as a prologue, fc2.  All packs
    use fmt / mode / had (the pages' recipe: E2M3, FLOOR scales, Hadamard-32
    along each GEMM's K).  ``h_in``: the bf16 pre-activation to pack from
    (defaults to this oracle's own h); pass the GPU's h to check the
    activation packs bit-for-bit."""
    px = quantize(X, M, D, fmt, mode, had, row=True, col=True)
    pw1 = quantize(W1, F, D, fmt, mode, had, row=True, col=True)
    pw2 = quantize(W2, D, F, fmt, mode, had, row=True, col=True)
    h64 = gemm(px["row_codes"], px["row_scales"], pw1["row_codes"], pw1["row_scales"], M, F, D, fmt,
               bias=b1)
    h = round_bf16(h64) if h_in is None else h_in
    pa = quantize(h, M, F, fmt, mode, had, pro=PRO_GELU, row=True, col=True)
    y64 = gemm(pa["row_codes"], pa["row_scales"], pw2["row_codes"], pw2["row_scales"], M, D, F, fmt,
               rows=rows)
    return {"X": px, "W1": pw1, "W2": pw2, "h64": h64, "h": h, "a": pa, "Y64": y64, "fmt": (fmt, mode, had)}


def mlp_bwd_ref(dY, fwd, M, D, F, da_in=None, h_in=None, rows=None):
    """Fused MXFP6 MLP backward [P1 description]: fc2 dgrad gives da (stored);
    the packer takes dGELU(da, h) as its prologue, so dh is never stored, and
    returns the fc1 bias gradient as a column sum; then fc1 dgrad and both
    weight gradients.  Format, scale mode and rotation are the forward's."""
    fmt, mode, had = fwd["fmt"]
    pdy = quantize(dY, M, D, fmt, mode, had, row=True, col=True)
    da64 = gemm(pdy["row_codes"], pdy["row_scales"], fwd["W2"]["col_codes"], fwd["W2"]["col_scales"],
                M, F, D, fmt)
    da = round_bf16(da64) if da_in is None else da_in
    h = fwd["h"] if h_in is None else h_in
    pdh = quantize(da, M, F, fmt, mode, had, pro=PRO_DGELU, aux=h, row=True, col=True, colsum=True)
    dx64 = gemm(pdh["row_codes"], pdh["row_scales"], fwd["W1"]["col_codes"], fwd["W1"]["col_scales"],
                M, D, F, fmt, rows=rows)
    dw1 = gemm(pdh["col_codes"], pdh["col_scales"], fwd["X"]["col_codes"], fwd["X"]["col_scales"],
               F, D, M, fmt, rows=None if rows is None else [r for r in rows if r < F])
    dw2 = gemm(pdy["col_codes"], pdy["col_scales"], fwd["a"]["col_codes"], fwd["a"]["col_scales"],
               D, F, M, fmt, rows=None if rows is None else [r for r in rows if r < D])
    return {"dY": pdy, "da64": da64, "da": da, "dh": pdh, "db1": pdh["colsum"], "dX64": dx64,
            "dW1_64": dw1, "dW2_64": dw2}


def grouped_ranges(offsets):
    ends = [int(v) for v in offsets]
    starts = [0] + ends[:-1]
    return list(zip(starts, ends))


def grouped_fwd_ref(X, W1, W2, offsets, R, D, F, H_in=None, fmt=E4M3, mode=RCEIL):
    """Routed-expert SwiGLU MLP forward (the pages' recipe: MXFP8 E4M3 with
    RCEIL scales [P4 commit messages]): expert g owns rows [off[g-1], off[g])
    (cumulative ends); per-expert counts are multiples of 128.  FC1 -> H
    (bf16, saved, [gate|up]); SwiGLU -> z, quantized rowwise 1x32 and
    columnwise 32x1; FC2 -> Y.  Rows at or past off[G-1] are not computed."""
    G = len(offsets)
    Ract = int(offsets[-1])
    px = quantize(X[:Ract], Ract, D, fmt, mode, row=True, col=True) if Ract else None
    H64 = np.zeros((Ract, 2 * F))
    w1 = [quantize(W1[g], 2 * F, D, fmt, mode, row=True, col=True) for g in range(G)]
    w2 = [quantize(W2[g], D, F, fmt, mode, row=True, col=True) for g in range(G)]
    for g, (s, e) in enumerate(grouped_ranges(offsets)):
        if e > s:
            H64[s:e] = gemm(px["row_codes"][s:e], px["row_scales"][s:e], w1[g]["row_codes"],
                            w1[g]["row_scales"], e - s, 2 * F, D, fmt)
    H = round_bf16(H64) if H_in is None else H_in[:Ract]
    pz = quantize(np.ascontiguousarray(H), Ract, F, fmt, mode, pro=PRO_SWIGLU, row=True, col=True) \
        if Ract else None
    Y64 = np.zeros((Ract, D))
    for g, (s, e) in enumerate(grouped_ranges(offsets)):
        if e > s:
            Y64[s:e] = gemm(pz["row_codes"][s:e], pz["row_scales"][s:e], w2[g]["row_codes"],
                            w2[g]["row_scales"], e - s, D, F, fmt)
    return {"X": px, "W1": w1, "W2": w2, "H64": H64, "H": H, "z": pz, "Y64": Y64, "fmt": (fmt, mode)}


def grouped_bwd_ref(dY, fwd, offsets, R, D, F, dz_in=None, H_in=None):
    """Routed-expert SwiGLU MLP backward: FC2 dgrad -> dz; dSwiGLU(dz, H) ->
    dH quantized rowwise and columnwise; FC1 dgrad; ragged-K weight
    gradients (K = the expert's tokens; an empty expert's gradient is 0).
    Format and scale mode are the forward's."""
    fmt, mode = fwd["fmt"]
    G = len(offsets)
    Ract = int(offsets[-1])
    pdy = quantize(dY[:Ract], Ract, D, fmt, mode, row=True, col=True) if Ract else None
    dz64 = np.zeros((Ract, F))
    for g, (s, e) in enumerate(grouped_ranges(offsets)):
        if e > s:
            dz64[s:e] = gemm(pdy["row_codes"][s:e], pdy["row_scales"][s:e], fwd["W2"][g]["col_codes"],
                             fwd["W2"][g]["col_scales"], e - s, F, D, fmt)
    dz = round_bf16(dz64) if dz_in is None else dz_in[:Ract]
    H = fwd["H"] if H_in is None else H_in[:Ract]
    pdh = quantize(np.ascontiguousarray(dz), Ract, 2 * F, fmt, mode, pro=PRO_DSWIGLU,
                   aux=np.ascontiguousarray(H), row=True, col=True) if Ract else None
    dX64 = np.zeros((Ract, D))
    dW1 = np.zeros((G, 2 * F, D))
    dW2 = np.zeros((G, D, F))
    for g, (s, e) in enumerate(grouped_ranges(offsets)):
        if e == s:
            continue
        dX64[s:e] = gemm(pdh["row_codes"][s:e], pdh["row_scales"][s:e], fwd["W1"][g]["col_codes"],
                         fwd["W1"][g]["col_scales"], e - s, D, 2 * F, fmt)
        ac, as_ = _kslice(pdy["col_codes"], pdy["col_scales"], fmt, s, e)
        bc, bs = _kslice(fwd["z"]["col_codes"], fwd["z"]["col_scales"], fmt, s, e)
        dW2[g] = gemm(ac, as_, bc, bs, D, F, e - s, fmt)
        ac, as_ = _kslice(pdh["col_codes"], pdh["col_scales"], fmt, s, e)
        bc, bs = _kslice(fwd["X"]["col_codes"], fwd["X"]["col_scales"], fmt, s, e)
        dW1[g] = gemm(ac, as_, bc, bs, 2 * F, D, e - s, fmt)
    return {"dY": pdy, "dz64": dz64, "dz": dz, "dH": pdh, "dX64": dX64, "dW1_64": dW1, "dW2_64": dW2}
