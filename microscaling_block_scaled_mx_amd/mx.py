"""Thin ctypes binding of libmx (include/mx.h).  Argument marshalling only:
every step of the path runs in the HIP kernels behind the C ABI.  torch is
used for device memory (tensors) and the current stream.  There is no
fallback: if libmx.so is missing or a call fails, an exception is raised."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmx.so")

# mx_fmt / mx_scale_mode / mx_prologue / mx_dtype / grouped enums (include/mx.h)
E2M1, E2M3, E4M3 = 1, 2, 3
FLOOR, RCEIL = 0, 1
PRO_IDENTITY, PRO_GELU_TANH, PRO_DGELU_TANH, PRO_SWIGLU, PRO_DSWIGLU = 0, 1, 2, 3, 4
BF16, F32 = 0, 1
RAGGED_M, RAGGED_K = 0, 1
EPI_NONE, EPI_SWIGLU, EPI_DSWIGLU = 0, 1, 2
BITS = {E2M1: 4, E2M3: 6, E4M3: 8}

STATUS = {0: "MX_OK", 1: "MX_ERR_NULL", 2: "MX_ERR_SHAPE", 3: "MX_ERR_ALIGN", 4: "MX_ERR_FORMAT",
          5: "MX_ERR_OFFSETS", 6: "MX_ERR_INDEX_OVERFLOW", 7: "MX_ERR_DEVICE", 8: "MX_ERR_LAUNCH",
          9: "MX_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 16 << 20  # MX_NOALLOC_SCRATCH_BYTES


class MXError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class Packed(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class MlpFwdArgs(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("D", ctypes.c_int64), ("F", ctypes.c_int64),
                ("fmt", ctypes.c_int32), ("scale_mode", ctypes.c_int32), ("hadamard", ctypes.c_int32),
                ("reserved", ctypes.c_int32),
                ("X", ctypes.c_void_p), ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("h", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("Xr", Packed), ("Xc", Packed), ("W1r", Packed), ("W1c", Packed), ("W2r", Packed),
                ("W2c", Packed), ("ar", Packed), ("ac", Packed)]


class MlpBwdArgs(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("D", ctypes.c_int64), ("F", ctypes.c_int64),
                ("fmt", ctypes.c_int32), ("scale_mode", ctypes.c_int32), ("hadamard", ctypes.c_int32),
                ("accumulate_wgrad", ctypes.c_int32),
                ("dY", ctypes.c_void_p), ("h", ctypes.c_void_p),
                ("Xc", Packed), ("W1c", Packed), ("W2c", Packed), ("ac", Packed),
                ("da", ctypes.c_void_p), ("dX", ctypes.c_void_p), ("dW1", ctypes.c_void_p),
                ("dW2", ctypes.c_void_p), ("db1", ctypes.c_void_p), ("db1_partials", ctypes.c_void_p),
                ("dYr", Packed), ("dYc", Packed), ("dhr", Packed), ("dhc", Packed)]


class GroupedArgs(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("epilogue", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32), ("G", ctypes.c_int32), ("validate_offsets", ctypes.c_int32),
                ("R", ctypes.c_int64), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("offsets", ctypes.c_void_p), ("A", Packed), ("B", Packed), ("C", ctypes.c_void_p),
                ("aux", ctypes.c_void_p), ("out_row", Packed), ("out_col", Packed)]


class QuantizeItem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("aux", ctypes.c_void_p), ("batch", ctypes.c_int64),
                ("R", ctypes.c_int64), ("C", ctypes.c_int64), ("row", Packed), ("col", Packed),
                ("colsum_partials", ctypes.c_void_p), ("colsum", ctypes.c_void_p)]


QUANTIZE_MANY_MAX = 8


class GemmItem(ctypes.Structure):
    _fields_ = [("A", Packed), ("B", Packed), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("bias", ctypes.c_void_p), ("bias_dtype", ctypes.c_int32), ("c_dtype", ctypes.c_int32),
                ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64), ("accumulate", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


GEMM_MANY_MAX = 4

_lib = None


def lib():
    """Load libmx.so (built in-tree by microscaling_block_scaled_mx_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m microscaling_block_scaled_mx_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.mx_quantize.restype = ci
        L.mx_quantize.argtypes = [vp, vp, i64, i64, i64, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, vp]
        L.mx_quantize_noalloc.restype = ci
        L.mx_quantize_noalloc.argtypes = [vp, vp, i64, i64, i64, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp]
        L.mx_quantize_sr.restype = ci
        L.mx_quantize_sr.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
        L.mx_quantize_many.restype = ci
        L.mx_quantize_many.argtypes = [ctypes.POINTER(QuantizeItem), ci, ci, ci, ci, ci, vp]
        L.mx_gemm_many.restype = ci
        L.mx_gemm_many.argtypes = [ctypes.POINTER(GemmItem), ci, ci, vp]
        L.mx_gemm.restype = ci
        L.mx_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp, ci, vp, ci, i64, vp]
        L.mx_gemm_tiled.restype = ci
        L.mx_gemm_tiled.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp, ci, vp, ci, i64, ci, ci, ci, vp]
        L.mx_gemm_splitk.restype = ci
        L.mx_gemm_splitk.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp, ci, vp, ci, i64, ci, ci, ci, ci, vp, i64,
                                     vp]
        L.mx_gemm_plan.restype = ci
        L.mx_gemm_plan.argtypes = [i64, i64, i64, ci, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int64)]
        L.mx_gemm_accumulate.restype = ci
        L.mx_gemm_accumulate.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp, ci, vp, ci, i64, vp]
        L.mx_fused_mlp_fwd.restype = ci
        L.mx_fused_mlp_fwd.argtypes = [ctypes.POINTER(MlpFwdArgs), vp]
        L.mx_fused_mlp_bwd.restype = ci
        L.mx_fused_mlp_bwd.argtypes = [ctypes.POINTER(MlpBwdArgs), vp]
        L.mx_grouped_gemm.restype = ci
        L.mx_grouped_gemm.argtypes = [ctypes.POINTER(GroupedArgs), vp]
        L.mx_status_str.restype = ctypes.c_char_p
        L.mx_status_str.argtypes = [ci]
        L.mx_device_supported.restype = ci
        L.mx_device_supported.argtypes = [ci]
        L.mx_codes_bytes.restype = i64
        L.mx_codes_bytes.argtypes = [ci, i64, i64]
        L.mx_scales_bytes.restype = i64
        L.mx_scales_bytes.argtypes = [i64, i64]
        L.mx_version.restype = ctypes.c_char_p
        L.mx_version.argtypes = []
        L.mx_clock_sample.restype = ci
        L.mx_clock_sample.argtypes = [i64, vp, vp]
        L.mx_wall_clock_khz.restype = i64
        L.mx_wall_clock_khz.argtypes = []
        _lib = L
    return _lib


def _ptr(t):
    """Device address of a tensor argument.  The C ABI reads and writes
    every buffer as a dense row-major array on the current device, so a
    host tensor, a tensor on another device or a strided view is refused
    here (a host pointer would reach the kernels, a view would be read with
    the wrong pitch).  Plain integers pass through as addresses."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise MXError(2, "tensor argument is a strided view; pass a contiguous tensor")
    if not t.is_cuda:
        raise MXError(7, "tensor argument is not on a GPU (the kernels take device memory)")
    if t.device.index != torch.cuda.current_device():
        raise MXError(7, f"tensor argument is on cuda:{t.device.index}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int, what: str):
    if st != 0:
        raise MXError(st, what)


# ---------------------------------------------------------------- buffers
def alloc_packed(rows: int, K: int, fmt: int, device="cuda", batch: int | None = None):
    """(codes, scales) uint8 tensors for a packed operand [rows] x K in the
    K-group-major layout: codes [ceil(K/128)][rows][16*bits], scales
    [ceil(K/128)][rows][4]."""
    groups = (K + 127) // 128
    shape = (groups, rows, 16 * BITS[fmt])
    sshape = (groups, rows, 4)
    if batch is not None:
        shape, sshape = (batch, *shape), (batch, *sshape)
    return (torch.empty(shape, dtype=torch.uint8, device=device),
            torch.empty(sshape, dtype=torch.uint8, device=device))


def _packed(p):
    return Packed(_ptr(p[0]), _ptr(p[1])) if p is not None else Packed(None, None)


# The C ABI takes bare pointers and cannot see buffer sizes; when the
# arguments are torch tensors, their sizes are checked here against what the
# call will touch (a short buffer, e.g. one packed in another format, would
# otherwise be read or written out of bounds).
def _nbytes(t):
    return t.numel() * t.element_size() if isinstance(t, torch.Tensor) else None


def _need(t, nbytes: int, what: str):
    n = _nbytes(t)
    if n is not None and n < nbytes:
        raise MXError(2, f"{what}: buffer holds {n} bytes, the call touches {nbytes}")


def _need_packed(p, rows: int, K: int, fmt: int, what: str, batch: int = 1):
    if p is None or fmt not in BITS:
        return
    _need(p[0], batch * lib().mx_codes_bytes(fmt, rows, K), what + " codes")
    _need(p[1], batch * lib().mx_scales_bytes(rows, K), what + " scales")


# ---------------------------------------------------------------- entry points
def quantize(x, R: int, C: int, fmt: int, scale_mode: int, hadamard: bool = False,
             prologue: int = PRO_IDENTITY, aux=None, row=None, col=None, colsum_partials=None, colsum=None,
             batch: int = 1, stream=None):
    """mx_quantize: row=(codes, scales) [R] x K=C, col=(codes, scales) [C] x K=R."""
    in_cols = 2 * C if prologue == PRO_SWIGLU else (C // 2 if prologue == PRO_DSWIGLU else C)
    _need(x, 2 * batch * R * in_cols, "quantize input")
    if prologue in (PRO_DGELU_TANH, PRO_DSWIGLU):
        _need(aux, 2 * batch * R * C, "quantize aux")
    _need_packed(row, R, C, fmt, "quantize row", batch)
    _need_packed(col, C, R, fmt, "quantize col", batch)
    _need(colsum_partials, 4 * batch * (R // 32) * C, "colsum partials")
    _need(colsum, 4 * batch * C, "colsum")
    st = lib().mx_quantize(_ptr(x), _ptr(aux), batch, R, C, fmt, scale_mode, int(hadamard), prologue,
                           _ptr(row[0]) if row else None, _ptr(row[1]) if row else None,
                           _ptr(col[0]) if col else None, _ptr(col[1]) if col else None,
                           _ptr(colsum_partials), _ptr(colsum), _stream(stream))
    _check(st, "mx_quantize")


def quantize_noalloc(x, R: int, C: int, fmt: int, scale_mode: int, hadamard: bool = False,
                     prologue: int = PRO_IDENTITY, aux=None, row=None, col=None, colsum=None, batch: int = 1,
                     stream=None):
    """mx_quantize_noalloc: mx_quantize whose column-sum partials live in the
    library's static device scratch (the call allocates nothing)."""
    in_cols = 2 * C if prologue == PRO_SWIGLU else (C // 2 if prologue == PRO_DSWIGLU else C)
    _need(x, 2 * batch * R * in_cols, "quantize_noalloc input")
    if prologue in (PRO_DGELU_TANH, PRO_DSWIGLU):
        _need(aux, 2 * batch * R * C, "quantize_noalloc aux")
    _need_packed(row, R, C, fmt, "quantize_noalloc row", batch)
    _need_packed(col, C, R, fmt, "quantize_noalloc col", batch)
    _need(colsum, 4 * batch * C, "colsum")
    st = lib().mx_quantize_noalloc(_ptr(x), _ptr(aux), batch, R, C, fmt, scale_mode, int(hadamard), prologue,
                                   _ptr(row[0]) if row else None, _ptr(row[1]) if row else None,
                                   _ptr(col[0]) if col else None, _ptr(col[1]) if col else None,
                                   _ptr(colsum), _stream(stream))
    _check(st, "mx_quantize_noalloc")


def quantize_sr(x, R: int, C: int, seed: int, row=None, col=None, colsum_partials=None, colsum=None,
                batch: int = 1, stream=None):
    """mx_quantize_sr: MXFP4 pack with stochastic rounding; row=(codes,
    scales) [R] x K=C, col=(codes, scales) [C] x K=R."""
    _need(x, 2 * batch * R * C, "quantize_sr input")
    _need_packed(row, R, C, E2M1, "quantize_sr row", batch)
    _need_packed(col, C, R, E2M1, "quantize_sr col", batch)
    _need(colsum_partials, 4 * batch * (R // 32) * C, "colsum partials")
    _need(colsum, 4 * batch * C, "colsum")
    st = lib().mx_quantize_sr(_ptr(x), batch, R, C, _ptr(row[0]) if row else None, _ptr(row[1]) if row else None,
                              _ptr(col[0]) if col else None, _ptr(col[1]) if col else None,
                              _ptr(colsum_partials), _ptr(colsum), seed & 0xFFFFFFFFFFFFFFFF, _stream(stream))
    _check(st, "mx_quantize_sr")


def quantize_many(items, fmt, scale_mode, hadamard=False, prologue=PRO_IDENTITY, stream=None):
    """mx_quantize_many: each item is a dict with the mx_quantize arguments
    x, R, C and optionally aux, batch (1), row=(codes, scales),
    col=(codes, scales), colsum_partials, colsum -- all packed in one launch."""
    n = len(items)
    arr = (QuantizeItem * max(n, 1))()
    for i, it in enumerate(items):
        R, C, batch = it["R"], it["C"], it.get("batch", 1)
        pro = prologue
        in_cols = 2 * C if pro == PRO_SWIGLU else (C // 2 if pro == PRO_DSWIGLU else C)
        what = f"quantize_many item {i}"
        _need(it["x"], 2 * batch * R * in_cols, what + " input")
        if pro in (PRO_DGELU_TANH, PRO_DSWIGLU):
            _need(it.get("aux"), 2 * batch * R * C, what + " aux")
        _need_packed(it.get("row"), R, C, fmt, what + " row", batch)
        _need_packed(it.get("col"), C, R, fmt, what + " col", batch)
        _need(it.get("colsum_partials"), 4 * batch * (R // 32) * C, what + " colsum partials")
        _need(it.get("colsum"), 4 * batch * C, what + " colsum")
        arr[i] = QuantizeItem(_ptr(it["x"]), _ptr(it.get("aux")), batch, R, C, _packed(it.get("row")),
                              _packed(it.get("col")), _ptr(it.get("colsum_partials")), _ptr(it.get("colsum")))
    st = lib().mx_quantize_many(arr, n, fmt, scale_mode, int(hadamard), prologue, _stream(stream))
    _check(st, "mx_quantize_many")


def gemm(a, b, M: int, N: int, K: int, fmt: int, c, bias=None, bias_dtype: int = BF16, c_dtype: int = BF16,
         ldc: int | None = None, stream=None):
    """mx_gemm: c [M][ldc] = A . B^T (+ bias); a, b = (codes, scales)."""
    _need_packed(a, M, K, fmt, "gemm A")
    _need_packed(b, N, K, fmt, "gemm B")
    _need(c, (4 if c_dtype == F32 else 2) * M * (N if ldc is None else ldc), "gemm C")
    _need(bias, (4 if bias_dtype == F32 else 2) * N, "gemm bias")
    st = lib().mx_gemm(_ptr(a[0]), _ptr(a[1]), _ptr(b[0]), _ptr(b[1]), M, N, K, fmt, _ptr(bias), bias_dtype,
                       _ptr(c), c_dtype, N if ldc is None else ldc, _stream(stream))
    _check(st, "mx_gemm")


def gemm_tiled(a, b, M: int, N: int, K: int, fmt: int, c, tile, bias=None, bias_dtype: int = BF16,
               c_dtype: int = BF16, ldc: int | None = None, stream=None):
    """mx_gemm_tiled: mx_gemm with the output tiling tile = (tile_m, tile_n,
    workgroups per compute unit), or (0, 0, 0) for mx_gemm's own choice; a
    pair (tile_m, tile_n) means one workgroup per compute unit."""
    _need_packed(a, M, K, fmt, "gemm_tiled A")
    _need_packed(b, N, K, fmt, "gemm_tiled B")
    _need(c, (4 if c_dtype == F32 else 2) * M * (N if ldc is None else ldc), "gemm_tiled C")
    _need(bias, (4 if bias_dtype == F32 else 2) * N, "gemm_tiled bias")
    st = lib().mx_gemm_tiled(_ptr(a[0]), _ptr(a[1]), _ptr(b[0]), _ptr(b[1]), M, N, K, fmt, _ptr(bias), bias_dtype,
                             _ptr(c), c_dtype, N if ldc is None else ldc, int(tile[0]), int(tile[1]),
                             int(tile[2]) if len(tile) > 2 else (0 if tuple(tile) == (0, 0) else 1),
                             _stream(stream))
    _check(st, "mx_gemm_tiled")


def gemm_plan(M: int, N: int, K: int, fmt: int):
    """mx_gemm_plan: ((tile_m, tile_n, wg_per_cu), split_k, workspace bytes)
    of a dense GEMM on this device."""
    plan = (ctypes.c_int * 4)()
    ws = ctypes.c_int64(0)
    _check(lib().mx_gemm_plan(M, N, K, fmt, plan, ctypes.byref(ws)), "mx_gemm_plan")
    return (plan[0], plan[1], plan[2]), plan[3], ws.value


def gemm_splitk(a, b, M: int, N: int, K: int, fmt: int, c, tile, split_k: int, workspace, bias=None,
                bias_dtype: int = BF16, c_dtype: int = BF16, ldc: int | None = None, stream=None,
                workspace_bytes: int | None = None):
    """mx_gemm_splitk: mx_gemm with the tiling tile = (tile_m, tile_n,
    workgroups per compute unit) and K cut into split_k parts, summed in order
    from the caller's workspace (split_k * M * N binary32 values; None when
    split_k is 1; workspace_bytes defaults to the tensor's size)."""
    _need_packed(a, M, K, fmt, "gemm_splitk A")
    _need_packed(b, N, K, fmt, "gemm_splitk B")
    _need(c, (4 if c_dtype == F32 else 2) * M * (N if ldc is None else ldc), "gemm_splitk C")
    _need(bias, (4 if bias_dtype == F32 else 2) * N, "gemm_splitk bias")
    ws_bytes = workspace_bytes if workspace_bytes is not None else _nbytes(workspace)
    st = lib().mx_gemm_splitk(_ptr(a[0]), _ptr(a[1]), _ptr(b[0]), _ptr(b[1]), M, N, K, fmt, _ptr(bias), bias_dtype,
                              _ptr(c), c_dtype, N if ldc is None else ldc, int(tile[0]), int(tile[1]), int(tile[2]),
                              int(split_k), _ptr(workspace), ws_bytes or 0, _stream(stream))
    _check(st, "mx_gemm_splitk")


def gemm_planned(a, b, M: int, N: int, K: int, fmt: int, c, bias=None, bias_dtype: int = BF16,
                 c_dtype: int = BF16, ldc: int | None = None, stream=None, workspace=None):
    """The GEMM under mx_gemm_plan's plan: mx_gemm_splitk with the planned
    tiling and split, taking the workspace it needs from `workspace` (a
    device tensor of at least that many bytes) or, if None, a new device
    tensor."""
    tile, split_k, ws_bytes = gemm_plan(M, N, K, fmt)
    if split_k > 1 and workspace is None:
        workspace = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    gemm_splitk(a, b, M, N, K, fmt, c, tile, split_k, workspace if split_k > 1 else None, bias, bias_dtype,
                c_dtype, ldc, stream)


def gemm_accumulate(a, b, M: int, N: int, K: int, fmt: int, c, bias=None, bias_dtype: int = BF16,
                    c_dtype: int = BF16, ldc: int | None = None, stream=None):
    """mx_gemm_accumulate: c [M][ldc] += A . B^T (+ bias); a, b = (codes, scales)."""
    _need_packed(a, M, K, fmt, "gemm_accumulate A")
    _need_packed(b, N, K, fmt, "gemm_accumulate B")
    _need(c, (4 if c_dtype == F32 else 2) * M * (N if ldc is None else ldc), "gemm_accumulate C")
    _need(bias, (4 if bias_dtype == F32 else 2) * N, "gemm_accumulate bias")
    st = lib().mx_gemm_accumulate(_ptr(a[0]), _ptr(a[1]), _ptr(b[0]), _ptr(b[1]), M, N, K, fmt, _ptr(bias),
                                  bias_dtype, _ptr(c), c_dtype, N if ldc is None else ldc, _stream(stream))
    _check(st, "mx_gemm_accumulate")


def gemm_many(items, fmt, stream=None):
    """mx_gemm_many: each item is a dict with the mx_gemm arguments a, b
    (packed operands), M, N, K, c and optionally c_dtype (BF16), ldc (N),
    bias, bias_dtype (BF16), accumulate (False: c = A.B^T; True: c += A.B^T)
    -- all computed in one launch where the tile shapes allow."""
    n = len(items)
    arr = (GemmItem * max(n, 1))()
    for i, it in enumerate(items):
        M, N, K = it["M"], it["N"], it["K"]
        c_dtype, bias_dtype = it.get("c_dtype", BF16), it.get("bias_dtype", BF16)
        ldc = it.get("ldc") or N
        what = f"gemm_many item {i}"
        _need_packed(it["a"], M, K, fmt, what + " A")
        _need_packed(it["b"], N, K, fmt, what + " B")
        _need(it["c"], (4 if c_dtype == F32 else 2) * M * ldc, what + " C")
        _need(it.get("bias"), (4 if bias_dtype == F32 else 2) * N, what + " bias")
        arr[i] = GemmItem(_packed(it["a"]), _packed(it["b"]), M, N, K, _ptr(it.get("bias")), bias_dtype, c_dtype,
                          _ptr(it["c"]), ldc, int(it.get("accumulate", 0)), 0)
    _check(lib().mx_gemm_many(arr, n, fmt, _stream(stream)), "mx_gemm_many")


def fused_mlp_fwd(M, D, F, X, W1, b1, W2, h, Y, Xr, Xc, W1r, W1c, W2r, W2c, ar, ac, fmt=E2M3,
                  scale_mode=FLOOR, hadamard=True, stream=None):
    for t, n, what in ((X, M * D, "X"), (W1, F * D, "W1"), (b1, F, "b1"), (W2, D * F, "W2"), (h, M * F, "h"),
                       (Y, M * D, "Y")):
        _need(t, 2 * n, "fused fwd " + what)
    for p, r, k, what in ((Xr, M, D, "Xr"), (Xc, D, M, "Xc"), (W1r, F, D, "W1r"), (W1c, D, F, "W1c"),
                          (W2r, D, F, "W2r"), (W2c, F, D, "W2c"), (ar, M, F, "ar"), (ac, F, M, "ac")):
        _need_packed(p, r, k, fmt, "fused fwd " + what)
    a = MlpFwdArgs(M, D, F, fmt, scale_mode, int(hadamard), 0, _ptr(X), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(h),
                   _ptr(Y), _packed(Xr), _packed(Xc), _packed(W1r), _packed(W1c), _packed(W2r), _packed(W2c),
                   _packed(ar), _packed(ac))
    _check(lib().mx_fused_mlp_fwd(ctypes.byref(a), _stream(stream)), "mx_fused_mlp_fwd")


def fused_mlp_bwd(M, D, F, dY, h, Xc, W1c, W2c, ac, da, dX, dW1, dW2, db1, db1_partials, dYr, dYc, dhr, dhc,
                  fmt=E2M3, scale_mode=FLOOR, hadamard=True, accumulate_wgrad=False, stream=None):
    for t, n, what in ((dY, 2 * M * D, "dY"), (h, 2 * M * F, "h"), (da, 2 * M * F, "da"), (dX, 2 * M * D, "dX"),
                       (dW1, 2 * F * D, "dW1"), (dW2, 2 * D * F, "dW2"), (db1, 4 * F, "db1"),
                       (db1_partials, 4 * (M // 32) * F, "db1 partials")):
        _need(t, n, "fused bwd " + what)
    for p, r, k, what in ((Xc, D, M, "Xc"), (W1c, D, F, "W1c"), (W2c, F, D, "W2c"), (ac, F, M, "ac"),
                          (dYr, M, D, "dYr"), (dYc, D, M, "dYc"), (dhr, M, F, "dhr"), (dhc, F, M, "dhc")):
        _need_packed(p, r, k, fmt, "fused bwd " + what)
    a = MlpBwdArgs(M, D, F, fmt, scale_mode, int(hadamard), int(accumulate_wgrad), _ptr(dY), _ptr(h), _packed(Xc), _packed(W1c),
                   _packed(W2c), _packed(ac), _ptr(da), _ptr(dX), _ptr(dW1), _ptr(dW2), _ptr(db1),
                   _ptr(db1_partials), _packed(dYr), _packed(dYc), _packed(dhr), _packed(dhc))
    _check(lib().mx_fused_mlp_bwd(ctypes.byref(a), _stream(stream)), "mx_fused_mlp_bwd")


def grouped_gemm(mode, G, R, offsets, A, B, C, fmt=E4M3, epilogue=EPI_NONE, scale_mode=RCEIL, M=0, N=0, K=0,
                 aux=None, out_row=None, out_col=None, validate_offsets=False, stream=None):
    _need(offsets, 4 * G, "grouped offsets")
    if mode == RAGGED_M:
        F = N // 2 if epilogue == EPI_SWIGLU else N
        _need_packed(A, R, K, fmt, "grouped A")
        _need_packed(B, N, K, fmt, "grouped B", G)
        _need(C, 2 * R * (F if epilogue == EPI_DSWIGLU else N), "grouped C")
        if epilogue == EPI_SWIGLU:
            _need_packed(out_row, R, F, fmt, "grouped out_row")
            _need_packed(out_col, F, R, fmt, "grouped out_col")
        elif epilogue == EPI_DSWIGLU:
            _need(aux, 2 * R * 2 * N, "grouped aux")
            _need_packed(out_row, R, 2 * N, fmt, "grouped out_row")
            _need_packed(out_col, 2 * N, R, fmt, "grouped out_col")
    else:
        _need_packed(A, M, R, fmt, "grouped A")
        _need_packed(B, N, R, fmt, "grouped B")
        _need(C, 2 * G * M * N, "grouped C")
    a = GroupedArgs(mode, epilogue, fmt, scale_mode, G, int(validate_offsets), R, M, N, K, _ptr(offsets),
                    _packed(A), _packed(B), _ptr(C), _ptr(aux), _packed(out_row), _packed(out_col))
    _check(lib().mx_grouped_gemm(ctypes.byref(a), _stream(stream)), "mx_grouped_gemm")


def device_supported(device: int = 0) -> bool:
    return bool(lib().mx_device_supported(device))


def status_str(st: int) -> str:
    return lib().mx_status_str(st).decode()


def clock_sample(microseconds: int, out, stream=None):
    """mx_clock_sample: out (uint64/int64 device tensor of 2) <- shader
    cycles and wall-clock ticks over `microseconds` of wall-clock time."""
    _need(out, 16, "clock_sample out")
    _check(lib().mx_clock_sample(int(microseconds), _ptr(out), _stream(stream)), "mx_clock_sample")


def wall_clock_khz() -> int:
    return int(lib().mx_wall_clock_khz())


def version() -> str:
    return lib().mx_version().decode()
