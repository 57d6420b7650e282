"""C-ABI boundary checks that need no GPU: libmx.so loads, exports every
function include/mx.h declares, and rejects malformed arguments on the host
with the documented status before touching a device.  With well-formed
arguments and no gfx950 device present the call must answer MX_ERR_DEVICE
(never a silent success or a CPU fallback)."""
import ctypes
import os
import re

import pytest

from microscaling_block_scaled_mx_amd import mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mx.h")

OK, NULL, SHAPE, ALIGN, FORMAT, OFFSETS, OVERFLOW, DEVICE = 0, 1, 2, 3, 4, 5, 6, 7
P = 0x10000  # a 16-byte aligned fake device address; never dereferenced on these paths
P2, P3, P4, P5, P6, P7, P8 = (P * i for i in range(2, 9))


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mx_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = mx.lib()
    names = header_functions()
    assert {"mx_quantize", "mx_gemm", "mx_fused_mlp_fwd", "mx_fused_mlp_bwd", "mx_grouped_gemm"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_sizes():
    assert mx.status_str(0) == "MX_OK"
    for st in range(1, 10):
        assert mx.status_str(st).startswith(mx.STATUS[st])
    L = mx.lib()
    assert L.mx_codes_bytes(mx.E2M1, 256, 256) == 256 * 128
    assert L.mx_codes_bytes(mx.E2M3, 256, 256) == 256 * 192
    assert L.mx_codes_bytes(mx.E4M3, 256, 256) == 256 * 256
    assert L.mx_codes_bytes(9, 256, 256) == 0 and L.mx_codes_bytes(mx.E2M1, 1, 33) == 0
    assert L.mx_scales_bytes(256, 512) == 256 * 16
    assert L.mx_scales_bytes(256, 160) == 2 * 256 * 4  # blocked: ceil(5 / 4) K groups of 4 bytes per row
    assert L.mx_codes_bytes(mx.E2M3, 256, 160) == 2 * 256 * 96  # K-group-major: 2 groups of 96 bytes per row
    assert "gfx950" in mx.version()


def q(**kw):
    a = dict(x=P, aux=None, batch=1, R=64, C=128, fmt=mx.E2M1, mode=mx.FLOOR, had=0, pro=mx.PRO_IDENTITY,
             rc=P2, rs=P3, cc=P4, cs=P5, part=None, sum=None)
    a.update(kw)
    return mx.lib().mx_quantize(a["x"], a["aux"], a["batch"], a["R"], a["C"], a["fmt"], a["mode"], a["had"],
                                a["pro"], a["rc"], a["rs"], a["cc"], a["cs"], a["part"], a["sum"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL),
    (dict(rc=None), NULL),                       # codes without scales
    (dict(cs=None), NULL),
    (dict(rc=None, rs=None, cc=None, cs=None), NULL),  # nothing requested
    (dict(sum=P6), NULL),                        # colsum without partials
    (dict(pro=mx.PRO_DGELU_TANH), NULL),         # aux required
    (dict(pro=mx.PRO_DSWIGLU), NULL),
    (dict(fmt=0), FORMAT), (dict(fmt=4), FORMAT),
    (dict(mode=2), FORMAT),
    (dict(fmt=mx.E2M1, mode=mx.RCEIL), FORMAT),  # RCEIL is E4M3's
    (dict(fmt=mx.E2M1, had=1), FORMAT),          # rotation is E2M3's
    (dict(fmt=mx.E4M3, mode=mx.RCEIL, had=1), FORMAT),
    (dict(pro=7), FORMAT),
    (dict(R=48), SHAPE), (dict(C=40), SHAPE), (dict(R=-32), SHAPE), (dict(batch=0), SHAPE),
    (dict(pro=mx.PRO_DSWIGLU, aux=P6, C=96), SHAPE),  # F = C/2 must be a multiple of 32
    (dict(x=P + 8), ALIGN), (dict(rs=P3 + 4), ALIGN), (dict(part=P6 + 2), ALIGN),
    (dict(batch=70000), OVERFLOW),
])
def test_quantize_rejections(kw, want):
    assert q(**kw) == want


def test_quantize_valid_args_need_the_device():
    # valid on the host; no gfx950 device here, so the library refuses
    for kw in (dict(), dict(fmt=mx.E2M3, had=1), dict(fmt=mx.E4M3, mode=mx.RCEIL),
               dict(fmt=mx.E4M3, mode=mx.FLOOR), dict(pro=mx.PRO_DGELU_TANH, aux=P6, part=P7, sum=P8),
               dict(R=0), dict(cc=None, cs=None), dict(rc=None, rs=None, part=P7)):
        st = q(**kw)
        assert st in (OK, DEVICE), (kw, st)
        if not mx.lib().mx_device_supported(0):
            assert st == DEVICE



def qmany(items, n=None, fmt=mx.E2M1, mode=mx.FLOOR, had=0, pro=mx.PRO_IDENTITY):
    arr = (mx.QuantizeItem * max(len(items), 1))()
    for k, it in enumerate(items):
        a = dict(x=P, aux=None, batch=1, R=64, C=128, row=(P2, P3), col=(P4, P5), part=None, sum=None)
        a.update(it)
        arr[k] = mx.QuantizeItem(a["x"], a["aux"], a["batch"], a["R"], a["C"], mx.Packed(*a["row"]),
                                 mx.Packed(*a["col"]), a["part"], a["sum"])
    return mx.lib().mx_quantize_many(arr, len(items) if n is None else n, fmt, mode, had, pro, None)


def test_quantize_many_rejections():
    L = mx.lib()
    assert L.mx_quantize_many(None, 1, mx.E2M1, mx.FLOOR, 0, 0, None) == NULL
    assert qmany([{}], n=0) == SHAPE
    assert qmany([{}] * 9) == SHAPE  # more than MX_QUANTIZE_MANY_MAX
    # each item is validated as mx_quantize validates its arguments
    assert qmany([{}, dict(R=48)]) == SHAPE
    assert qmany([{}, dict(x=None)]) == NULL
    assert qmany([dict(row=(P2, None))]) == NULL
    assert qmany([{}, dict(x=P + 8)]) == ALIGN
    assert qmany([{}], fmt=mx.E2M1, had=1) == FORMAT
    assert qmany([{}], pro=mx.PRO_DGELU_TANH) == NULL  # aux required


def test_quantize_many_valid_args_need_the_device():
    for items, kw in (([{}], {}), ([{}, dict(R=160, C=96), dict(R=0)], dict(fmt=mx.E2M3, had=1)),
                      ([dict(batch=8)] * 8, dict(fmt=mx.E4M3, mode=mx.RCEIL))):
        st = qmany(items, **kw)
        assert st in (OK, DEVICE)
        if not mx.lib().mx_device_supported(0):
            assert st == DEVICE

def g(fn="mx_gemm", **kw):
    a = dict(ac=P, as_=P2, bc=P3, bs=P4, M=256, N=512, K=768, fmt=mx.E2M3, bias=None, bt=mx.BF16, c=P5,
             ct=mx.BF16, ldc=512)
    a.update(kw)
    return getattr(mx.lib(), fn)(a["ac"], a["as_"], a["bc"], a["bs"], a["M"], a["N"], a["K"], a["fmt"], a["bias"],
                                 a["bt"], a["c"], a["ct"], a["ldc"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(ac=None), NULL), (dict(bs=None), NULL), (dict(c=None), NULL),
    (dict(fmt=5), FORMAT), (dict(bt=2), FORMAT), (dict(ct=3), FORMAT),
    (dict(M=128), SHAPE), (dict(N=300), SHAPE), (dict(K=384), SHAPE), (dict(M=-256), SHAPE),
    (dict(ldc=256), SHAPE), (dict(ldc=516), SHAPE),
    (dict(ac=P + 4), ALIGN), (dict(c=P5 + 2), ALIGN), (dict(bias=P6 + 8), ALIGN),
])
@pytest.mark.parametrize("fn", ["mx_gemm", "mx_gemm_accumulate"])
def test_gemm_rejections(fn, kw, want):
    assert g(fn, **kw) == want


@pytest.mark.parametrize("fn", ["mx_gemm", "mx_gemm_accumulate"])
def test_gemm_valid_args_need_the_device(fn):
    for kw in (dict(), dict(bias=P6, bt=mx.F32, ct=mx.F32, ldc=1024), dict(M=0), dict(K=0)):
        st = g(fn, **kw)
        assert st in (OK, DEVICE)
        if not mx.lib().mx_device_supported(0):
            assert st == DEVICE


def grouped(**kw):
    a = dict(mode=mx.RAGGED_M, epilogue=mx.EPI_NONE, fmt=mx.E4M3, scale_mode=mx.RCEIL, G=8,
             validate_offsets=0, R=32768, M=0, N=2048, K=768, offsets=P, A=(P2, P3), B=(P4, P5), C=P6, aux=None,
             out_row=(None, None), out_col=(None, None))
    a.update(kw)
    args = mx.GroupedArgs(a["mode"], a["epilogue"], a["fmt"], a["scale_mode"], a["G"], a["validate_offsets"],
                          a["R"], a["M"], a["N"], a["K"], a["offsets"], mx.Packed(*a["A"]), mx.Packed(*a["B"]),
                          a["C"], a["aux"], mx.Packed(*a["out_row"]), mx.Packed(*a["out_col"]))
    return mx.lib().mx_grouped_gemm(ctypes.byref(args), None)


@pytest.mark.parametrize("kw,want", [
    (dict(offsets=None), NULL), (dict(A=(P2, None)), NULL), (dict(C=None), NULL),
    (dict(epilogue=mx.EPI_SWIGLU), NULL),                          # quantization outputs missing
    (dict(epilogue=mx.EPI_DSWIGLU, C=None, out_row=(P7, P8), out_col=(P7, P8)), NULL),  # H missing
    (dict(mode=2), FORMAT), (dict(epilogue=3), FORMAT), (dict(fmt=0), FORMAT),
    (dict(mode=mx.RAGGED_K, epilogue=mx.EPI_SWIGLU, out_row=(P7, P8), out_col=(P7, P8)), FORMAT),
    (dict(epilogue=mx.EPI_SWIGLU, fmt=mx.E2M1, scale_mode=mx.RCEIL, out_row=(P7, P8), out_col=(P7, P8)), FORMAT),
    (dict(G=0), SHAPE), (dict(G=-1), SHAPE), (dict(R=1000), SHAPE), (dict(N=1000), SHAPE), (dict(K=100), SHAPE),
    (dict(K=384), SHAPE),                                          # K a multiple of 128 but not of 256
    (dict(mode=mx.RAGGED_K, M=100, N=256), SHAPE),
    (dict(offsets=P + 4), ALIGN), (dict(C=P6 + 2), ALIGN),
])
def test_grouped_rejections(kw, want):
    assert grouped(**kw) == want


def test_grouped_valid_args_need_the_device():
    for kw in (dict(), dict(mode=mx.RAGGED_K, M=2048, N=768), dict(R=0),
               dict(epilogue=mx.EPI_SWIGLU, N=1536, K=2048, out_row=(P7, P8), out_col=(P7, P8))):
        st = grouped(**kw)
        assert st in (OK, DEVICE)
        if not mx.lib().mx_device_supported(0):
            assert st == DEVICE


def mlp_fwd_args(**kw):
    base = dict(M=256, D=256, F=512, fmt=mx.E2M3, mode=mx.FLOOR, had=1)
    base.update(kw)
    packs = [mx.Packed(P * (10 + 2 * i), P * (11 + 2 * i)) for i in range(8)]
    return mx.MlpFwdArgs(base["M"], base["D"], base["F"], base["fmt"], base["mode"], base["had"], 0,
                         P, P2, None, P3, P4, P5, *packs)


def test_fused_mlp_rejections():
    L = mx.lib()
    assert L.mx_fused_mlp_fwd(None, None) == NULL
    assert L.mx_fused_mlp_fwd(ctypes.byref(mlp_fwd_args(M=100)), None) == SHAPE
    assert L.mx_fused_mlp_fwd(ctypes.byref(mlp_fwd_args(fmt=mx.E2M1, had=1)), None) == FORMAT
    a = mlp_fwd_args()
    a.Xr = mx.Packed(None, None)
    assert L.mx_fused_mlp_fwd(ctypes.byref(a), None) == NULL
    a = mlp_fwd_args()
    a.Y = P5 + 2
    assert L.mx_fused_mlp_fwd(ctypes.byref(a), None) == ALIGN
    st = L.mx_fused_mlp_fwd(ctypes.byref(mlp_fwd_args()), None)
    assert st in (OK, DEVICE)
    # X rows [M] x K=D in E4M3 past 2^31 bytes: the GEMM's 32-bit offsets cannot reach them
    assert L.mx_fused_mlp_fwd(ctypes.byref(mlp_fwd_args(M=1 << 20, D=4096, fmt=mx.E4M3, mode=mx.RCEIL, had=0)),
                              None) == OVERFLOW
    b = mx.MlpBwdArgs()
    assert L.mx_fused_mlp_bwd(ctypes.byref(b), None) == NULL


def mlp_bwd_args(**kw):
    base = dict(M=256, D=256, F=512, fmt=mx.E2M3, mode=mx.FLOOR, had=1, acc=0, db1=P6, part=P7)
    base.update(kw)
    packs = [mx.Packed(P * (10 + 2 * i), P * (11 + 2 * i)) for i in range(8)]
    return mx.MlpBwdArgs(base["M"], base["D"], base["F"], base["fmt"], base["mode"], base["had"], base["acc"],
                         P, P2, *packs[:4], P3, P4, P5, P8, base["db1"], base["part"], *packs[4:])


@pytest.mark.parametrize("kw,want", [
    (dict(M=100), SHAPE), (dict(D=0, F=300), SHAPE), (dict(F=-256), SHAPE),
    (dict(fmt=mx.E2M1, had=1), FORMAT), (dict(fmt=mx.E2M3, mode=mx.RCEIL), FORMAT), (dict(fmt=7), FORMAT),
    (dict(acc=2), FORMAT),
    (dict(part=None), NULL),                                  # a bias gradient needs its partials buffer
    (dict(db1=P6 + 4), ALIGN), (dict(part=P7 + 8), ALIGN),
    (dict(M=1 << 20, D=4096, fmt=mx.E4M3, mode=mx.RCEIL, had=0), OVERFLOW),
])
def test_fused_mlp_bwd_rejections(kw, want):
    assert mx.lib().mx_fused_mlp_bwd(ctypes.byref(mlp_bwd_args(**kw)), None) == want


def test_fused_mlp_bwd_rejects_each_missing_pointer_and_misaligned_pack():
    L = mx.lib()
    for name in ("dY", "h", "da", "dX", "dW1", "dW2"):
        a = mlp_bwd_args()
        setattr(a, name, None)
        assert L.mx_fused_mlp_bwd(ctypes.byref(a), None) == NULL, name
    for name in ("Xc", "W1c", "W2c", "ac", "dYr", "dYc", "dhr", "dhc"):
        a = mlp_bwd_args()
        setattr(a, name, mx.Packed(P, None))
        assert L.mx_fused_mlp_bwd(ctypes.byref(a), None) == NULL, name
        a = mlp_bwd_args()
        setattr(a, name, mx.Packed(P + 4, P2))
        assert L.mx_fused_mlp_bwd(ctypes.byref(a), None) == ALIGN, name


def test_fused_mlp_bwd_valid_args_need_the_device():
    for kw in (dict(), dict(db1=None, part=None), dict(acc=1), dict(M=0)):
        st = mx.lib().mx_fused_mlp_bwd(ctypes.byref(mlp_bwd_args(**kw)), None)
        assert st in (OK, DEVICE), kw
        if not mx.lib().mx_device_supported(0):
            assert st == DEVICE


def gt(tile_m, tile_n, occ=1, M=768, N=768, K=512):
    return mx.lib().mx_gemm_tiled(P, P2, P3, P4, M, N, K, mx.E2M1, None, mx.BF16, P5, mx.BF16, N, tile_m, tile_n, occ,
                                  None)


def test_gemm_tiled_rejects_shapes_it_cannot_serve():
    assert gt(128, 128) == SHAPE                  # not one of the tile shapes
    assert gt(256, 192, M=512, N=768) == OK or gt(256, 192, M=512, N=768) == DEVICE
    assert gt(192, 256, M=512, N=768) == SHAPE    # 192 does not divide M = 512
    assert gt(256, 64) == SHAPE
    assert gt(256, 256, 2) == SHAPE and gt(256, 128, 3) == SHAPE and gt(0, 0, 1) == SHAPE
    for tile in ((0, 0, 0), (256, 256, 1), (256, 192, 1), (192, 256, 1), (192, 192, 1), (256, 128, 1),
                 (256, 128, 2), (128, 256, 2), (192, 192, 2)):
        st = gt(*tile)
        assert st in (OK, DEVICE), tile
        if not mx.lib().mx_device_supported(0):
            assert st == DEVICE


def gs(split_k, ws=P6, ws_bytes=None, tile=(0, 0, 0), M=768, N=768, K=1536):
    nb = split_k * M * N * 4 if ws_bytes is None else ws_bytes
    return mx.lib().mx_gemm_splitk(P, P2, P3, P4, M, N, K, mx.E2M1, None, mx.BF16, P5, mx.BF16, N, tile[0], tile[1],
                                   tile[2], split_k, ws, nb, None)


def test_gemm_splitk_rejects_what_it_cannot_serve():
    ok = (OK, DEVICE)
    assert gs(2) in ok and gs(3) in ok and gs(4) in ok and gs(12) in ok  # K = 1536 = 128 * 12
    assert gs(1, ws=None, ws_bytes=0) in ok       # no split: no workspace
    assert gs(0) == SHAPE and gs(17) == SHAPE     # 1 .. MX_SPLIT_K_MAX
    assert gs(5) == SHAPE and gs(16) == SHAPE     # K not a multiple of 128 * split_k
    assert gs(2, ws=None) == NULL                 # a split needs the workspace
    assert gs(2, ws=P6 + 8) == ALIGN
    assert gs(2, ws_bytes=2 * 768 * 768 * 4 - 1) == SHAPE
    assert gs(2, tile=(128, 128, 1)) == SHAPE     # not a tile shape
    assert gs(2, tile=(192, 256, 1), M=512) == SHAPE
    assert gs(2, tile=(128, 256, 2)) in ok
    if not mx.lib().mx_device_supported(0):
        assert gs(2) == DEVICE


def test_gemm_plan_without_a_tuned_entry_is_the_rule():
    # a shape no tuned entry names gets mx_gemm's rule and no split: the
    # tile with the fewest rounds x tile area on this device's compute units
    tile, split, ws = mx.gemm_plan(4096 + 256 * 7, 2304, 2816, mx.E2M3)
    assert split == 1 and ws == 0 and tile[2] == 1
    assert tile in ((256, 256, 1), (256, 192, 1), (192, 256, 1), (192, 192, 1), (256, 128, 1))
    L = mx.lib()
    plan = (ctypes.c_int * 4)()
    assert L.mx_gemm_plan(512, 512, 500, mx.E2M1, plan, None) == SHAPE
    assert L.mx_gemm_plan(512, 512, 512, 9, plan, None) == FORMAT
    assert L.mx_gemm_plan(512, 512, 512, mx.E2M1, None, None) == NULL
    assert L.mx_gemm_plan(512, 512, 512, mx.E2M1, plan, None) == OK


def test_tuned_table_entries_are_servable():
    # every line of the tuned table names a tiling mx_gemm_tiled accepts and
    # a split that divides K into 128-element groups
    src = open(os.path.join(ROOT, "microscaling_block_scaled_mx_amd", "csrc", "mx_tuned.inc")).read()
    rows = re.findall(r"\{(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*\{(\d+),\s*(\d+),\s*(\d+),\s*(\d+)\}\}", src)
    shapes = {(256, 256, 1), (256, 192, 1), (192, 256, 1), (192, 192, 1), (256, 128, 1), (256, 128, 2), (128, 256, 2),
              (192, 192, 2)}
    seen = set()
    for r in rows:
        cus, fmt, M, N, K, tm, tn, wg, split = (int(v) for v in r)
        assert cus > 0 and fmt in (mx.E2M1, mx.E2M3, mx.E4M3)
        assert (tm, tn, wg) in shapes and M % tm == 0 and N % tn == 0
        assert 1 <= split <= 16 and K % (128 * split) == 0
        assert (cus, fmt, M, N, K) not in seen
        seen.add((cus, fmt, M, N, K))


def test_binding_refuses_host_tensors_and_strided_views():
    # buffers of sufficient size that the kernels could not read correctly:
    # a host tensor (its address is not device memory) and a strided view
    import torch
    M, N, K = 256, 256, 256
    a, b = mx.alloc_packed(M, K, mx.E2M1, device="cpu"), mx.alloc_packed(N, K, mx.E2M1, device="cpu")
    C = torch.empty(M, N, dtype=torch.int16)
    with pytest.raises(mx.MXError) as e:
        mx.gemm(a, b, M, N, K, mx.E2M1, C)
    assert e.value.status == DEVICE and "not on a GPU" in str(e.value)
    with pytest.raises(mx.MXError) as e:
        mx.quantize(torch.empty(K, M, dtype=torch.int16).t(), M, K, mx.E2M1, mx.FLOOR, row=a)
    assert e.value.status == SHAPE and "strided view" in str(e.value)


def test_binding_rejects_short_buffers_before_the_call():
    # Buffers packed for E2M1 are half the size an E4M3 call touches: the
    # binding must refuse before the C ABI (which sees only pointers) runs.
    import torch
    M, N, K = 256, 256, 512
    small = mx.alloc_packed(M, K, mx.E2M1, device="cpu")
    b = mx.alloc_packed(N, K, mx.E4M3, device="cpu")
    C = torch.empty(M, N, dtype=torch.int16)
    with pytest.raises(mx.MXError, match="gemm A codes"):
        mx.gemm(small, b, M, N, K, mx.E4M3, C)
    with pytest.raises(mx.MXError, match="gemm C"):
        mx.gemm(mx.alloc_packed(M, K, mx.E4M3, device="cpu"), b, M, N, K, mx.E4M3, C[:128])
    with pytest.raises(mx.MXError, match="quantize row codes"):
        mx.quantize(torch.empty(M, K, dtype=torch.int16), M, K, mx.E4M3, mx.RCEIL, row=small)
    off = torch.tensor([M], dtype=torch.int32)
    with pytest.raises(mx.MXError, match="grouped A codes"):
        mx.grouped_gemm(mx.RAGGED_M, 1, M, off, small, b, C, N=N, K=K)


def gmany(items, n=None, fmt=mx.E2M1):
    arr = (mx.GemmItem * max(len(items), 1))()
    for k, it in enumerate(items):
        a = dict(A=(P, P2), B=(P3, P4), M=256, N=256, K=256, bias=None, bias_dtype=mx.BF16, c_dtype=mx.BF16, C=P5,
                 ldc=256, accumulate=0)
        a.update(it)
        arr[k] = mx.GemmItem(mx.Packed(*a["A"]), mx.Packed(*a["B"]), a["M"], a["N"], a["K"], a["bias"],
                             a["bias_dtype"], a["c_dtype"], a["C"], a["ldc"], a["accumulate"], 0)
    return mx.lib().mx_gemm_many(arr, len(items) if n is None else n, fmt, None)


def test_gemm_many_rejections():
    assert mx.lib().mx_gemm_many(None, 1, mx.E2M1, None) == NULL
    assert gmany([{}], n=0) == SHAPE
    assert gmany([{}] * 5) == SHAPE  # more than MX_GEMM_MANY_MAX
    assert gmany([{}, dict(M=100)]) == SHAPE
    assert gmany([{}, dict(ldc=128)]) == SHAPE
    assert gmany([{}, dict(C=None)]) == NULL
    assert gmany([dict(B=(P3, None))]) == NULL
    assert gmany([{}, dict(C=P5 + 2)]) == ALIGN
    assert gmany([{}], fmt=5) == FORMAT
    assert gmany([dict(c_dtype=7)]) == FORMAT
    assert gmany([{}, dict(accumulate=2)]) == FORMAT


def test_gemm_many_valid_args_need_the_device():
    for items, fmt in (([{}], mx.E2M1), ([{}, dict(M=4096, N=3072, K=3072, ldc=3072), dict(M=0)], mx.E2M3),
                       ([dict(bias=P6, bias_dtype=mx.F32, c_dtype=mx.F32)] * 4, mx.E4M3),
                       ([{}, dict(accumulate=1)], mx.E2M1)):
        st = gmany(items, fmt=fmt)
        assert st in (OK, DEVICE)
        if not mx.lib().mx_device_supported(0):
            assert st == DEVICE


def qna(**kw):
    a = dict(x=P, aux=None, batch=1, R=64, C=128, fmt=mx.E2M1, mode=mx.FLOOR, had=0, pro=mx.PRO_IDENTITY,
             rc=P2, rs=P3, cc=P4, cs=P5, sum=P6)
    a.update(kw)
    return mx.lib().mx_quantize_noalloc(a["x"], a["aux"], a["batch"], a["R"], a["C"], a["fmt"], a["mode"],
                                        a["had"], a["pro"], a["rc"], a["rs"], a["cc"], a["cs"], a["sum"], None)


SCRATCH = 9


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(rc=None), NULL), (dict(rc=None, rs=None, cc=None, cs=None, sum=None), NULL),
    (dict(pro=mx.PRO_DGELU_TANH), NULL), (dict(fmt=mx.E2M1, had=1), FORMAT), (dict(R=48), SHAPE),
    (dict(sum=P6 + 4), ALIGN),
    # partials of (R/32) * C * batch floats past the 16 MiB static array
    (dict(R=8192, C=16384 + 32), SCRATCH), (dict(batch=3, R=4096, C=16384), SCRATCH),
])
def test_quantize_noalloc_rejections(kw, want):
    assert qna(**kw) == want


def test_quantize_noalloc_valid_args_need_the_device():
    # the largest call the array holds, no colsum (no scratch), and R = 0
    for kw in (dict(), dict(R=8192, C=16384), dict(sum=None), dict(R=0), dict(batch=2, R=4096, C=16384)):
        st = qna(**kw)
        assert st in (OK, DEVICE), (kw, st)
        if not mx.lib().mx_device_supported(0):
            assert st == DEVICE


def qsr(**kw):
    a = dict(x=P, batch=1, R=64, C=128, rc=P2, rs=P3, cc=P4, cs=P5, part=None, sum=None, seed=1)
    a.update(kw)
    return mx.lib().mx_quantize_sr(a["x"], a["batch"], a["R"], a["C"], a["rc"], a["rs"], a["cc"], a["cs"],
                                   a["part"], a["sum"], a["seed"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(rc=None), NULL), (dict(rc=None, rs=None, cc=None, cs=None), NULL),
    (dict(sum=P6), NULL),
    (dict(R=48), SHAPE), (dict(C=40), SHAPE), (dict(batch=0), SHAPE),
    (dict(x=P + 8), ALIGN), (dict(cs=P5 + 4), ALIGN),
    (dict(batch=70000), OVERFLOW),
])
def test_quantize_sr_rejections(kw, want):
    assert qsr(**kw) == want


def test_quantize_sr_valid_args_need_the_device():
    for kw in (dict(), dict(seed=2**64 - 1), dict(R=0), dict(cc=None, cs=None, part=P6, sum=P7)):
        st = qsr(**kw)
        assert st in (OK, DEVICE), (kw, st)
        if not mx.lib().mx_device_supported(0):
            assert st == DEVICE


def test_binding_quantize_sr_rejects_short_buffers():
    import torch
    R, C = 64, 128
    small = (torch.empty(8, dtype=torch.uint8), torch.empty(8, dtype=torch.uint8))
    with pytest.raises(mx.MXError, match="quantize_sr row"):
        mx.quantize_sr(torch.empty(R, C, dtype=torch.int16), R, C, 1, row=small)


def test_clock_sample_rejections():
    L = mx.lib()
    assert L.mx_clock_sample(100, None, None) == NULL
    assert L.mx_clock_sample(100, P + 8, None) == ALIGN
    assert L.mx_clock_sample(0, P, None) == SHAPE and L.mx_clock_sample(2_000_000, P, None) == SHAPE
    st = L.mx_clock_sample(100, P, None)
    assert st in (OK, DEVICE)
    if not L.mx_device_supported(0):
        assert st == DEVICE
