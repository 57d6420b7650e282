"""The comparisons the parity tests make, in one place, so that the
negative controls (tests/test_negative_controls.py) exercise exactly the
checks the GPU tests rely on.

Bars: packed codes, scales and column sums bit-exact; a GEMM output within
max|got - ref| <= 2e-3 * max|ref| of the oracle's unrounded binary64 result
(infinity-norm relative error: elementwise relative error is ill-posed
under cancellation); a bf16 output additionally allowed the half ulp of its
one rounding."""
import numpy as np

REL = 2e-3


def bf16_to_f64(u16) -> np.ndarray:
    return (np.ascontiguousarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_rel_err(got, ref64) -> float:
    """max|got - ref| / max|ref| for a binary32 or binary64 result."""
    g = np.asarray(got, np.float64)
    return float(np.max(np.abs(g - ref64)) / max(np.max(np.abs(ref64)), 1e-300))


def gemm_close(got, ref64, rel=REL) -> bool:
    return gemm_rel_err(got, ref64) <= rel


def bf16_rel_err(got_bf16, ref64) -> float:
    return gemm_rel_err(bf16_to_f64(got_bf16), ref64)


def bf16_close(got_bf16, ref64, rel=REL) -> bool:
    """|got - ref| <= rel * max|ref| + half a bf16 ulp of ref, elementwise."""
    g = bf16_to_f64(got_bf16)
    half_ulp = np.abs(ref64) * 2.0 ** -8
    return bool(np.all(np.abs(g - ref64) <= rel * np.max(np.abs(ref64)) + half_ulp))


def pack_mismatches(got: dict, want: dict, keys) -> dict:
    """Number of differing bytes per key (shape mismatches count as all)."""
    out = {}
    for k in keys:
        g, w = np.asarray(got[k]), np.asarray(want[k])
        if g.shape != w.shape:
            out[k] = max(g.size, w.size)
            continue
        n = int(np.count_nonzero(g.view(np.uint8) != w.view(np.uint8)))
        if n:
            out[k] = n
    return out


def packs_equal(got: dict, want: dict, keys) -> bool:
    return not pack_mismatches(got, want, keys)


def assert_packs_equal(got: dict, want: dict, keys):
    bad = pack_mismatches(got, want, keys)
    assert not bad, f"mismatching bytes per array: {bad}"
