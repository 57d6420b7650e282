"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- numbers the pages print, closed forms, invariants, library
routines that a special case reduces to, or exact brute force on tiny inputs.
CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from microscaling_block_scaled_mx_amd import inputs as I

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
BF16_F32 = I.bf16_bits_to_f32(ALL_BF16)
FINITE = np.isfinite(BF16_F32)


def exact(x) -> Fraction:
    return Fraction(float(x))


# ------------------------------------------------------------------ formats
def test_e2m1_grid(orc):
    # E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; the sign bit is bit 3.
    assert [orc.decode(orc.E2M1, c) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert [orc.decode(orc.E2M1, c | 8) for c in range(8)] == [-v for v in [0, 0.5, 1, 1.5, 2, 3, 4, 6]]
    assert math.copysign(1, orc.decode(orc.E2M1, 8)) == -1.0


def test_e2m3_grid(orc):
    vals = [orc.decode(orc.E2M3, c) for c in range(32)]
    assert max(vals) == 7.5 and vals[31] == 7.5
    assert vals[1] == 0.125  # smallest subnormal
    # strictly increasing over the positive codes, steps 1/8 below 2, 1/4 below 4, 1/2 below 7.5
    diffs = np.diff(vals)
    assert np.all(diffs[:16] == 0.125) and np.all(diffs[16:24] == 0.25) and np.all(diffs[24:] == 0.5)


def test_e4m3_decode_matches_torch(orc):
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ours = np.array([orc.decode(orc.E4M3, c) for c in range(256)])
    nan = np.isnan(b)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(b[~nan], ours[~nan])
    assert orc.decode(orc.E4M3, 0x7E) == 448.0


@pytest.mark.parametrize("fmt,n", [(1, 16), (2, 64), (3, 256)])
def test_representable_values_round_trip(orc, fmt, n):
    for c in range(n):
        v = orc.decode(fmt, c)
        if math.isnan(v):
            continue
        assert orc.encode(fmt, v) == c, (fmt, c, v)


def brute_nearest(grid_codes, grid_vals, a: Fraction):
    """Nearest representable magnitude by exhaustive comparison; ties to the
    even code; saturate at the top."""
    if a >= grid_vals[-1]:
        return grid_codes[-1]
    best = None
    for c, g in zip(grid_codes, grid_vals):
        d = abs(a - g)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


@pytest.mark.parametrize("fmt,n", [(1, 8), (2, 32)])
def test_small_format_encode_brute_force(orc, fmt, n):
    codes = list(range(n))
    vals = [exact(orc.decode(fmt, c)) for c in codes]
    probes = set()
    for i in range(n - 1):  # every midpoint, and its neighbours
        mid = (vals[i] + vals[i + 1]) / 2
        for d in (Fraction(0), Fraction(1, 1 << 20), -Fraction(1, 1 << 20)):
            probes.add(mid + d)
    rng = np.random.default_rng(0)
    for v in rng.uniform(0, 9, 2000):
        probes.add(exact(v))
    probes |= {Fraction(7), Fraction(8) - Fraction(1, 1 << 20), Fraction(100)}
    sign = 8 if fmt == 1 else 32
    for a in probes:
        want = brute_nearest(codes, vals, a)
        assert orc.encode(fmt, float(a)) == want, (fmt, a)
        assert orc.encode(fmt, -float(a)) == want | sign


def test_e4m3_encode_matches_torch_on_all_bf16(orc):
    # torch's cast is nearest-even (non-saturating); below 448 the two agree.
    sel = FINITE & (np.abs(BF16_F32) <= 448.0)
    xs = BF16_F32[sel]
    want = torch.from_numpy(xs.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.encode(orc.E4M3, float(v)) for v in xs], np.uint8)
    assert np.array_equal(got, want)
    # beyond the largest finite magnitude the oracle saturates
    assert orc.encode(orc.E4M3, 480.0) == 0x7E and orc.encode(orc.E4M3, -1e6) == 0xFE


def test_negative_zero_kept(orc):
    assert orc.encode(orc.E2M1, -0.1) == 0x8
    assert orc.encode(orc.E2M3, -0.01) == 0x20
    assert orc.encode(orc.E4M3, -1e-5) == 0x80


# ------------------------------------------------------------------ E8M0 scales
def test_floor_scale_definition(orc):
    # For every positive finite bf16 amax not hitting the clamp:
    # 2^2 <= amax * 2^-X < 2^3 (emax of E2M1 and E2M3 is 2).
    pos = BF16_F32[FINITE & (BF16_F32 > 0)]
    for fmt in (orc.E2M1, orc.E2M3):
        for a in pos[::7]:
            b = orc.scale_floor(fmt, float(a))
            X = b - 127
            v = exact(a) / Fraction(2) ** X if X >= 0 else exact(a) * Fraction(2) ** (-X)
            if X == -127:
                assert v < 8
            else:
                assert 4 <= v < 8, (a, b)
    assert orc.scale_floor(orc.E2M1, 0.0) == 0
    assert orc.scale_floor(orc.E2M1, float("nan")) == 0xFF
    assert orc.scale_floor(orc.E2M1, float("inf")) == 0xFF
    assert orc.scale_floor(orc.E2M1, 6.0) == 127 and orc.scale_floor(orc.E2M1, 7.99) == 127
    assert orc.scale_floor(orc.E2M1, 8.0) == 128 and orc.scale_floor(orc.E2M1, 3.99) == 126


def test_rceil_is_exact_ceiling_on_all_bf16(orc):
    # RCEIL: the smallest X with 448 * 2^X >= amax, for every positive finite
    # bf16 amax (the oracle computes it from fl32(amax / 448); this checks the
    # exact rational definition).  torch's float8_e8m0fnu cast is not used as
    # a reference: it rounds to nearest (1.4999 -> 2^0, 1.5 -> 2^1).
    pos = BF16_F32[FINITE & (BF16_F32 > 0)]
    two = Fraction(2)
    for a in pos:
        b = orc.scale_rceil(float(a))
        X = int(b) - 127
        if X == -127:
            assert exact(a) <= 448 * two ** -127
            continue
        assert 448 * two ** X >= exact(a) > 448 * two ** (X - 1), (a, b)
    assert orc.scale_rceil(0.0) == 0 and orc.scale_rceil(float("nan")) == 0xFF
    assert orc.scale_rceil(448.0) == 127 and orc.scale_rceil(449.0) == 128
    assert orc.scale_rceil(float("inf")) == 0xFF


# ------------------------------------------------------------------ Hadamard
def test_hadamard_orthogonality(orc):
    c = orc.hadamard_c()
    # c = fl32(1/sqrt(32)), bit pattern 0x3E3504F3; nearest binary32 to 2^-2.5
    assert np.float32(c).view(np.uint32) == 0x3E3504F3
    H = np.zeros((32, 32), np.int64)
    for j in range(32):
        e = np.zeros(32, np.float32)
        e[j] = 1.0
        r = orc.hadamard32(e)
        assert np.all(np.abs(r) == np.float32(c))
        H[:, j] = np.sign(r).astype(np.int64)
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=np.int64))
    assert np.array_equal(H, H.T)
    assert np.all(H[0] == 1) and np.all(H[:, 0] == 1)


def fwht_butterfly(x: np.ndarray) -> np.ndarray:
    """Radix-2 in-place fast Walsh-Hadamard transform in binary32,
    strides 1, 2, 4, 8, 16 (a+b, a-b), then one multiply by c."""
    y = x.astype(np.float32).copy()
    h = 1
    while h < 32:
        for i in range(0, 32, 2 * h):
            for j in range(i, i + h):
                a, b = y[j], y[j + h]
                y[j], y[j + h] = np.float32(a + b), np.float32(a - b)
        h *= 2
    return (y * np.float32(1.0 / math.sqrt(32.0))).astype(np.float32)


def test_hadamard_pairwise_equals_butterfly_and_bound(orc):
    rng = np.random.default_rng(1)
    Hm = np.array([[(-1) ** bin(i & j).count("1") for j in range(32)] for i in range(32)], np.float64)
    for t in range(300):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 3, 32)).astype(np.float32)
        r = orc.hadamard32(x)
        assert np.array_equal(r, fwht_butterfly(x)), t
        ex = Hm @ x.astype(np.float64) / math.sqrt(32.0)
        bound = 7 * 2.0 ** -24 * np.sum(np.abs(x)) / math.sqrt(32.0)
        assert np.all(np.abs(r - ex) <= bound)
        # energy preserved (orthogonal up to rounding)
        assert abs(np.sum(r.astype(np.float64) ** 2) - np.sum(x.astype(np.float64) ** 2)) <= \
            1e-5 * np.sum(x.astype(np.float64) ** 2)


# ------------------------------------------------------------------ activations
def f32(x):
    return float(np.float32(x))


def ulp32(x):
    x = abs(np.float32(x))
    return float(np.spacing(x))


def test_exp_within_2ulp_of_libm(orc):
    xs = np.concatenate([np.linspace(-87.0, 88.7, 20001, dtype=np.float32),
                         np.float32([0.0, -0.0, 1e-8, -1e-8, 0.5, -0.5])])
    for x in xs:
        e = orc.exp(float(x))
        ref = math.exp(float(x))
        assert abs(e - ref) <= 2 * ulp32(ref), (x, e, ref)
    assert orc.exp(0.0) == 1.0
    assert orc.exp(-90.0) == 0.0 and orc.exp(89.5) == math.inf and math.isnan(orc.exp(math.nan))


def test_one_plus_tanh_relative_error(orc):
    # 1 + tanh(u) is accurate in both tails (no cancellation)
    for x in np.linspace(-40, 12, 5201, dtype=np.float32):
        xf = float(x)
        # closed form without cancellation: 1 + tanh(x) = 2 / (exp(-2x) + 1)
        ref = 2.0 / (math.exp(-2.0 * xf) + 1.0) if xf > -300 else 0.0
        got = orc.one_plus_tanh(xf)
        assert abs(got - ref) <= 8 * 2.0 ** -24 * ref + 2.0 ** -125, (x, got, ref)
    assert orc.one_plus_tanh(0.0) == 1.0 and orc.one_plus_tanh(50.0) == 2.0
    assert orc.one_plus_tanh(-60.0) == 0.0


def bf16_round_f64(v: float) -> float:
    """Nearest-even bf16 of a real number given in binary64 (test-side helper)."""
    f = np.float64(v)
    if not np.isfinite(f):
        return float(f)
    m, e = math.frexp(f)
    q = Fraction(f)
    step = Fraction(2) ** (e - 8)  # 8 significant bits
    if e - 8 < -133:
        step = Fraction(2) ** -133
    n = q / step
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return float(fl * step)


def gelu64(x):
    # binary64 reference; 1 + tanh(u) = 2 / (1 + exp(-2u)) has no cancellation
    k0 = math.sqrt(2 / math.pi)
    u = k0 * (x + 0.044715 * x ** 3)
    return 0.5 * x * (2.0 / (1.0 + math.exp(-2.0 * u)) if u > -350 else 0.0)


def test_gelu_against_fp64(orc):
    sel = FINITE & (np.abs(BF16_F32) <= 16.0) & (np.abs(BF16_F32) >= 2.0 ** -20)
    xs_bits = ALL_BF16[sel]
    mism = 0
    for b in xs_bits[::3]:
        x = float(I.bf16_bits_to_f32(np.array([b]))[0])
        got = float(I.bf16_bits_to_f32(np.array([orc.gelu_bf16(int(b))], np.uint16))[0])
        ref = gelu64(x)
        want = bf16_round_f64(ref)
        if got != want:
            mism += 1
            # only a near-tie may round the other way (within one bf16 ulp);
            # results under 2^-126 may flush (exp's contract has no subnormals)
            assert abs(got - ref) <= abs(want - ref) + 2.0 ** -7 * abs(ref) + 2.0 ** -126, (x, got, ref)
    assert mism <= 0.01 * len(xs_bits[::3])


def test_dgelu_against_fp64(orc):
    k0, k1 = math.sqrt(2 / math.pi), 0.044715
    rng = np.random.default_rng(3)
    hs = I.f32_to_bf16_bits(rng.standard_normal(4000).astype(np.float32) * 3)
    das = I.f32_to_bf16_bits(rng.standard_normal(4000).astype(np.float32))
    for hb, db in zip(hs, das):
        x = float(I.bf16_bits_to_f32(np.array([hb]))[0])
        da = float(I.bf16_bits_to_f32(np.array([db]))[0])
        t = math.tanh(k0 * (x + k1 * x ** 3))
        d = 0.5 * (1 + t) + 0.5 * x * (1 - t * t) * k0 * (1 + 3 * k1 * x * x)
        ref = da * d
        got = float(I.bf16_bits_to_f32(np.array([orc.dgelu_bf16(int(db), int(hb))], np.uint16))[0])
        assert abs(got - ref) <= 2.0 ** -8 * abs(ref) + 1e-6 * abs(da), (x, da, got, ref)


def test_swiglu_against_fp64_and_saturated_gate(orc):
    rng = np.random.default_rng(4)
    gs = I.f32_to_bf16_bits(rng.standard_normal(3000).astype(np.float32) * 4)
    us = I.f32_to_bf16_bits(rng.standard_normal(3000).astype(np.float32))
    dz = I.f32_to_bf16_bits(rng.standard_normal(3000).astype(np.float32))
    for gb, ub, db in zip(gs, us, dz):
        g, u, d = (float(I.bf16_bits_to_f32(np.array([v]))[0]) for v in (gb, ub, db))
        s = 1 / (1 + math.exp(-g))
        z = g * s * u
        got = float(I.bf16_bits_to_f32(np.array([orc.swiglu_bf16(int(gb), int(ub))], np.uint16))[0])
        assert abs(got - z) <= 2.0 ** -8 * abs(z) + 1e-30
        dgate, dup = orc.dswiglu_bf16(int(db), int(gb), int(ub))
        dgate = float(I.bf16_bits_to_f32(np.array([dgate], np.uint16))[0])
        dup = float(I.bf16_bits_to_f32(np.array([dup], np.uint16))[0])
        rg = d * u * s * (1 + g * (1 - s))
        ru = d * g * s
        assert abs(dup - ru) <= 2.0 ** -8 * abs(ru) + 1e-30
        assert abs(dgate - rg) <= 2.0 ** -8 * abs(rg) + 2.0 ** -20 * abs(d * u)
    # saturated gate: exp(-g) < 2^-25 -> s == 1 exactly -> z = bf16(g*u), an exact-product rounding
    for g in (20.0, 32.0, 100.0):
        for u in (1.5, -3.0, 0.15625):
            gb = int(I.f32_to_bf16_bits(np.float32([g]))[0])
            ub = int(I.f32_to_bf16_bits(np.float32([u]))[0])
            z = orc.swiglu_bf16(gb, ub)
            assert z == int(I.f32_to_bf16_bits(np.float32([np.float32(g) * np.float32(u)]))[0])


# ------------------------------------------------------------------ quantize
def deq_rows(orc, codes, scales, fmt, k):
    c = orc.unpack_codes(codes, fmt, k)
    table = np.array([orc.decode(fmt, i) for i in range(1 << orc.BITS[fmt])])
    return table[c] * np.exp2(np.repeat(scales.astype(np.int64) - 127, 32, axis=1))


def test_quantize_special_blocks(orc):
    x = np.zeros((32, 128), np.float32)
    x[:, 32:64] = np.nan
    x[:, 64:96] = np.inf
    x[5, 96:128] = 3.0
    xb = I.f32_to_bf16_bits(x)
    x2 = xb.copy()
    x2[:, 10] = 0x8000  # -0.0 in an otherwise zero block
    for fmt, mode in ((1, 0), (2, 0), (3, 1)):
        q = orc.quantize(x2, 32, 128, fmt, mode, hadamard=False, row=True, col=True)
        rs = q["row_scales"]
        assert np.all(rs[:, 0] == 0) and np.all(rs[:, 1] == 0xFF) and np.all(rs[:, 2] == 0xFF)
        codes = orc.unpack_codes(q["row_codes"], fmt, 128)
        assert np.all(codes[:, 32:96] == 0)
        sign = {1: 8, 2: 32, 3: 128}[fmt]
        assert np.all(codes[:, 10] == sign) and np.all(codes[:, :10] == 0)


def test_quantize_representable_blocks_round_trip(orc):
    # blocks made of representable values times a power of two come back exactly
    rng = np.random.default_rng(5)
    for fmt, mode in ((1, 0), (2, 0), (3, 1)):
        n = 1 << orc.BITS[fmt]
        vals = np.array([orc.decode(fmt, c) for c in range(n)])
        ok = np.isfinite(vals)
        R, C = 64, 256
        codes = rng.choice(np.arange(n)[ok], size=(R, C))
        x = vals[codes]
        top = np.max(vals[ok])
        x[:, ::32] = top  # pin each block's amax to the format maximum
        exps = rng.integers(-20, 20, size=(R, C // 32))
        x = x * np.exp2(np.repeat(exps, 32, axis=1))
        xb = I.f32_to_bf16_bits(x.astype(np.float32))
        assert np.array_equal(I.bf16_bits_to_f32(xb).astype(np.float64), x)  # inputs exact in bf16
        q = orc.quantize(xb, R, C, fmt, mode)
        back = deq_rows(orc, q["row_codes"], q["row_scales"], fmt, C)
        assert np.array_equal(back, x), fmt


def test_col_mode_is_row_mode_of_transpose(orc):
    X, W, dY = I.linear(7, 64, 96, 128)
    for fmt, mode, had in ((1, 0, False), (2, 0, True), (3, 1, False)):
        q = orc.quantize(X, 64, 128, fmt, mode, had, row=True, col=True)
        qt = orc.quantize(np.ascontiguousarray(X.T), 128, 64, fmt, mode, had, row=True, col=False)
        assert np.array_equal(q["col_codes"], qt["row_codes"])
        assert np.array_equal(q["col_scales"], qt["row_scales"])


def test_colsum_exact_on_integers_and_single_block(orc):
    rng = np.random.default_rng(6)
    R, C = 256, 64
    xi = rng.integers(-100, 100, size=(R, C)).astype(np.float32)
    q = orc.quantize(I.f32_to_bf16_bits(xi), R, C, 1, 0, colsum=True, row=False)
    assert np.array_equal(q["colsum"], xi.sum(0))
    assert np.array_equal(q["colsum_partials"], xi.reshape(R // 32, 32, C).sum(1))
    # R == 32: a plain sequential binary32 sum of the column
    x = rng.standard_normal((32, C)).astype(np.float32)
    xb = I.f32_to_bf16_bits(x)
    xf = I.bf16_bits_to_f32(xb)
    q = orc.quantize(xb, 32, C, 1, 0, colsum=True, row=False)
    for c in range(C):
        s = np.float32(0)
        for r in range(32):
            s = np.float32(s + xf[r, c])
        assert q["colsum"][c] == s


def test_mxfp8_quantizer_snr_matches_page(orc):
    g = GOLDEN["mxfp8_rceil_quantizer_snr_db"]
    X = I.bf16_normal(np.random.default_rng(11), (512, 2048))
    q = orc.quantize(X, 512, 2048, orc.E4M3, orc.RCEIL)
    back = deq_rows(orc, q["row_codes"], q["row_scales"], orc.E4M3, 2048)
    xf = I.bf16_bits_to_f32(X).astype(np.float64)
    snr = 10 * np.log10(np.sum(xf ** 2) / np.sum((xf - back) ** 2))
    assert abs(snr - g["value"]) <= g["tolerance_db"], snr


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("narrow", [True, False])
def test_gemm_exact_bruteforce_small(orc, narrow):
    # narrow: all terms of a dot product fit binary64's 53-bit window, so the
    # binary64 sum must equal the exact rational sum; wide: scales spread over
    # ~100 binades, so only the binary64 error bound holds.
    rng = np.random.default_rng(8)
    for fmt in (1, 2, 3):
        n = 1 << orc.BITS[fmt]
        vals = [orc.decode(fmt, c) for c in range(n)]
        okc = [c for c in range(n) if not math.isnan(vals[c])]
        for K in (32, 64):
            M, N = 3, 4
            ca = rng.choice(okc, size=(M, K))
            cb = rng.choice(okc, size=(N, K))
            lo, hi = ((125, 130) if narrow else (100, 150))
            sa = rng.integers(lo, hi, size=(M, K // 32)).astype(np.uint8)
            sb = rng.integers(lo, hi, size=(N, K // 32)).astype(np.uint8)
            pa = np.zeros((M, K * orc.BITS[fmt] // 8), np.uint8)
            pb = np.zeros((N, K * orc.BITS[fmt] // 8), np.uint8)
            # pack through a quantize-free path: write codes bit by bit
            for arr, codes in ((pa, ca), (pb, cb)):
                for r in range(arr.shape[0]):
                    bits = 0
                    for j, c in enumerate(codes[r]):
                        bits |= int(c) << (orc.BITS[fmt] * j)
                    arr[r] = np.frombuffer(bits.to_bytes(arr.shape[1], "little"), np.uint8)
            assert np.array_equal(orc.unpack_codes(pa, fmt, K), ca)
            got = orc.gemm(pa, sa, pb, sb, M, N, K, fmt)
            for m in range(M):
                for nn in range(N):
                    s = Fraction(0)
                    sabs = Fraction(0)
                    for k in range(K):
                        t = (exact(vals[ca[m, k]]) * Fraction(2) ** (int(sa[m, k // 32]) - 127) *
                             exact(vals[cb[nn, k]]) * Fraction(2) ** (int(sb[nn, k // 32]) - 127))
                        s += t
                        sabs += abs(t)
                    if narrow:
                        assert Fraction(got[m, nn]) == s, (fmt, K, m, nn)
                    else:
                        assert abs(Fraction(got[m, nn]) - s) <= K * Fraction(2) ** -52 * sabs


def test_gemm_matches_numpy_on_dequantized(orc):
    X, W, _ = I.linear(9, 64, 96, 256)
    for fmt, mode in ((1, 0), (2, 0), (3, 1)):
        qa = orc.quantize(X, 64, 256, fmt, mode)
        qb = orc.quantize(W, 96, 256, fmt, mode)
        A = deq_rows(orc, qa["row_codes"], qa["row_scales"], fmt, 256)
        B = deq_rows(orc, qb["row_codes"], qb["row_scales"], fmt, 256)
        bias = I.bf16_normal(np.random.default_rng(2), (96,), 0.01)
        got = orc.gemm(qa["row_codes"], qa["row_scales"], qb["row_codes"], qb["row_scales"], 64, 96, 256, fmt,
                       bias=bias)
        ref = A @ B.T + I.bf16_bits_to_f32(bias).astype(np.float64)
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
        sub = orc.gemm(qa["row_codes"], qa["row_scales"], qb["row_codes"], qb["row_scales"], 64, 96, 256, fmt,
                       bias=bias, rows=[5, 0, 63])
        assert np.array_equal(sub, got[[5, 0, 63]])


def test_mxfp6_hadamard_linear_snr_matches_page(orc):
    g = GOLDEN["mxfp6_linear_snr_vs_bf16_db"]
    M, N, K = 256, 256, 3072
    X, W, dY = I.linear(201, M, N, K)
    Xf, Wf, dYf = (I.bf16_bits_to_f32(a).astype(np.float64) for a in (X, W, dY))
    r = orc.linear_ref(X, W, dY, orc.E2M3, orc.FLOOR, True, M, N, K)

    def snr(ref, got):
        return 10 * np.log10(np.sum(ref ** 2) / np.sum((ref - got) ** 2))
    for name, ref in (("Y", Xf @ Wf.T), ("dX", dYf @ Wf), ("dW", dYf.T @ Xf)):
        s = snr(ref, r[name])
        assert abs(s - g["value"]) <= g["tolerance_db"], (name, s)


def test_rotation_cancels_in_gemm(orc):
    # With rotation on both operands the product approximates X.W^T as well
    # as without it (H/sqrt(32) orthogonal); rotating only one side does not.
    M, N, K = 64, 64, 512
    X, W, _ = I.linear(12, M, N, K)
    Xf, Wf = (I.bf16_bits_to_f32(a).astype(np.float64) for a in (X, W))
    ref = Xf @ Wf.T
    qa = orc.quantize(X, M, K, orc.E2M3, orc.FLOOR, True)
    qb = orc.quantize(W, N, K, orc.E2M3, orc.FLOOR, True)
    qb0 = orc.quantize(W, N, K, orc.E2M3, orc.FLOOR, False)
    both = orc.gemm(qa["row_codes"], qa["row_scales"], qb["row_codes"], qb["row_scales"], M, N, K, 2)
    one = orc.gemm(qa["row_codes"], qa["row_scales"], qb0["row_codes"], qb0["row_scales"], M, N, K, 2)
    e_both = np.linalg.norm(both - ref) / np.linalg.norm(ref)
    e_one = np.linalg.norm(one - ref) / np.linalg.norm(ref)
    assert e_both < 0.06 and e_one > 0.5


# ------------------------------------------------------------------ chains
def test_zero_output_projection_gives_zero_gradients(orc):
    # A zero-initialised fc2 weight makes da == 0, hence dh, dX, dW1 and the
    # bias gradient exactly zero; dW2 = dY^T a stays non-zero.
    M, D, F = 64, 64, 128
    X, W1, b1, W2, dY = I.mlp(13, M, D, F)
    W2 = np.zeros_like(W2)
    fwd = orc.mlp_fwd_ref(X, W1, b1, W2, M, D, F)
    assert np.all(fwd["Y64"] == 0)
    bwd = orc.mlp_bwd_ref(dY, fwd, M, D, F)
    assert np.all(bwd["da64"] == 0)
    assert np.all(bwd["dX64"] == 0) and np.all(bwd["dW1_64"] == 0) and np.all(bwd["db1"] == 0)
    assert np.any(bwd["dW2_64"] != 0)


def test_grouped_chain_empty_expert_and_shapes(orc):
    R, D, F, G = 512, 64, 32, 4
    counts, offsets, X, W1, W2, dY = I.grouped_mlp(17, R, D, F, G, zero_expert=1)
    assert counts[1] == 0 and counts.sum() == R and np.all(counts % 128 == 0)
    fwd = orc.grouped_fwd_ref(X, W1, W2, offsets, R, D, F)
    bwd = orc.grouped_bwd_ref(dY, fwd, offsets, R, D, F)
    assert np.all(bwd["dW1_64"][1] == 0) and np.all(bwd["dW2_64"][1] == 0)
    assert np.any(bwd["dW1_64"][0] != 0)
    # FC1 per expert equals a dense GEMM over that expert's rows only
    s, e = int(offsets[1]), int(offsets[2])
    q = fwd["X"]
    w = fwd["W1"][2]
    dense = orc.gemm(q["row_codes"][s:e], q["row_scales"][s:e], w["row_codes"], w["row_scales"], e - s, 2 * F,
                     D, orc.E4M3)
    assert np.array_equal(dense, fwd["H64"][s:e])


def test_gemm_accumulate_is_linear_in_k_and_exact_on_grid_values(orc):
    # Operands whose values lie on the E2M1 grid quantize exactly under any
    # FLOOR scale, and their dot products are small multiples of 1/4: every
    # partial sum is exact in binary32.  Splitting K into two halves and
    # accumulating the second GEMM into the first one's binary32 result must
    # then give the whole-K GEMM exactly; a zero C_old gives the plain GEMM.
    rng = np.random.default_rng(77)
    M, N, K = 64, 96, 128
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    vals = lambda shape: (rng.choice(grid, shape) * rng.choice([-1, 1], shape)).astype(np.float32)
    X = I.f32_to_bf16_bits(vals((M, K)))
    W = I.f32_to_bf16_bits(vals((N, K)))
    fmt = orc.E2M1
    qx, qw = orc.quantize(X, M, K, fmt, orc.FLOOR), orc.quantize(W, N, K, fmt, orc.FLOOR)
    whole = orc.gemm(qx["row_codes"], qx["row_scales"], qw["row_codes"], qw["row_scales"], M, N, K, fmt)
    exact = I.bf16_bits_to_f32(X).astype(np.float64) @ I.bf16_bits_to_f32(W).astype(np.float64).T
    assert np.array_equal(whole, exact)
    half = lambda q: orc._kslice(q["row_codes"], q["row_scales"], fmt, 0, K // 2)
    rest = lambda q: orc._kslice(q["row_codes"], q["row_scales"], fmt, K // 2, K)
    first = orc.gemm(*half(qx), *half(qw), M, N, K // 2, fmt)
    acc = orc.gemm_accumulate(first.astype(np.float32), *rest(qx), *rest(qw), M, N, K // 2, fmt)
    assert np.array_equal(acc, whole)
    zero = orc.gemm_accumulate(np.zeros((M, N), np.uint16), *rest(qx), *rest(qw), M, N, K // 2, fmt)
    assert np.array_equal(zero, orc.gemm(*rest(qx), *rest(qw), M, N, K // 2, fmt))
    # a bf16 C_old enters with its exact value
    old = I.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    got = orc.gemm_accumulate(old, *rest(qx), *rest(qw), M, N, K // 2, fmt)
    assert np.array_equal(got - I.bf16_bits_to_f32(old).astype(np.float64), zero)


# ------------------------------------------------------------------ stochastic rounding (MXFP4 gradients)
def test_philox_known_answer_vectors(orc):
    kat = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")))
    for v in kat["vectors"]:
        h = lambda xs: [int(t, 16) for t in xs]
        assert orc.philox4x32_10(h(v["ctr"]), h(v["key"])) == h(v["out"])


def test_sr_word_counter_layout(orc):
    # element i takes word i % 4 of the Philox block with counter
    # (i // 4 low, i // 4 high, axis, 0) and key (seed low, seed high)
    seed = 0x0123456789ABCDEF
    for axis in (0, 1):
        for i in (0, 1, 2, 3, 4, 7, 2**32 * 4 + 5, 2**40 + 3):
            q = i // 4
            want = orc.philox4x32_10([q & 0xFFFFFFFF, q >> 32, axis, 0], [seed & 0xFFFFFFFF, seed >> 32])[i % 4]
            assert orc.sr_word(seed, axis, i) == want


def test_e2m1_sr_rule_brute_force(orc):
    # every E2M1 grid interval, at fractions t = j/8, against the rule
    # written with exact rationals: up iff (r >> 8) < floor(t * 2^24)
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    rs = [0, 1, 255, 256, 0x7FFFFF00, 0x80000000, 0xFFFFFFFF] + [int(v) for v in
                                                             np.random.default_rng(5).integers(0, 2**32, 40)]
    for c in range(7):
        lo, hi = Fraction(grid[c]), Fraction(grid[c + 1])
        for j in range(8):
            t = Fraction(j, 8)
            v = lo + t * (hi - lo)
            for sign in (1, -1):
                for r in rs:
                    up = (r >> 8) < math.floor(t * 2**24)
                    want = (c + up) | (8 if sign < 0 else 0)
                    assert orc.encode_e2m1_sr(math.copysign(float(v), sign), r) == want, (float(v), r)
    # saturation at and above the largest magnitude; -0 keeps its sign
    for r in rs:
        assert orc.encode_e2m1_sr(6.0, r) == 7 and orc.encode_e2m1_sr(7.9, r) == 7
        assert orc.encode_e2m1_sr(-0.0, r) == 8 and orc.encode_e2m1_sr(0.0, r) == 0


def test_e2m1_sr_is_unbiased_and_keeps_grid_values(orc):
    rng = np.random.default_rng(6)
    # grid values never move, whatever the random word
    for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -3):
        for r in rng.integers(0, 2**32, 50):
            assert orc.decode(orc.E2M1, orc.encode_e2m1_sr(v, int(r))) == v
    # E[q] = v: mean of 20000 draws within 5 standard errors, for values
    # inside each spacing regime
    for v in (0.3, 1.1, 2.6, 4.5, -5.2):
        draws = np.array([orc.decode(orc.E2M1, orc.encode_e2m1_sr(v, int(r)))
                          for r in rng.integers(0, 2**32, 20000)])
        assert abs(draws.mean() - v) < 5 * draws.std() / math.sqrt(len(draws)) + 1e-9, v


def test_quantize_sr_matches_nearest_scales_and_neighbour_codes(orc):
    # SR packing keeps the nearest-rounding pack's scales; each code is one
    # of the two grid neighbours of x / 2^X (the nearest-rounding code or
    # its neighbour toward x); the same seed gives the same bytes, another
    # seed other bytes; columnwise SR is rowwise SR of the transpose with
    # axis 1 (checked element by element through the rule)
    rng = np.random.default_rng(8)
    R, C = 64, 96
    x = I.bf16_normal(rng, (R, C))
    sr = orc.quantize_sr(x, R, C, seed=42, row=True, col=True)
    rn = orc.quantize(x, R, C, orc.E2M1, orc.FLOOR, row=True, col=True)
    assert np.array_equal(sr["row_scales"], rn["row_scales"]) and np.array_equal(sr["col_scales"], rn["col_scales"])
    codes = orc.unpack_codes(sr["row_codes"], orc.E2M1, C)
    xf = I.bf16_bits_to_f32(x).astype(np.float64)
    moved = 0
    for r in range(R):
        for k in range(C):
            X = int(sr["row_scales"][r, k // 32]) - 127
            v = math.ldexp(xf[r, k], -X)
            want = orc.encode_e2m1_sr(v, orc.sr_word(42, 0, r * C + k))
            assert codes[r, k] == want
            moved += want != orc.encode(orc.E2M1, v)
            grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
            lo = max(g for g in grid if g <= min(abs(v), 6))
            hi = min(g for g in grid if g >= min(abs(v), 6))
            assert abs(orc.decode(orc.E2M1, want)) in (lo, hi)
    assert 0 < moved < R * C  # some elements round away from the nearest code, not all
    ccodes = orc.unpack_codes(sr["col_codes"], orc.E2M1, R)
    for c in range(0, C, 7):
        for r in range(R):
            X = int(sr["col_scales"][c, r // 32]) - 127
            assert ccodes[c, r] == orc.encode_e2m1_sr(math.ldexp(xf[r, c], -X), orc.sr_word(42, 1, c * R + r))
    again = orc.quantize_sr(x, R, C, seed=42, row=True)
    other = orc.quantize_sr(x, R, C, seed=43, row=True)
    assert np.array_equal(again["row_codes"], sr["row_codes"])
    assert not np.array_equal(other["row_codes"], sr["row_codes"])


# ------------------------------------------------------------------ prologues through orc_quantize
# The prologue tests above pin the scalar functions; these pin the indexing
# of the tensors the packer reads them from ([gate | up] halves of H, the
# (da, h) operand order), through the whole orc_quantize path, on inputs
# whose prologue output is an exact product with a single rounding.
def _bf16_of(x):
    return I.f32_to_bf16_bits(np.asarray(x, np.float32))


def _same_pack(orc, got_x, got_aux, want_v, R, C, fmt, mode, pro):
    """orc_quantize with prologue `pro` must pack exactly what the identity
    prologue packs from the expected prologue output want_v (bf16 bits)."""
    got = orc.quantize(got_x, R, C, fmt, mode, pro=pro, aux=got_aux, row=True, col=True, colsum=True)
    want = orc.quantize(want_v, R, C, fmt, mode, row=True, col=True, colsum=True)
    for k in want:
        assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), (pro, k)


@pytest.mark.parametrize("fmt,mode", [(3, 1), (1, 0)])
def test_swiglu_prologue_reads_gate_then_up(orc, fmt, mode):
    # a saturated gate (g >= 20: exp(-g) < 2^-25, so s == 1 exactly) makes
    # z = bf16(g * u): the product of two bf16 values is exact in binary32
    rng = np.random.default_rng(41)
    R, F = 64, 96
    g = _bf16_of(rng.uniform(20, 100, (R, F)))
    u = _bf16_of(rng.standard_normal((R, F)))
    H = np.ascontiguousarray(np.concatenate([g, u], 1))
    z = _bf16_of(I.bf16_bits_to_f32(g) * I.bf16_bits_to_f32(u))
    assert np.array_equal(orc.prologue(H, None, R, F, orc.PRO_SWIGLU), z)
    _same_pack(orc, H, None, z, R, F, fmt, mode, orc.PRO_SWIGLU)
    # the gate and up halves swapped would give silu(u) * g instead
    Hs = np.ascontiguousarray(np.concatenate([u, g], 1))
    assert not np.array_equal(orc.prologue(Hs, None, R, F, orc.PRO_SWIGLU), z)


@pytest.mark.parametrize("fmt,mode", [(3, 1), (1, 0)])
def test_dswiglu_prologue_reads_dz_and_gate_up(orc, fmt, mode):
    # saturated gate: s == 1, so d_gate = bf16((dz*u) * (1 * (1 + g*0))) =
    # bf16(dz*u) and d_up = bf16(dz * g), both single roundings of exact
    # binary32 products; dH = [d_gate | d_up]
    rng = np.random.default_rng(42)
    R, F = 64, 64
    g = _bf16_of(rng.uniform(20, 100, (R, F)))
    u = _bf16_of(rng.standard_normal((R, F)))
    dz = _bf16_of(rng.standard_normal((R, F)))
    H = np.ascontiguousarray(np.concatenate([g, u], 1))
    gf, uf, dzf = (I.bf16_bits_to_f32(a) for a in (g, u, dz))
    dH = np.ascontiguousarray(np.concatenate([_bf16_of(dzf * uf), _bf16_of(dzf * gf)], 1))
    assert np.array_equal(orc.prologue(dz, H, R, 2 * F, orc.PRO_DSWIGLU), dH)
    _same_pack(orc, dz, H, dH, R, 2 * F, fmt, mode, orc.PRO_DSWIGLU)


@pytest.mark.parametrize("fmt,mode,had", [(2, 0, True), (3, 1, False)])
def test_gelu_and_dgelu_prologues_on_exact_points(orc, fmt, mode, had):
    # h = 0: u = 0, exp(0) = 1, q = 1, so GELU(0) = 0 and dGELU = 0.5 exactly;
    # |h| >= 12: exp(2|u|) overflows, q = 0, so GELU(h) = h and dGELU = 1 for
    # h > 0, GELU(h) = -0 and dGELU = 0 for h < 0.  So a = {0, h, -0} and dh = {da/2, da, 0} exactly; with the
    # (da, h) operands swapped dh would be dgelu(h) * da evaluated at da.
    rng = np.random.default_rng(43)
    R, C = 64, 128
    pick = rng.integers(0, 3, (R, C))
    hv = np.where(pick == 0, 0.0, np.where(pick == 1, rng.uniform(12, 60, (R, C)), -rng.uniform(12, 60, (R, C))))
    h = _bf16_of(hv)
    da = _bf16_of(rng.standard_normal((R, C)))
    hf, daf = I.bf16_bits_to_f32(h), I.bf16_bits_to_f32(da)
    a = np.where(pick == 0, np.uint16(0), np.where(pick == 1, h, np.uint16(0x8000))).astype(np.uint16)
    dh = _bf16_of(np.where(pick == 0, daf * np.float32(0.5), np.where(pick == 1, daf, np.float32(0) * daf)))
    assert np.array_equal(orc.prologue(h, None, R, C, orc.PRO_GELU), a)
    assert np.array_equal(orc.prologue(da, h, R, C, orc.PRO_DGELU), dh)
    _same_pack(orc, h, None, a, R, C, fmt, mode, orc.PRO_GELU)
    _same_pack(orc, da, h, dh, R, C, fmt, mode, orc.PRO_DGELU)
    assert not np.array_equal(orc.prologue(h, da, R, C, orc.PRO_DGELU), dh)
    assert np.all(np.abs(hf[pick > 0]) >= 12)


# ------------------------------------------------------------------ chains against unquantized chains
def snr_db(ref, got):
    return 10 * np.log10(np.sum(ref ** 2) / np.sum((ref - got) ** 2))


def test_grouped_chain_snr_against_unquantized_chain(orc):
    # The pages check the grouped SwiGLU MLP against a chain without any
    # quantization, computed from the original bf16 tensors, and report the
    # MXFP8 outputs on a band: 28.5 dB for z, the FC1 GEMM output, and
    # 23.7 dB for y, the FC2 output after a second quantized stage; their
    # gate is the band minus 6 dB.  The oracle lands on the band.  Backward
    # reading: dz (FC2 dgrad, one quantized GEMM like z) on z's band; dX,
    # dW1 and dW2 (through the quantized dH, like y) on y's band.
    g = GOLDEN["mxfp8_grouped_chain_snr_vs_bf16_db"]
    R, D, F, G = 1024, 512, 256, 4
    counts, offsets, X, W1, W2, dY = I.grouped_mlp(17, R, D, F, G, zero_expert=1)
    fwd = orc.grouped_fwd_ref(X, W1, W2, offsets, R, D, F)
    bwd = orc.grouped_bwd_ref(dY, fwd, offsets, R, D, F)
    f64 = lambda a: I.bf16_bits_to_f32(a).astype(np.float64)
    Xf, W1f, W2f, dYf = f64(X), f64(W1), f64(W2), f64(dY)
    ref = {k: np.zeros(s) for k, s in (("H", (R, 2 * F)), ("Y", (R, D)), ("dz", (R, F)), ("dX", (R, D)),
                                       ("dW1", (G, 2 * F, D)), ("dW2", (G, D, F)))}
    for e, (s, t) in enumerate(orc.grouped_ranges(offsets)):
        if t == s:
            continue
        H = Xf[s:t] @ W1f[e].T
        gate, up = H[:, :F], H[:, F:]
        sg = 1 / (1 + np.exp(-gate))
        z = gate * sg * up
        dz = dYf[s:t] @ W2f[e]
        dH = np.concatenate([dz * up * sg * (1 + gate * (1 - sg)), dz * gate * sg], 1)
        ref["H"][s:t], ref["Y"][s:t], ref["dz"][s:t] = H, z @ W2f[e].T, dz
        ref["dX"][s:t] = dH @ W1f[e]
        ref["dW1"][e], ref["dW2"][e] = dH.T @ Xf[s:t], dYf[s:t].T @ z
    got = {"H": fwd["H64"], "Y": fwd["Y64"], "dz": bwd["dz64"], "dX": bwd["dX64"], "dW1": bwd["dW1_64"],
           "dW2": bwd["dW2_64"]}
    band = {"H": g["z"], "dz": g["z"], "Y": g["y"], "dX": g["y"], "dW1": g["y"], "dW2": g["y"]}
    for k in got:
        s = snr_db(ref[k], got[k])
        assert s >= band[k] - g["gate_below_band_db"], (k, s)
        assert abs(s - band[k]) <= g["tolerance_db"], (k, s)


def test_mlp_chain_snr_against_unquantized_mlp(orc):
    # The MXFP6 (+Hadamard) linear lands at about 28 dB SNR against BF16 in
    # the forward and both gradients (the MXFP6 page).  In the fused MLP, h
    # (fc1 forward) and da (fc2 data gradient) are such single linears and
    # must land there; Y, dX, dW1, dW2 and db1 pass a second quantized stage
    # and are held to the grouped page's gate, the band minus 6 dB.  The
    # reference is the unquantized tanh-GELU MLP from the same bf16 inputs.
    g = GOLDEN["mxfp6_linear_snr_vs_bf16_db"]
    gate = g["value"] - GOLDEN["mxfp8_grouped_chain_snr_vs_bf16_db"]["gate_below_band_db"]
    M, D, F = 512, 256, 1024
    X, W1, b1, W2, dY = I.mlp(301, M, D, F)
    fwd = orc.mlp_fwd_ref(X, W1, b1, W2, M, D, F)
    bwd = orc.mlp_bwd_ref(dY, fwd, M, D, F)
    f64 = lambda a: I.bf16_bits_to_f32(a).astype(np.float64)
    Xf, W1f, b1f, W2f, dYf = f64(X), f64(W1), f64(b1), f64(W2), f64(dY)
    h = Xf @ W1f.T + b1f
    k0, k1 = math.sqrt(2 / math.pi), 0.044715
    t = np.tanh(k0 * (h + k1 * h ** 3))
    a = 0.5 * h * (1 + t)
    da = dYf @ W2f
    dh = da * (0.5 * (1 + t) + 0.5 * h * (1 - t * t) * k0 * (1 + 3 * k1 * h * h))
    single = {"h": (h, fwd["h64"]), "da": (da, bwd["da64"])}
    for k, (r, o) in single.items():
        s = snr_db(r, o)
        assert abs(s - g["value"]) <= g["tolerance_db"], (k, s)
    two = {"Y": (a @ W2f.T, fwd["Y64"]), "dX": (dh @ W1f, bwd["dX64"]), "dW1": (dh.T @ Xf, bwd["dW1_64"]),
           "dW2": (dYf.T @ a, bwd["dW2_64"]), "db1": (dh.sum(0), bwd["db1"].astype(np.float64))}
    for k, (r, o) in two.items():
        s = snr_db(r, o)
        assert gate <= s < g["value"] + g["tolerance_db"], (k, s)
