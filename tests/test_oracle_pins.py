"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage (page title + section) it follows. None of them
re-types the oracle's formula: they use closed forms, hand-derived instances
(tests/golden), library routines (torch's bf16 conversion, numpy's IEEE
float32 sqrt and divide, float64 / exact-rational references) and brute force
on tiny inputs.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
D = 8192


def f32_of_bf16(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_of(vals):
    """bf16 bit patterns of exactly representable values (torch's conversion)."""
    import torch

    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ bf16()

def _exhaustive(check):
    """Run check(start, bits) over all 2^32 patterns in chunks on a thread
    pool (numpy, torch and the ctypes calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    step = 1 << 24

    def one(start):
        bits = np.arange(step, dtype=np.uint32) + np.uint32(start)
        return check(bits)

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        for msg in ex.map(one, range(0, 1 << 32, step)):
            if msg:
                pytest.fail(msg)


def test_bf16_exhaustive_matches_torch(oracle):
    """f32 -> bf16 round-to-nearest-even over all 2^32 patterns: every
    non-NaN input against torch's CPU conversion (a library routine), every
    NaN to 0x7FC0 (torch keeps other NaN patterns, so NaN is checked apart)."""
    import torch

    def check(bits):
        f = bits.view(np.float32)
        ours = oracle.bf16(f)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        ok = np.where(nan, ours == 0x7FC0, ours == ref)
        if not ok.all():
            bad = np.nonzero(~ok)[0][:5]
            return (f"bf16 mismatch at {[hex(int(bits[i])) for i in bad]}: "
                    f"{[hex(int(ours[i])) for i in bad]} vs {[hex(int(ref[i])) for i in bad]}")
        return None

    _exhaustive(check)


def test_bf16_nearest_even_by_midpoints(oracle):
    """An independent formulation on random and special inputs: the result is
    the nearer of the two bf16 neighbours (compared in float64), ties to the
    even one; overflow past the largest finite midpoint gives Inf."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x3F808000, 0x3F818000,
                         0x3F80C000, 0x7F7FFFFF, 0x7F7F7FFF, 0x7F7F8000, 0xFF7F8000, 0x7F800000,
                         0xFF800000, 0x00008000, 0x00018000, 0x7F7F7FFF], dtype=np.uint32)
    bits = np.concatenate([bits, specials])
    f = bits.view(np.float32)
    finite = np.isfinite(f)
    f, bits = f[finite], bits[finite]
    got = oracle.bf16(f)
    lo = (bits >> 16).astype(np.uint16)  # truncation toward zero
    hi = (lo + 1).astype(np.uint16)      # next magnitude up
    vlo = f32_of_bf16(lo).astype(np.float64)
    vhi = f32_of_bf16(hi).astype(np.float64)
    # next magnitude past the largest finite bf16 is Inf, whose "value" for
    # the midpoint rule is 2^128
    vhi = np.where(np.isinf(vhi), np.sign(vlo) * 2.0 ** 128 + (vlo == 0), vhi)
    x = f.astype(np.float64)
    dlo, dhi = np.abs(x - vlo), np.abs(vhi - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo & 1) == 1))
    expect = np.where(pick_hi, hi, lo).astype(np.uint16)
    assert np.array_equal(got, expect)


def test_bf16_nan_and_signed_values(oracle):
    for b in (0x7F800001, 0x7FC00000, 0xFFC00000, 0xFFFFFFFF, 0x7FBFFFFF):
        assert int(oracle.bf16(np.array([b], dtype=np.uint32).view(np.float32))[0]) == 0x7FC0
    assert int(oracle.bf16(np.float32(-0.0))) == 0x8000
    assert int(oracle.bf16(np.float32(np.inf))) == 0x7F80
    assert int(oracle.bf16(np.float32(-np.inf))) == 0xFF80
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    assert int(oracle.bf16(np.float32(1.0 + 2.0 ** -8))) == 0x3F80
    # 1 + 3 * 2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    assert int(oracle.bf16(np.float32(1.0 + 3 * 2.0 ** -8))) == 0x3F82


# -------------------------------------------------------------------- rs()

def test_rs_exhaustive_matches_ieee_float32(oracle):
    """rs(v) = 1 / sqrt(v), both IEEE correctly rounded, over all 2^32
    patterns, against numpy's float32 sqrt and divide."""
    one = np.float32(1.0)

    def check(bits):
        v = bits.view(np.float32)
        ours = oracle.rs(v)
        with np.errstate(all="ignore"):
            ref = one / np.sqrt(v)
        same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
        if not same.all():
            bad = np.nonzero(~same)[0][:5]
            return f"rs mismatch at {[hex(int(bits[i])) for i in bad]}"
        return None

    _exhaustive(check)


def _round_f32_exact(q):
    """Round a positive Fraction to the nearest float32 (ties to even), normal range."""
    e = math.floor(math.log2(q.numerator) - math.log2(q.denominator))
    # adjust e so that 2^e <= q < 2^(e+1)
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    scale = Fraction(2) ** (23 - e)
    m = q * scale
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return float(Fraction(fl) / scale)


def test_rs_against_exact_rationals(oracle):
    """Correctly rounded sqrt (decided by exact squared midpoints) then a
    correctly rounded 1/s, on random normal inputs, in exact rationals."""
    rng = np.random.default_rng(11)
    vals = (rng.random(300) * 2.0 ** rng.integers(-60, 60, 300)).astype(np.float32)
    vals = vals[vals > 0]
    got = oracle.rs(vals)
    up, down = np.float32(np.inf), np.float32(0)
    for v, g in zip(vals, got):
        fv = Fraction(float(v))
        s0 = np.float32(math.sqrt(float(v)))
        s = None
        for c in (np.nextafter(s0, down), s0, np.nextafter(s0, up)):
            lo = (Fraction(float(np.nextafter(c, down))) + Fraction(float(c))) / 2
            hi = (Fraction(float(c)) + Fraction(float(np.nextafter(c, up)))) / 2
            if lo * lo < fv < hi * hi:
                s = c
        assert s is not None, v
        expect = _round_f32_exact(Fraction(1) / Fraction(float(s)))
        assert float(g) == expect, (v, g, expect)


def test_rs_closed_forms(oracle):
    ks = np.arange(-60, 61, dtype=np.int64)
    v = np.ldexp(np.float32(1.0), 2 * ks).astype(np.float32)
    assert np.array_equal(oracle.rs(v), np.ldexp(np.float32(1.0), -ks).astype(np.float32))
    with np.errstate(all="ignore"):
        r = oracle.rs(np.array([0.0, -0.0, np.inf, -1.0, np.nan], dtype=np.float32))
    assert r[0] == np.inf and r[1] == -np.inf and r[2] == 0.0 and not np.signbit(r[2])
    assert np.isnan(r[3]) and np.isnan(r[4])


# ------------------------------------------------------------- row ΣSq order

def _row_from(nonzero):
    u = np.zeros(D, dtype=np.float32)
    for c, val in nonzero.items():
        u[int(c)] = val
    return u


def test_row_sumsq_order_golden(oracle):
    """Hand-derived sums that fix the row reduction order (tests/golden)."""
    with open(os.path.join(GOLDEN, "row_sumsq_order.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        got = oracle.sumsq_row(_row_from(case["nonzero"]))
        assert float(got) == case["expected"], case["name"]


def test_row_sumsq_within_recursive_summation_bound(oracle):
    """|S - S*| <= gamma_25 * S* (S* the exact sum of squares; the longest
    rounding path is 16 FMAs + 1 + 6 + 2 = 25 operations)."""
    rng = np.random.default_rng(3)
    g25 = 25 * 2.0 ** -24 / (1 - 25 * 2.0 ** -24)
    for scale in (1e-3, 1.0, 37.0, 1e5):
        u = f32_of_bf16(bf16_bits_of(rng.standard_normal(D) * scale))
        exact = math.fsum(float(a) * float(a) for a in u)
        got = float(oracle.sumsq_row(u))
        assert abs(got - exact) <= g25 * exact


def test_row_sumsq_permutation_sensitivity_is_bounded(oracle):
    """Any reordering of the columns stays within the summation bound
    (sanity for the oracle's order being a plain sum of all 8192 squares:
    a dropped or doubled column would leave it)."""
    rng = np.random.default_rng(5)
    u = f32_of_bf16(bf16_bits_of(rng.standard_normal(D)))
    exact = math.fsum(float(a) * float(a) for a in u)
    g25 = 25 * 2.0 ** -24 / (1 - 25 * 2.0 ** -24)
    for _ in range(4):
        p = rng.permutation(D)
        assert abs(float(oracle.sumsq_row(u[p])) - exact) <= g25 * exact
    # drop one column: leaves the bound for a large column
    u2 = u.copy()
    j = int(np.argmax(np.abs(u2)))
    u2[j] = 0
    assert abs(float(oracle.sumsq_row(u2)) - exact) > g25 * exact


# ---------------------------------------------------------------- the norms

def _norms(oracle, x, hw, pw, L, he=1e-6, pe=1e-6, hc=0.0, pc=0.0):
    return oracle.context_norms(x, hw, pw, L, he, pe, hc, pc)


def test_norms_constant_power_of_two_rows_give_unit_outputs(oracle):
    """Page '...draft_boundary', boundary_fragments: r = rsqrt(S/D + eps),
    y = x r. A row of c = +-2^k with eps = 0 has S = 8192 c^2 exactly, so
    every weightless output is exactly +-1.0 (0x3F80 / 0xBF80) and every
    weighted layer output exactly +-gamma_l."""
    ks = [-20, -3, 0, 1, 7, 30]
    rows = []
    for k in ks:
        rows.append(np.full(D, 2.0 ** k))
        rows.append(np.full(D, -(2.0 ** k)))
    mixed = np.where(np.arange(D) % 3 == 0, -1.0, 1.0) * 2.0 ** 5
    rows.append(mixed)
    x = bf16_bits_of(np.stack(rows))
    out = _norms(oracle, x, None, None, 3, 0.0, 0.0)
    sign = np.signbit(f32_of_bf16(x))
    expect = np.where(sign, np.uint16(0xBF80), np.uint16(0x3F80))
    for l in range(3):
        assert np.array_equal(out[l], expect)
    rng = np.random.default_rng(1)
    pw = bf16_bits_of(1.0 + 0.1 * rng.standard_normal((3, D)))
    out = _norms(oracle, x, None, pw, 3, 0.0, 0.0)
    for l in range(3):
        expect_l = np.where(sign, pw[l] | np.uint16(0x8000), pw[l])
        assert np.array_equal(out[l], expect_l), l


def test_norms_hidden_weight_on_constant_rows(oracle):
    """x = +-2^9 everywhere, gamma_h = 4, eps = 0: h = bf16((x r) gamma) =
    +-4 exactly, and the weightless layer norm of that constant row is +-1."""
    g = bf16_bits_of(np.full(D, 4.0))
    x = bf16_bits_of(np.stack([np.full(D, 2.0 ** 9), np.full(D, -(2.0 ** -9))]))
    out = _norms(oracle, x, g, None, 1, 0.0, 0.0)
    assert np.array_equal(out[0, 0], np.full(D, 0x3F80, dtype=np.uint16))
    assert np.array_equal(out[0, 1], np.full(D, 0xBF80, dtype=np.uint16))


def test_norms_power_of_two_scaling_is_bit_exact(oracle):
    """With eps = 0 and no under/overflow, scaling x by 2^k leaves every
    output bit unchanged (rounding, sqrt and divide commute with 2^k)."""
    rng = np.random.default_rng(2)
    x = bf16_bits_of(rng.standard_normal((3, D)))
    hw = bf16_bits_of(1.0 + 0.1 * rng.standard_normal(D))
    pw = bf16_bits_of(1.0 + 0.1 * rng.standard_normal((2, D)))
    base = _norms(oracle, x, hw, pw, 2, 0.0, 0.0)
    for k in (-12, -1, 3, 17):
        xs = bf16_bits_of(f32_of_bf16(x) * 2.0 ** k)
        assert np.array_equal(_norms(oracle, xs, hw, pw, 2, 0.0, 0.0), base), k


def test_norms_multiply_order_x_r_then_gamma(oracle):
    """Page '...draft_boundary', boundary_fragments: y = x * r first, then
    y * gamma. With x = 2^50 (r = 2^-50) and gamma = 2^-100 the stated order
    gives exactly 2^-100, while x * (r * gamma) would underflow r * gamma =
    2^-150 to 0. Checked at the hidden norm (x = 2^50, gamma_h = 2^-100,
    pre eps = 1 so r_p = 1) and at the layer norm (x = 1, gamma_h = 2^50,
    gamma_l = 2^-100)."""
    x = bf16_bits_of(np.full((1, D), 2.0 ** 50))
    gh = bf16_bits_of(np.full(D, 2.0 ** -100))
    out = _norms(oracle, x, gh, None, 1, 0.0, 1.0)
    # h = 2^-100, S_p underflows to 0, r_p = rs(1) = 1: out = 2^-100 (0x0D80)
    assert np.all(out[0, 0] == 0x0D80)
    x1 = bf16_bits_of(np.ones((1, D)))
    gh = bf16_bits_of(np.full(D, 2.0 ** 50))
    gp = bf16_bits_of(np.full((1, D), 2.0 ** -100))
    out = _norms(oracle, x1, gh, gp, 1, 0.0, 0.0)
    assert np.all(out[0, 0] == 0x0D80)


def test_norms_weightless_rms(oracle):
    """Weightless norms: the output RMS is within 2^-8 of sqrt(ms/(ms+eps))."""
    rng = np.random.default_rng(4)
    for scale, eps in ((1.0, 1e-6), (1e-3, 1e-6), (1.0, 0.5)):
        x = bf16_bits_of(rng.standard_normal((4, D)) * scale)
        out = _norms(oracle, x, None, None, 1, eps, eps)
        xf = f32_of_bf16(x).astype(np.float64)
        of = f32_of_bf16(out[0]).astype(np.float64)
        for t in range(4):
            ms = np.mean(xf[t] ** 2)
            h_rms = math.sqrt(ms / (ms + eps))
            # second norm of h (whose mean square is h_rms^2)
            want = math.sqrt(h_rms ** 2 / (h_rms ** 2 + eps))
            got = math.sqrt(np.mean(of[t] ** 2))
            assert abs(got - want) <= 2.0 ** -8 * want


def test_norms_float64_model_within_one_ulp(oracle):
    """The exact result within the rounding bound: a float64 evaluation of
    the hidden norm (torch rounds h to bf16), then of each layer norm from
    the oracle's own h, agrees with the oracle to 1 bf16 ulp per element.
    Catches a wrong 1/D, eps, weight index, layer layout or missing weight."""
    import torch

    rng = np.random.default_rng(6)
    T, L = 3, 3
    x = bf16_bits_of(rng.standard_normal((T, D)) * 1.7)
    hw = bf16_bits_of(1.0 + 0.1 * rng.standard_normal(D))
    pw = bf16_bits_of(1.0 + 0.1 * rng.standard_normal((L, D)))
    he, pe = 1e-6, 3e-2
    out = _norms(oracle, x, hw, pw, L, he, pe)
    xf = f32_of_bf16(x).astype(np.float64)
    g_h = f32_of_bf16(hw).astype(np.float64)
    g_p = f32_of_bf16(pw).astype(np.float64)

    def ulp_ok(got_bits, want):
        got = f32_of_bf16(got_bits).astype(np.float64)
        tol = np.maximum(np.abs(want), 1e-30) * 2.0 ** -7
        return np.all(np.abs(got - want) <= tol)

    for t in range(T):
        r = 1.0 / math.sqrt(math.fsum(xf[t] ** 2) / D + float(np.float32(he)))
        h_model = xf[t] * r * g_h
        h_bits = torch.tensor(h_model, dtype=torch.float64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        hf = f32_of_bf16(h_bits).astype(np.float64)
        rp = 1.0 / math.sqrt(math.fsum(hf ** 2) / D + float(np.float32(pe)))
        for l in range(L):
            assert ulp_ok(out[l, t], hf * rp * g_p[l]), (t, l)


def test_norms_zero_and_overflow_rows(oracle):
    """Zero rows give signed zeros (r = 1/sqrt(eps) is finite); a row whose
    squares overflow has S = +Inf, r = +0 and gives signed zeros too; -0.0
    weights turn into +0.0 through the gain center add (w + 0.0)."""
    big = 0x7F7F  # the largest finite bf16
    x = np.zeros((3, D), dtype=np.uint16)
    x[1, :] = 0x8000
    x[2, :] = bf16_bits_of(np.where(np.arange(D) % 2 == 0, 1.0, -1.0))
    x[2, 5] = big
    pw = bf16_bits_of(np.full((1, D), 1.5))
    out = _norms(oracle, x, None, pw, 1)
    assert np.all(out[0, 0] == 0x0000)
    assert np.all(out[0, 1] == 0x8000)
    sign = np.signbit(f32_of_bf16(x[2]))
    assert np.array_equal(out[0, 2], np.where(sign, np.uint16(0x8000), np.uint16(0)))
    # -0.0 weight becomes +0.0 through the center: x>0 * +0 = +0
    pw0 = np.full((1, D), 0x8000, dtype=np.uint16)
    x1 = bf16_bits_of(np.ones((1, D)))
    assert np.all(_norms(oracle, x1, None, pw0, 1)[0, 0] == 0x0000)
    # ... unless a center of -0.0 keeps it: (-0) + (-0) = -0
    assert np.all(_norms(oracle, x1, None, pw0, 1, pc=-0.0)[0, 0] == 0x8000)


def test_norms_nan_rows_quiet(oracle):
    """A NaN anywhere in a row makes S NaN and every output of that row the
    bf16 quiet NaN 0x7FC0; other rows are unaffected."""
    rng = np.random.default_rng(8)
    x = bf16_bits_of(rng.standard_normal((2, D)))
    ref = _norms(oracle, x, None, None, 1)
    x[0, 77] = 0xFFC1
    out = _norms(oracle, x, None, None, 1)
    assert np.all(out[0, 0] == 0x7FC0)
    assert np.array_equal(out[0, 1], ref[0, 1])


def test_norms_layer_layout(oracle):
    """out[l, t] depends on layer l's weight only and on row t only (the
    [L, T, D] stack of the context page's ContextNorms)."""
    rng = np.random.default_rng(9)
    T, L = 4, 3
    x = bf16_bits_of(rng.standard_normal((T, D)))
    hw = bf16_bits_of(1.0 + 0.1 * rng.standard_normal(D))
    pw = bf16_bits_of(1.0 + 0.1 * rng.standard_normal((L, D)))
    out = _norms(oracle, x, hw, pw, L)
    for l in range(L):
        single = _norms(oracle, x, hw, pw[l:l + 1], 1)
        assert np.array_equal(single[0], out[l])
    for t in range(T):
        assert np.array_equal(_norms(oracle, x[t:t + 1], hw, pw, L)[:, 0], out[:, t])


def test_hidden_norm_pieces_rebuild_the_norms(oracle):
    """The pre-pass quantities (h, r) rebuild every layer output as
    bf16((h * r) * gamma_l): checked against the full norms on rows with
    weights, without weights, and with a zero row."""
    import torch

    rng = np.random.default_rng(21)
    T, L = 5, 3
    x = bf16_bits_of(rng.standard_normal((T, D)) * 1.3)
    x[2] = 0
    hw = bf16_bits_of(1.0 + 0.1 * rng.standard_normal(D))
    pw = bf16_bits_of(1.0 + 0.1 * rng.standard_normal((L, D)))
    for w_h, w_p in ((hw, pw), (None, pw), (hw, None)):
        full = _norms(oracle, x, w_h, w_p, L, 1e-6, 3e-3)
        h, r = oracle.hidden_norm(x, w_h, 1e-6, 0.0, 3e-3)
        y = f32_of_bf16(h) * r[:, None]  # float32 products, one rounding each
        for l in range(L):
            z = y * (f32_of_bf16(w_p[l]) if w_p is not None else np.float32(1.0))
            want = torch.from_numpy(np.ascontiguousarray(z.astype(np.float32))).to(torch.bfloat16)
            assert np.array_equal(full[l], want.view(torch.int16).numpy().view(np.uint16)), l


def test_projection_nd_layout(oracle):
    """The [L, N, D] weight storage holds the transpose of the bmm's operand:
    the same FP32 sums in the same d order, so equal bits to the [L, D, N]
    routine on the transposed weight; one-hot rows pick B's bf16 rows exactly
    and zero rows give +0."""
    rng = np.random.default_rng(51)
    L, T, Dd, N = 2, 5, 256, 24
    A = bf16_bits_of(rng.standard_normal((L, T, Dd)))
    Bnd = bf16_bits_of(rng.standard_normal((L, N, Dd)) * 0.05)
    got = oracle.kv_project_nd(A, Bnd)
    want = oracle.kv_project(A, np.ascontiguousarray(Bnd.transpose(0, 2, 1)))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    oh = np.zeros((L, T, Dd), dtype=np.uint16)
    cols = [3, 200, 17, 255]
    for t, c in enumerate(cols):
        oh[:, t, c] = 0x3F80
    C = oracle.kv_project_nd(oh, Bnd)
    for l in range(L):
        for t, c in enumerate(cols):
            assert np.array_equal(C[l, t], f32_of_bf16(Bnd[l, :, c]))
        assert np.all(C[l, len(cols):] == 0) and not np.signbit(C[l, len(cols):]).any()


# ------------------------------------------- norm variants (FP32, input scale)

def _bf16_round_indep(f):
    """bf16 bits of float32 values (no NaN) by the midpoint rule in float64,
    independently of the oracle's bit trick."""
    f = np.asarray(f, dtype=np.float32)
    bits = f.view(np.uint32)
    lo = (bits >> 16).astype(np.uint16)
    hi = (lo + 1).astype(np.uint16)
    vlo = f32_of_bf16(lo).astype(np.float64)
    vhi = f32_of_bf16(hi).astype(np.float64)
    x = f.astype(np.float64)
    dlo, dhi = np.abs(x - vlo), np.abs(vhi - x)
    return np.where((dhi < dlo) | ((dhi == dlo) & ((lo & 1) == 1)), hi, lo).astype(np.uint16)


def test_norms_ex_default_form_equals_the_norms(oracle):
    """The general entry with bf16 weights applied to the outputs is the plain
    norms; FP32 weights holding exactly the bf16 values give the same bits."""
    rng = np.random.default_rng(31)
    T, L = 4, 3
    x = bf16_bits_of(rng.standard_normal((T, D)))
    hw = bf16_bits_of(1.0 + 0.2 * rng.standard_normal(D))
    pw = bf16_bits_of(1.0 + 0.2 * rng.standard_normal((L, D)))
    want = oracle.context_norms(x, hw, pw, L, 1e-6, 1e-6, 0.25, -0.5)
    got = oracle.context_norms_ex(x, hw, pw, L, 1e-6, 1e-6, 0.25, -0.5)
    assert np.array_equal(got, want)
    got32 = oracle.context_norms_ex(x, f32_of_bf16(hw), f32_of_bf16(pw), L, 1e-6, 1e-6, 0.25, -0.5)
    assert np.array_equal(got32, want)


def test_norms_input_scaled_constant_rows_are_unit(oracle):
    """Page '...draft_boundary', boundary_fragments, input-scaled form:
    v = gamma x, S sums v^2, y = v r, no weight afterwards. A constant row
    x = +-2^k with a constant gamma c (8 significant bits) has S = 8192 (c x)^2
    exactly, so y = v / |v| rounds to exactly +-1: the hidden output is +-1
    whatever c is (the output-scaled form would give +-c), and each input-
    scaled layer norm of it, with its own constant c_l, again gives +-1 (each
    layer has its own sum). Negative c flips the sign."""
    ks = [-12, 0, 3, 20]
    rows = []
    for k in ks:
        rows.append(np.full(D, 2.0 ** k))
        rows.append(np.full(D, -(2.0 ** k)))
    x = bf16_bits_of(np.stack(rows))
    sign = np.signbit(f32_of_bf16(x))
    L = 3
    for c, cl in ((1.5, [0.75, 3.0, 5.0]), (-2.5, [1.25, -0.375, 40.0])):
        for kind in ("bf16", "f32"):
            hw = np.full(D, c, dtype=np.float32)
            pw = np.stack([np.full(D, v, dtype=np.float32) for v in cl])
            if kind == "bf16":
                hw, pw = bf16_bits_of(hw), bf16_bits_of(pw)
            out = oracle.context_norms_ex(x, hw, pw, L, 0.0, 0.0, 0.0, 0.0, True, True)
            h_neg = sign ^ (c < 0)
            for l in range(L):
                neg = h_neg ^ (cl[l] < 0)
                assert np.array_equal(out[l], np.where(neg, np.uint16(0xBF80), np.uint16(0x3F80))), (c, kind, l)
            # hidden input-scaled, layers output-scaled: +-c_l exactly
            out = oracle.context_norms_ex(x, hw, pw, L, 0.0, 0.0, 0.0, 0.0, True, False)
            for l in range(L):
                mag = bf16_bits_of(np.full(D, abs(cl[l]), dtype=np.float32))
                neg = h_neg ^ (cl[l] < 0)
                assert np.array_equal(out[l], np.where(neg, mag | np.uint16(0x8000), mag)), (c, kind, l)


def test_norms_ex_large_eps_closed_form(oracle):
    """With eps = 2^20 and rows of |x| <= 0.25, fma(S, 2^-13, eps) = 2^20
    exactly (S 2^-13 is below half an ulp of 2^20), so r = 2^-10 exactly and
    each norm reduces to one rounded product: output-scaled
    bf16((x 2^-10) gamma), input-scaled bf16((gamma x) 2^-10), gamma =
    w + center. The expected bits come from numpy's IEEE float32 products and
    a midpoint-rule bf16 rounding. Random FP32 weights carry bits below bf16
    precision, so reading them through bf16 would change many outputs."""
    rng = np.random.default_rng(41)
    T, L = 3, 2
    x = bf16_bits_of(np.clip(rng.standard_normal((T, D)) * 0.08, -0.25, 0.25))
    eps = np.float32(2.0 ** 20)
    r = np.float32(2.0 ** -10)
    hc, pc = np.float32(0.125), np.float32(-0.0625)
    for hk in ("bf16", "f32", None):
        for pk in ("bf16", "f32", None):
            hw = (1.0 + 0.3 * rng.standard_normal(D)).astype(np.float32)
            pw = (1.0 + 0.3 * rng.standard_normal((L, D))).astype(np.float32)
            if hk == "bf16":
                hw = bf16_bits_of(hw)
            if pk == "bf16":
                pw = bf16_bits_of(pw)
            hwv = None if hk is None else (f32_of_bf16(hw) if hk == "bf16" else hw)
            pwv = None if pk is None else (f32_of_bf16(pw) if pk == "bf16" else pw)
            for his in (False, True):
                for pis in (False, True):
                    got = oracle.context_norms_ex(x, None if hk is None else hw, None if pk is None else pw, L,
                                                  float(eps), float(eps), float(hc), float(pc), his, pis)
                    xf = f32_of_bf16(x)
                    if hwv is None:
                        hy = xf * r
                    elif his:
                        hy = ((hwv + hc) * xf) * r
                    else:
                        hy = (xf * r) * (hwv + hc)
                    hf = f32_of_bf16(_bf16_round_indep(hy))
                    for l in range(L):
                        if pwv is None:
                            y = hf * r
                        elif pis:
                            y = ((pwv[l] + pc) * hf) * r
                        else:
                            y = (hf * r) * (pwv[l] + pc)
                        assert np.array_equal(got[l], _bf16_round_indep(y)), (hk, pk, his, pis, l)
    if True:  # the FP32 weights do matter: their bf16 copies give other bits
        hw = (1.0 + 0.3 * rng.standard_normal(D)).astype(np.float32)
        a = oracle.context_norms_ex(x, hw, None, 1, float(eps), float(eps))
        b = oracle.context_norms_ex(x, bf16_bits_of(hw), None, 1, float(eps), float(eps))
        assert (a != b).mean() > 0.05


# ------------------------------------------------------ the residual boundary

def test_f16_to_f32_exhaustive(oracle):
    """Every f16 bit pattern converts as numpy's float16 -> float32 (a NaN
    stays a NaN)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(b) for b in bits], dtype=np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def _boundary_case(rng, m, small):
    x = rng.standard_normal((m, D)) * (0.08 if small else 1.0)
    if small:
        x = np.clip(x, -0.25, 0.25)
    x = bf16_bits_of(x)
    x[x == 0] = 0x3F80
    x[x == 0x8000] = 0x3F80
    s = (rng.standard_normal((m, D)) * (0.05 if small else 1.0)).astype(np.float32)
    alpha = rng.uniform(0.5, 1.5, D).astype(np.float32)
    beta = rng.uniform(0.5, 1.5, D).astype(np.float32)
    return x, s, alpha, beta


def _weights(rng, kind):
    w = (1.0 + 0.3 * rng.standard_normal(D)).astype(np.float32)
    if kind == "bf16":
        return bf16_bits_of(w), f32_of_bf16(bf16_bits_of(w))
    if kind == "f16":
        h = w.astype(np.float16)
        return h.view(np.uint16), h.astype(np.float32)
    if kind == "f32":
        return w, w
    return None, None


def test_boundary_with_zero_alpha_is_the_two_norms(oracle):
    """Page '...draft_boundary' (module summary): with alpha = 0 and beta = 1
    the residual is the post norm's bf16 output itself (0 * stream adds a
    zero), so the boundary's output is pre_norm(bf16(post_norm(x))), which
    is the (pinned) context norms with one layer: post -> hidden norm, pre ->
    layer norm. FP16 weights read exactly equal their FP32 values."""
    rng = np.random.default_rng(61)
    m = 3
    x, s, _, _ = _boundary_case(rng, m, False)
    alpha = np.zeros(D, dtype=np.float32)
    beta = np.ones(D, dtype=np.float32)
    for pk in ("bf16", "f16", "f32", None):
        for qk in ("bf16", "f16", "f32", None):
            pw, pv = _weights(rng, pk)
            qw, qv = _weights(rng, qk)
            for pin, qin in ((False, False), (True, True), (True, False)):
                _, out = oracle.draft_boundary(x, s, alpha, beta, pw, qw, 1e-6, 2e-6, 0.125, -0.25, pin, qin,
                                               pk or "bf16", qk or "bf16")
                hw = None if pk is None else (pw if pk in ("bf16", "f32") else pv)
                lw = None if qk is None else (qw if qk in ("bf16", "f32") else qv)[None, :]
                want = oracle.context_norms_ex(x, hw, lw, 1, 1e-6, 2e-6, 0.125, -0.25, pin, qin)[0]
                assert np.array_equal(out, want), (pk, qk, pin, qin)


def test_boundary_large_eps_closed_form(oracle):
    """With both eps = 2^20 and small rows, both scales are exactly 2^-10, so
    the boundary is a short chain of rounded FP32 operations: y = (x 2^-10)
    gamma (input-scaled: (gamma x) 2^-10), res = alpha s + beta bf16(y) with
    each product rounded, z = bf16(res), out = bf16((z 2^-10) gamma') (or
    (gamma' z) 2^-10); the new stream is res. Expected values from numpy's
    IEEE float32 ops and a midpoint-rule bf16 rounding, for every weight
    kind, both scalings, FP32 and bf16 streams and non-zero centers."""
    rng = np.random.default_rng(62)
    m = 2
    eps = np.float32(2.0 ** 20)
    r = np.float32(2.0 ** -10)
    pc, qc = np.float32(0.0625), np.float32(-0.125)
    for pk in ("bf16", "f16", "f32", None):
        for qk in ("bf16", "f16", "f32", None):
            x, s, alpha, beta = _boundary_case(rng, m, True)
            pw, pv = _weights(rng, pk)
            qw, qv = _weights(rng, qk)
            for stream_bf16 in (False, True):
                sin = bf16_bits_of(s) if stream_bf16 else s
                sv = f32_of_bf16(sin) if stream_bf16 else s
                for pin in (False, True):
                    for qin in (False, True):
                        new, out = oracle.draft_boundary(x, sin, alpha, beta, pw, qw, float(eps), float(eps),
                                                         float(pc), float(qc), pin, qin, pk or "bf16", qk or "bf16")
                        xf = f32_of_bf16(x)
                        if pv is None:
                            y = xf * r
                        elif pin:
                            y = ((pv + pc) * xf) * r
                        else:
                            y = (xf * r) * (pv + pc)
                        res = alpha * sv + beta * f32_of_bf16(_bf16_round_indep(y))
                        assert np.array_equal(new.view(np.uint32), res.view(np.uint32)), (pk, qk, pin, qin)
                        z = f32_of_bf16(_bf16_round_indep(res))
                        if qv is None:
                            o = z * r
                        elif qin:
                            o = ((qv + qc) * z) * r
                        else:
                            o = (z * r) * (qv + qc)
                        assert np.array_equal(out, _bf16_round_indep(o)), (pk, qk, pin, qin, stream_bf16)


# ------------------------------------------------------------ K-norm + RoPE

def test_head_sumsq_order_golden(oracle):
    with open(os.path.join(GOLDEN, "head_sumsq_order.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        k = np.zeros(64, dtype=np.float32)
        for i, val in case["nonzero"].items():
            k[int(i)] = val
        assert float(oracle.sumsq_head(k)) == case["expected"], case["name"]


def test_knorm_constant_heads(oracle):
    """Page '...draft.context', _ContextKvStoreKernel: r = rsqrt(S/64 + eps),
    n = bf16(k r). A head of +-2^k with eps = 0 gives n = +-1 exactly."""
    for k in (-30, -1, 0, 5, 40):
        for sgn in (1.0, -1.0):
            head = bf16_bits_of(np.full(64, sgn * 2.0 ** k))
            n = oracle.knorm_rope_head(head, None, 0.0)
            assert np.all(n == (0xBF80 if sgn < 0 else 0x3F80))


def test_knorm_against_float64_within_two_ulp(oracle):
    rng = np.random.default_rng(12)
    for _ in range(200):
        scale = 10.0 ** rng.uniform(-4, 4)
        head = bf16_bits_of(rng.standard_normal(64) * scale)
        kf = f32_of_bf16(head).astype(np.float64)
        eps = float(np.float32(1e-6))
        want = kf / math.sqrt(math.fsum(kf ** 2) / 64 + eps)
        got = f32_of_bf16(oracle.knorm_rope_head(head, None, 1e-6)).astype(np.float64)
        assert np.all(np.abs(got - want) <= 2 * 2.0 ** -8 * np.abs(want) + 1e-30)


def _table_row(c, s):
    return bf16_bits_of(np.concatenate([np.full(32, c), np.full(32, s)]))


def test_rope_position_zero_is_identity(oracle):
    """cos 0 = 1, sin 0 = +0 (exact in bf16): the rotation returns n in value;
    +-0 may differ in sign only where a' = (-0) + (+0) or b' = (-0) + (+0)."""
    rng = np.random.default_rng(13)
    row0 = _table_row(1.0, 0.0)
    for _ in range(50):
        head = bf16_bits_of(rng.standard_normal(64))
        head[rng.integers(0, 64, 4)] = 0x8000
        n = oracle.knorm_rope_head(head, None, 1e-6)
        r = oracle.knorm_rope_head(head, row0, 1e-6)
        assert np.array_equal(f32_of_bf16(n), f32_of_bf16(r))


def test_rope_quarter_turns(oracle):
    """(c, s) = (0, 1): (a, b) -> (-b, a); (-1, 0): (-a, -b); (0, -1):
    (b, -a); exact in value (one FMA on exact products)."""
    rng = np.random.default_rng(14)
    head = bf16_bits_of(rng.standard_normal(64))
    n = f32_of_bf16(oracle.knorm_rope_head(head, None, 1e-6))
    a, b = n[0::2], n[1::2]
    for (c, s), (ea, eb) in {(0.0, 1.0): (-b, a), (-1.0, 0.0): (-a, -b), (0.0, -1.0): (b, -a)}.items():
        r = f32_of_bf16(oracle.knorm_rope_head(head, _table_row(c, s), 1e-6))
        assert np.array_equal(r[0::2], ea) and np.array_equal(r[1::2], eb), (c, s)


def test_rope_reads_the_bf16_key(oracle):
    """Page '...draft.context', _ContextKvStoreKernel: the normed key is
    rounded to bf16 before RoPE. With the table row (c, s) = (1, 1) the
    rotation is (n0 - n1, n1 + n0): two bf16 values whose f32 difference and
    sum are exact here, rounded once (torch) - built from the oracle's own
    un-rotated key, so a rotation of the unrounded k * r would differ."""
    import torch

    rng = np.random.default_rng(19)
    row = _table_row(1.0, 1.0)
    for _ in range(50):
        head = bf16_bits_of(rng.standard_normal(64))
        n = f32_of_bf16(oracle.knorm_rope_head(head, None, 1e-6))
        a, b = n[0::2], n[1::2]
        want = np.empty(64, dtype=np.float32)
        want[0::2], want[1::2] = a - b, b + a
        want_bits = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        got = oracle.knorm_rope_head(head, row, 1e-6)
        assert np.array_equal(f32_of_bf16(got), f32_of_bf16(want_bits))


def test_rope_preserves_pair_norms(oracle):
    """A rotation keeps each pair's norm: |out| = |n| sqrt(c^2 + s^2), within
    2^-7 relative (bf16 roundings of n, the table and the result)."""
    from norm_rope_cache_amd import synth

    tab = synth.rope_table(4096)
    rng = np.random.default_rng(15)
    for p in rng.integers(0, 4096, 40):
        head = bf16_bits_of(rng.standard_normal(64))
        n = f32_of_bf16(oracle.knorm_rope_head(head, None, 1e-6)).astype(np.float64)
        r = f32_of_bf16(oracle.knorm_rope_head(head, tab[p], 1e-6)).astype(np.float64)
        cs = f32_of_bf16(tab[p]).astype(np.float64)
        scale = np.sqrt(cs[:32] ** 2 + cs[32:] ** 2)
        nin = np.hypot(n[0::2], n[1::2]) * scale
        nout = np.hypot(r[0::2], r[1::2])
        assert np.all(np.abs(nout - nin) <= 2.0 ** -7 * nin + 1e-6)


def test_rope_specials(oracle):
    """Overflowing heads: S = +Inf, r = +0, n = signed zeros; a NaN element
    makes the head NaN (0x7FC0)."""
    head = bf16_bits_of(np.ones(64))
    head[3] = 0x7F7F
    n = oracle.knorm_rope_head(head, None, 1e-6)
    assert np.all((n & 0x7FFF) == 0)
    head[3] = 0x7FC1
    assert np.all(oracle.knorm_rope_head(head, None, 1e-6) == 0x7FC0)


# ------------------------------------------------------------------- insert

def test_insert_brute_force_tiny(oracle):
    """Brute force on a tiny cache: every cell either holds the (row, head)
    whose slot maps to it (found by searching all rows: block = s // bs,
    page = s % bs) or keeps its prior bits. V bits are copied exactly;
    negative slots and rows >= rows never write."""
    rng = np.random.default_rng(16)
    L, T, H, bs, nb = 2, 12, 2, 4, 5
    rows = 10
    N = 2 * H * 64
    kv = bf16_bits_of(rng.standard_normal((L, T, N)) * 1.8)
    pos = rng.integers(0, 64, T).astype(np.int64)
    tab = bf16_bits_of(rng.uniform(-1, 1, (64, 64)))
    slots = np.stack([rng.permutation(nb * bs)[:rows] for _ in range(L)]).astype(np.int64)
    slots[0, 3] = -1
    slots[1, 0] = -7
    prior = rng.integers(0, 1 << 16, (L, nb, H, bs, 128)).astype(np.uint16)
    caches = prior.copy()
    oracle.context_kv_store(kv, H, pos, slots, tab, caches, bs, 1e-6)
    for l in range(L):
        for b in range(nb):
            for h in range(H):
                for o in range(bs):
                    writers = [t for t in range(rows) if slots[l, t] >= 0
                               and slots[l, t] // bs == b and slots[l, t] % bs == o]
                    cell = caches[l, b, h, o]
                    if not writers:
                        assert np.array_equal(cell, prior[l, b, h, o])
                        continue
                    (t,) = writers
                    kh = kv[l, t, h * 64:(h + 1) * 64]
                    assert np.array_equal(cell[:64], oracle.knorm_rope_head(kh, tab[pos[t]], 1e-6))
                    assert np.array_equal(cell[64:], kv[l, t, (H + h) * 64:(H + h + 1) * 64])


def test_insert_strided_views_and_slot_groups_brute_force(oracle):
    """The store's full operand surface (context page ContextKvStore: a
    strided key-cache view; runtime page _slot_groups: per-layer slot lists
    of their own lengths, None for a layer that stores nothing). Brute force
    over every cell of padded strided buffers: a cell holds the (row, head)
    whose slot maps to it among the layer's first rows_l rows (K-norm + RoPE
    of K by the pinned head routine, V copied) or keeps its prior bits; the
    padding between runs is never written; a None layer is untouched."""
    rng = np.random.default_rng(17)
    L, T, H, bs, nb = 3, 12, 2, 4, 5
    N = 2 * H * 64
    kv = bf16_bits_of(rng.standard_normal((L, T, N)) * 1.8)
    pos = rng.integers(0, 64, T).astype(np.int64)
    tab = bf16_bits_of(rng.uniform(-1, 1, (64, 64)))
    # lists of their own lengths: the first layer's is the shortest
    slots = [rng.permutation(nb * bs)[:6].astype(np.int64), None, rng.permutation(nb * bs)[:11].astype(np.int64)]
    slots[0][3] = -1
    slots[2][0] = -5
    layouts = {
        # backend layout [nb, H, bs, 128] with 8 spare elements after every run and 64 after every block
        "head-major padded": (H * bs * 136 + 64, 136, bs * 136),
        # [nb, bs, H, 128] (page-major) with no padding
        "page-major": (bs * H * 128, H * 128, 128),
    }
    for name, (bstr, pstr, hstr) in layouts.items():
        size = (nb - 1) * bstr + (bs - 1) * pstr + (H - 1) * hstr + 128
        prior = [rng.integers(0, 1 << 16, size).astype(np.uint16) for _ in range(L)]
        caches = [p.copy() for p in prior]
        oracle.context_kv_store_ex(kv, H, pos, slots, tab, caches, bs, nb, bstr, pstr, hstr, 1e-6)
        for l in range(L):
            written = np.zeros(size, dtype=bool)
            for b in range(nb):
                for o in range(bs):
                    for h in range(H):
                        off = b * bstr + o * pstr + h * hstr
                        cell = caches[l][off:off + 128]
                        sl = slots[l]
                        writers = [] if sl is None else [t for t in range(sl.shape[0]) if sl[t] >= 0
                                                         and sl[t] // bs == b and sl[t] % bs == o]
                        if not writers:
                            assert np.array_equal(cell, prior[l][off:off + 128]), (name, l, b, o, h)
                            continue
                        (t,) = writers
                        written[off:off + 128] = True
                        kh = kv[l, t, h * 64:(h + 1) * 64]
                        assert np.array_equal(cell[:64], oracle.knorm_rope_head(kh, tab[pos[t]], 1e-6))
                        assert np.array_equal(cell[64:], kv[l, t, (H + h) * 64:(H + h + 1) * 64])
            assert np.array_equal(caches[l][~written], prior[l][~written]), (name, l)


def test_insert_preconditions(oracle):
    L, T, H, bs, nb = 1, 4, 1, 4, 2
    kv = np.zeros((L, T, 128), dtype=np.uint16)
    caches = np.zeros((L, nb, H, bs, 128), dtype=np.uint16)
    pos = np.zeros(T, dtype=np.int64)
    with pytest.raises(oracle.OracleError):  # duplicate slot
        oracle.context_kv_store(kv, H, pos, np.array([[1, 1, -1, 2]]), None, caches, bs)
    with pytest.raises(oracle.OracleError):  # slot out of range
        oracle.context_kv_store(kv, H, pos, np.array([[8, 1, -1, 2]]), None, caches, bs)
    with pytest.raises(oracle.OracleError):  # position out of range
        oracle.context_kv_store(kv, H, np.array([0, 0, 9, 0]), np.array([[0, 1, 2, 3]]),
                                np.zeros((4, 64), dtype=np.uint16), caches, bs)
    # rows == 0: nothing happens
    oracle.context_kv_store(kv, H, pos, np.zeros((1, 0), dtype=np.int64), None, caches, bs)
    assert not caches.any()


# ---------------------------------------------------------------- projection

def test_project_one_hot_rows_and_zero_rows(oracle):
    """Page '...runtime.draft', ContextKV._project: C = A B. A one-hot row of
    A selects one row of B exactly; a zero row gives zeros."""
    rng = np.random.default_rng(17)
    L, T, Dd, N = 2, 5, 64, 128
    B = bf16_bits_of(rng.standard_normal((L, Dd, N)) * 0.02)
    A = np.zeros((L, T, Dd), dtype=np.uint16)
    for l in range(L):
        for t in range(4):
            A[l, t, (7 * t + l) % Dd] = 0x3F80
    C = oracle.kv_project(A, B)
    for l in range(L):
        for t in range(4):
            assert np.array_equal(C[l, t], f32_of_bf16(B[l, (7 * t + l) % Dd]))
        assert np.all(C[l, 4] == 0)


def test_project_float64_bound(oracle):
    """|C - C64| <= gamma_D sum |a||b| (FP32 recursive summation), C64 from
    numpy's float64 matmul."""
    rng = np.random.default_rng(18)
    L, T, Dd, N = 2, 6, 8192, 128
    A = bf16_bits_of(rng.standard_normal((L, T, Dd)))
    B = bf16_bits_of(rng.standard_normal((L, Dd, N)) * 0.02)
    C = oracle.kv_project(A, B).astype(np.float64)
    Af, Bf = f32_of_bf16(A).astype(np.float64), f32_of_bf16(B).astype(np.float64)
    gD = Dd * 2.0 ** -24 / (1 - Dd * 2.0 ** -24)
    for l in range(L):
        ref = Af[l] @ Bf[l]
        bound = gD * (np.abs(Af[l]) @ np.abs(Bf[l]))
        assert np.all(np.abs(C[l] - ref) <= bound)


def test_project_sequential_order_instance(oracle):
    """The oracle sums in increasing d: 2^24 + 1 + 1 -> 2^24 (each +1 is a
    tie that rounds to even), where a pairwise sum would give 2^24 + 2."""
    A = bf16_bits_of(np.array([[[1.0, 1.0, 1.0, 0.0]]]))
    Bcol = np.zeros((1, 4, 128))
    Bcol[0, 0, :] = 2.0 ** 24
    Bcol[0, 1, :] = 1.0
    Bcol[0, 2, :] = 1.0
    C = oracle.kv_project(A, bf16_bits_of(Bcol))
    assert np.all(C == 2.0 ** 24)


# ------------------------------------------------------------------- chain

def test_chain_composes_the_three_stages(oracle):
    from norm_rope_cache_amd import synth

    cfg = synth.scaled(synth.TINY, 16)
    d = synth.make_inputs(cfg)
    caches = d["caches"].copy()
    normed, kv = oracle.chain(d["x"], d["hidden_w"], d["pre_w"], cfg.L, d["w_kv"], cfg.H, d["positions"],
                              d["slots"], d["cos_sin"], caches, cfg.block_size)
    assert np.array_equal(normed, oracle.context_norms(d["x"], d["hidden_w"], d["pre_w"], cfg.L))
    assert np.array_equal(kv, oracle.bf16(oracle.kv_project(normed, d["w_kv"])))
    c2 = d["caches"].copy()
    oracle.context_kv_store(kv, cfg.H, d["positions"], d["slots"], d["cos_sin"], c2, cfg.block_size)
    assert np.array_equal(c2, caches)


# --------------------------------------------------------------- generator

def test_splitmix64_known_answers():
    from norm_rope_cache_amd import synth

    with open(os.path.join(GOLDEN, "splitmix64.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        got = [int(v) for v in synth.splitmix64(case["seed"], len(case["outputs"]))]
        assert got == [int(s, 0) for s in case["outputs"]]
