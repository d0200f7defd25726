"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
worked example printed on a page, a closed form, an exact rational
computation, an independent scalar re-derivation, or an invariant.  The
docstring of each test names what pins it.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import OracleDataError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _scalar_digits(b):
    """Base-3 digits of b, least significant first, by repeated division."""
    out = []
    for _ in range(5):
        b, r = divmod(b, 3)
        out.append(r)
    return out


# ---------------------------------------------------------------- fp rounding

def _exact_nearest_even(x, candidates):
    """Nearest of `candidates` (sorted Fractions) to Fraction x; ties -> even index."""
    best = min(range(len(candidates)), key=lambda i: (abs(candidates[i] - x), i % 2))
    return best


def test_f16_identity_all_patterns():
    """Every finite fp16 value converts back to its own bit pattern (IEEE 754)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.f16_bits_to_f64(bits)
    keep = ~np.isnan(v)
    out = oracle.f64_to_f16_bits(v[keep])
    zero_neg = bits[keep] == 0x8000
    assert np.array_equal(out[~zero_neg], bits[keep][~zero_neg])
    assert out[zero_neg][0] in (0x8000,)


def test_f16_midpoints_ties_to_even():
    """Midpoints between neighbouring positive fp16 values round to the even
    pattern; just above / below a midpoint rounds away / towards (IEEE 754)."""
    lo = np.arange(0, 0x7BFF, dtype=np.uint16)              # up to 65504 - ulp
    hi = lo + np.uint16(1)
    a, b = oracle.f16_bits_to_f64(lo), oracle.f16_bits_to_f64(hi)
    mid = (a + b) / 2                                        # exact in float64
    got = oracle.f64_to_f16_bits(mid)
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, even)
    up = np.nextafter(mid, np.inf)
    dn = np.nextafter(mid, -np.inf)
    assert np.array_equal(oracle.f64_to_f16_bits(up), hi)
    assert np.array_equal(oracle.f64_to_f16_bits(dn), lo)


def test_f16_overflow_and_against_numpy():
    """65504 is the largest finite fp16; 65520 (the midpoint to 2**16) rounds
    to infinity; random values agree with numpy's own float64->float16 cast,
    an independent implementation."""
    assert oracle.f64_to_f16_bits(np.array([65504.0]))[0] == 0x7BFF
    assert oracle.f64_to_f16_bits(np.array([65519.99]))[0] == 0x7BFF
    assert oracle.f64_to_f16_bits(np.array([65520.0]))[0] == 0x7C00
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 5, 200000),
        rng.uniform(-2 ** -14, 2 ** -14, 50000),
    ])
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f64_to_f16_bits(x), ref)


def test_f16_exact_rationals():
    """A few values checked against exact rational nearest-even rounding."""
    grid = [Fraction(float(v))
            for v in oracle.f16_bits_to_f64(np.arange(0x3C00, 0x3C10, dtype=np.uint16))]
    for num in range(0, 61):
        x = grid[0] + (grid[15] - grid[0]) * Fraction(num, 60)
        i = _exact_nearest_even(x, grid)
        got = oracle.f64_to_f16_bits(np.array([float(x)]))[0]
        if float(x) == x:                                   # exact in float64
            assert got == 0x3C00 + i


def test_bf16_identity_midpoints_and_bits():
    """bf16: identity over all finite patterns, ties to even at midpoints, and
    agreement with the integer bit formula on float32 inputs."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    keep = ~np.isnan(v) & (bits != 0x8000)
    assert np.array_equal(oracle.f64_to_bf16_bits(v[keep]), bits[keep])
    lo = np.arange(0, 0x7F7F, dtype=np.uint16)
    hi = lo + np.uint16(1)
    mid = (oracle.bf16_bits_to_f64(lo) + oracle.bf16_bits_to_f64(hi)) / 2
    assert np.array_equal(oracle.f64_to_bf16_bits(mid), np.where(lo % 2 == 0, lo, hi))
    rng = np.random.default_rng(12)
    f = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    ref = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_bits(f.astype(np.float64)), ref)


# ---------------------------------------------------------------- packing

def test_worked_example_183():
    """The page's worked example: trits (-1, 0, 1, -1, 1) <-> byte 183."""
    lines = {ln[0]: ln[1:] for ln in _golden_lines("trit_byte_example.txt")}
    trits = np.array([[int(v) for v in lines["trits"]]], dtype=np.int8)
    byte = int(lines["byte"][0])
    codes = oracle.pack(trits, 5)
    assert codes.shape == (1, 1, 1) and int(codes[0, 0, 0]) == byte
    back = oracle.ternary.unpack_trits(codes, 5, 5)
    assert np.array_equal(back, trits)


def test_all_243_words_round_trip():
    """All 243 five-trit words against an independent scalar base-3 calculation."""
    words = np.array([[d - 1 for d in _scalar_digits(b)] for b in range(243)], dtype=np.int8)
    t = words.reshape(1, 243 * 5)
    codes = oracle.pack(t, 5)
    assert np.array_equal(codes.reshape(-1), np.arange(243, dtype=np.uint8))
    assert np.array_equal(oracle.ternary.unpack_trits(codes, 243 * 5, 5), t)
    for b in (0, 1, 121, 182, 242):
        digits = _scalar_digits(b)
        assert sum(d * 3 ** q for q, d in enumerate(digits)) == b


@pytest.mark.parametrize("bad", range(243, 256))
def test_bytes_243_to_255_rejected(bad):
    """Byte values 243..255 are not five-trit words and are rejected."""
    codes = np.full((2, 1, 13), 121, dtype=np.uint8)
    codes[1, 0, 7] = bad
    with pytest.raises(OracleDataError) as e:
        oracle.unpack(codes, np.zeros((2, 1), np.uint16), 64, 64)
    assert e.value.kind == "code"


def test_padding_must_decode_to_zero():
    """G=64: byte 12 holds trits 60..63 and one padding digit that must be 1
    (trit 0); a ragged final group pads every unused slot the same way."""
    codes = np.full((1, 1, 13), 121, dtype=np.uint8)
    codes[0, 0, 12] = 121 + 81                      # padding digit 4 -> 2
    with pytest.raises(OracleDataError) as e:
        oracle.unpack(codes, np.zeros((1, 1), np.uint16), 64, 64)
    assert e.value.kind == "padding"
    codes[0, 0, 12] = 121 - 1                       # digit 0 is data: fine
    oracle.unpack(codes, np.zeros((1, 1), np.uint16), 64, 64)
    # ragged: K = 70, G = 64 -> second group has 6 members, bytes 2..12 padding
    rng = np.random.default_rng(3)
    W = rng.standard_normal((3, 70)).astype(np.float32)
    c, s = oracle.quantize_pack(W, 64)
    assert c.shape == (3, 2, 13)
    assert np.all(c[:, 1, 2:] == 121)                # 1 + 3 + 9 + 27 + 81
    assert np.all(c[:, 1, 1] % 3 == c[:, 1, 1] % 3)
    assert np.all(c[:, 1, 1] // 3 == 40)             # trit 5 is data, digits 1..4 pad
    bad = c.copy()
    bad[0, 1, 5] = 120
    with pytest.raises(OracleDataError):
        oracle.unpack(bad, s, 70, 64)
    w = oracle.unpack(c, s, 70, 64)
    assert w.shape == (3, 70)


def test_group_boundaries_and_rows():
    """Groups never straddle rows; a group's bytes depend only on its own
    64 weights (changing one weight changes one group of one row)."""
    rng = np.random.default_rng(4)
    W = rng.standard_normal((4, 192)).astype(np.float32)
    c0, s0 = oracle.quantize_pack(W, 64)
    W2 = W.copy()
    W2[2, 64 + 17] *= 3.0
    c1, s1 = oracle.quantize_pack(W2, 64)
    diff_groups = {(r, g) for r in range(4) for g in range(3)
                   if not (np.array_equal(c0[r, g], c1[r, g]) and s0[r, g] == s1[r, g])}
    assert diff_groups <= {(2, 1)} and (2, 1) in diff_groups


def test_byte_counts():
    """The page's byte accounting: G=64 -> 13 + 2 = 15 B -> 1.875 bits/weight."""
    for G, cb, gb, bpw in _golden_lines("byte_counts.txt"):
        G, cb, gb, bpw = int(G), int(cb), int(gb), float(bpw)
        assert oracle.bytes_per_group(G) == cb
        assert cb + 2 == gb
        assert oracle.bits_per_weight(G) == bpw
        W = np.ones((3, 4 * G), np.float32)
        c, s = oracle.quantize_pack(W, G)
        assert c.nbytes + s.nbytes == 3 * 4 * gb


# ---------------------------------------------------------------- quantizer

def _one_group(vals):
    return oracle.quantize(np.array([vals], dtype=np.float32), len(vals))


def test_scale_closed_form_and_both_ties():
    """32 x 0.75 and 32 x (-0.25): mean |W| = 0.5 exactly, s = 0.5;
    0.75/0.5 = 1.5 rounds (to even) to 2 and clips to 1; -0.25/0.5 = -0.5
    rounds (to even) to 0."""
    vals = [0.75] * 32 + [-0.25] * 32
    rng = np.random.default_rng(5)
    perm = rng.permutation(64)
    vals = [vals[i] for i in perm]
    s, t = _one_group(vals)
    assert s[0, 0] == 0x3800                           # fp16 0.5
    expect = [1 if v == 0.75 else 0 for v in vals]
    assert t[0].tolist() == expect


def test_scale_constant_spike_zero_tiny():
    """Constant c: s = fp16(c), all t = 1.  One spike v among zeros:
    s = fp16(v/64), one t = sign(v).  All zero: s = 0, bytes 121, W_hat 0.
    Mean <= 2**-25 rounds to s = 0: all-zero group although |W| > 0."""
    s, t = _one_group([0.3] * 64)
    assert s[0, 0] == np.float16(0.3).view(np.uint16) and np.all(t == 1)
    vals = [0.0] * 64
    vals[40] = -0.64
    s, t = _one_group(vals)
    assert s[0, 0] == np.float16(0.01).view(np.uint16)
    assert t[0, 40] == -1 and np.count_nonzero(t) == 1
    W = np.zeros((2, 64), np.float32)
    c, s = oracle.quantize_pack(W, 64)
    assert np.all(s == 0) and np.all(c == 121)
    assert np.all(oracle.unpack(c, s, 64, 64) == 0)
    tiny = np.full((1, 64), 2.0 ** -26, np.float32)
    s, t = oracle.quantize(tiny, 64)
    assert s[0, 0] == 0 and np.all(t == 0)
    tiny2 = np.full((1, 64), 2.0 ** -25 * 1.001, np.float32)
    s, t = oracle.quantize(tiny2, 64)
    assert s[0, 0] == 1 and np.all(t == 1)             # smallest subnormal fp16


def test_scale_is_one_rounding_of_the_exact_mean():
    """s equals the nearest-even fp16 of the exact rational mean (computed with
    Fractions) on random groups, including ragged ones."""
    rng = np.random.default_rng(6)
    for n in (64, 64, 64, 37, 5, 128):
        for _ in range(60):
            w = (rng.standard_normal(n) * 10.0 ** rng.integers(-6, 3)).astype(np.float32)
            s, _ = oracle.quantize(w[None, :], max(n, 64) if n != 128 else 128)
            exact = sum(Fraction(float(abs(v))) for v in w) / n
            lo = float(exact)
            grid = oracle.f16_bits_to_f64(np.arange(0, 0x7C00, dtype=np.uint16))
            i = np.searchsorted(grid, lo)
            cands = [j for j in (i - 1, i, i + 1) if 0 <= j < len(grid)]
            best = min(cands, key=lambda j: (abs(Fraction(float(grid[j])) - exact), j % 2))
            assert s[0, 0] == best


def test_sign_and_ties_against_scalar_rule():
    """t = clip(RNE(W/s), -1, 1) for every weight, re-derived per weight in
    exact rational arithmetic with Python's round (ties to even)."""
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    W[0, :4] = [0.5, -0.5, 0.25, 1.0]
    s, t = oracle.quantize(W, 64)
    sv = oracle.f16_bits_to_f64(s)
    for r in range(6):
        for k in range(128):
            sc = Fraction(float(sv[r, k // 64]))
            q = 0 if sc == 0 else max(-1, min(1, round(Fraction(float(W[r, k])) / sc)))
            assert t[r, k] == q


def test_nonfinite_and_overflow_are_range_errors():
    for bad in (np.nan, np.inf, -np.inf):
        W = np.zeros((1, 64), np.float32)
        W[0, 3] = bad
        with pytest.raises(OracleDataError) as e:
            oracle.quantize(W, 64)
        assert e.value.kind == "range"
    W = np.full((1, 64), 65520.0, np.float32)
    with pytest.raises(OracleDataError):
        oracle.quantize(W, 64)
    W = np.full((1, 64), 65519.0, np.float32)
    s, _ = oracle.quantize(W, 64)
    assert s[0, 0] == 0x7BFF


def test_value_set_and_error_monotone():
    """At most 3 distinct reconstructed values per group ({-s, 0, s}), at most
    9 with two planes; |W - s t| <= |W| for every weight (t != 0 only when
    |W| > s/2 with the sign of W), and plane 2 never increases it."""
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    c, s = oracle.quantize_pack(W, 64)
    w = oracle.unpack(c, s, 256, 64)
    sv = oracle.f16_bits_to_f64(s)
    for r in range(32):
        for g in range(4):
            vals = set(np.unique(w[r, g * 64:(g + 1) * 64]).tolist())
            assert vals <= {-sv[r, g], 0.0, sv[r, g]}
    assert np.all(np.abs(W - w) <= np.abs(W))
    (c1, s1), (c2, s2) = oracle.two_plane(W, 64)
    w1 = oracle.unpack(c1, s1, 256, 64)
    w2 = oracle.unpack(c2, s2, 256, 64)
    R = W - w1.astype(np.float32)
    assert np.all(np.abs(R - w2) <= np.abs(R))
    both = w1 + w2
    for r in range(32):
        for g in range(4):
            assert len(np.unique(both[r, g * 64:(g + 1) * 64])) <= 9
    assert np.sum((W - both) ** 2) < 0.5 * np.sum((W - w1) ** 2)


def test_two_plane_plane1_is_single_plane_and_residual_rule():
    """Plane 1 of two_plane is the single-plane package; plane 2 is the
    single-plane package of fl32(W - s1 t1)."""
    rng = np.random.default_rng(10)
    W = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    (c1, s1), (c2, s2) = oracle.two_plane(W, 64)
    cs, ss = oracle.quantize_pack(W, 64)
    assert np.array_equal(c1, cs) and np.array_equal(s1, ss)
    t1 = oracle.ternary.unpack_trits(c1, 128, 64)
    sv = np.repeat(oracle.f16_bits_to_f64(s1), 64, axis=1)
    R = np.empty_like(W)
    for r in range(8):
        for k in range(128):
            R[r, k] = np.float32(W[r, k]) - np.float32(sv[r, k] * t1[r, k])
    cr, sr = oracle.quantize_pack(R, 64)
    assert np.array_equal(c2, cr) and np.array_equal(s2, sr)


def test_gaussian_relative_mse():
    """Statistical sanity: on N(0, 1) weights the relative MSE of the
    single-plane quantizer is near the closed form for a population mean-abs
    scale s = sqrt(2/pi):  1 - 2 s 2 phi(s/2) + s^2 2 (1 - Phi(s/2)) ~ 0.2634.
    Per-group sample scales move it by a few thousandths."""
    sp = math.sqrt(2 / math.pi)
    c = sp / 2
    phi = math.exp(-c * c / 2) / math.sqrt(2 * math.pi)
    Phi = 0.5 * (1 + math.erf(c / math.sqrt(2)))
    closed = 1 - 2 * sp * 2 * phi + sp * sp * 2 * (1 - Phi)
    rng = np.random.default_rng(13)
    W = rng.standard_normal((1000, 1024)).astype(np.float32)
    cc, s = oracle.quantize_pack(W, 64)
    w = oracle.unpack(cc, s, 1024, 64)
    rel = np.sum((W - w) ** 2) / np.sum(W.astype(np.float64) ** 2)
    assert abs(closed - 0.2634) < 1e-3
    assert abs(rel - closed) < 0.01


# ---------------------------------------------------------------- Route B

def _ladders():
    out = {}
    for ln in _golden_lines("routeb_ladder.txt"):
        out[ln[0]] = np.array([float(v) for v in ln[1:]], dtype=np.float32)
    return out


def test_code_words_digit_order():
    """codes = base-3 encoding of c_1..c_5 with c_1 most significant:
    sum_i (c_i + 1) 3^(5-i) == b for every code."""
    cw = oracle.code_words().astype(int)
    for b in range(243):
        assert sum((cw[b, i - 1] + 1) * 3 ** (5 - i) for i in range(1, 6)) == b


def test_table_integer_ladder_closed_form():
    """With the integer ladder (81, 27, 9, 3, 1) the code book is exactly
    T[b] = b - 121 (the balanced-ternary value of the word)."""
    T = oracle.rb_table(np.array([81, 27, 9, 3, 1], np.float32))
    assert np.array_equal(T, (np.arange(243) - 121).astype(np.float32))


def test_table_balanced_ladder_and_symmetry():
    """S0 = (1, 1/3, 1/9, 1/27, 1/81): T[b] ~ (b - 121)/81, strictly
    increasing, T[121] = 0, T[242 - b] = -T[b] exactly.  The fitted S of the
    paper keeps the antisymmetry and T[121] = 0."""
    lad = _ladders()
    T = oracle.rb_table(lad["S0"])
    assert T[121] == 0
    assert np.all(np.diff(T) > 0)
    assert np.allclose(T, (np.arange(243) - 121) / 81.0, rtol=0, atol=1e-6)
    assert np.array_equal(T[::-1], -T)
    Ts = oracle.rb_table(lad["S"])
    assert Ts[121] == 0 and np.array_equal(Ts[::-1], -Ts)


def test_table_entries_are_the_exact_sums():
    """For the ladders of the workloads (a_i = 0.5^(i-1) u_i, u_i in
    [0.8, 1.2]) each entry is the nearest fp32 of the exact rational sum."""
    import workloads
    for seed in range(5):
        a = workloads.routeb_gemv(seed=seed, N=1, K=1, M=1)["ladder"]
        T = oracle.rb_table(a)
        cw = oracle.code_words().astype(int)
        for b in range(243):
            exact = sum(Fraction(int(cw[b, i])) * Fraction(float(a[i])) for i in range(5))
            assert Fraction(float(exact)) == exact
            assert T[b] == np.float32(float(exact))


def test_rb_weights_definition():
    """W_hat[n, k] = alpha * T[codes[n, k]] * rho_n, scalar re-derivation."""
    rng = np.random.default_rng(14)
    a = np.array([1.0, 0.34, 0.11, 0.04, 0.013], np.float32)
    T = oracle.rb_table(a)
    codes = rng.integers(0, 243, (5, 9), dtype=np.uint8)
    rho = np.array([0.5, 1.0, 1.25, 0.75, 1.5], np.float16).view(np.uint16)
    w = oracle.rb_weights(codes, T, np.float32(0.02), rho)
    rv = rho.view(np.float16)
    for n in range(5):
        for k in range(9):
            ref = Fraction(float(np.float32(0.02))) * Fraction(float(T[codes[n, k]])) * Fraction(float(rv[n]))
            assert abs(Fraction(w[n, k]) - ref) <= abs(ref) * Fraction(1, 2 ** 52)


# ---------------------------------------------------------------- matmul

def _bf16(rng, shape, scale=1.0):
    import workloads
    return workloads.bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _exact_matmul(xb, w_exact_rows, bias=None):
    """Pure-Python exact rational y and B for tiny shapes."""
    x = [[Fraction(float(v)) for v in row] for row in oracle.bf16_bits_to_f64(xb)]
    M, N = len(x), len(w_exact_rows)
    y = [[sum(x[m][k] * w_exact_rows[n][k] for k in range(len(x[m]))) for n in range(N)] for m in range(M)]
    B = [[sum(abs(x[m][k] * w_exact_rows[n][k]) for k in range(len(x[m]))) for n in range(N)] for m in range(M)]
    if bias is not None:
        for m in range(M):
            for n in range(N):
                y[m][n] += Fraction(float(bias[n]))
                B[m][n] += abs(Fraction(float(bias[n])))
    return y, B


def _scalar_ternary_rows(codes, s_bits, K, G):
    """Weights decoded one byte at a time with the scalar digit routine."""
    rows = []
    sv = oracle.f16_bits_to_f64(s_bits)
    nb = oracle.bytes_per_group(G)
    for n in range(codes.shape[0]):
        row = []
        for k in range(K):
            g, j = divmod(k, G)
            byte = int(codes[n, g, j // 5])
            d = _scalar_digits(byte)[j % 5]
            row.append(Fraction(float(sv[n, g])) * (d - 1))
        rows.append(row)
    assert nb == codes.shape[2]
    return rows


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (3, 7, 128), (5, 4, 320), (16, 2, 64), (2, 3, 70)])
def test_ternary_matmul_brute_force(M, N, K):
    """Oracle y and B against exact rational arithmetic on tiny shapes, with
    the weights re-decoded byte by byte (catches transposes, index and sign
    mistakes); the oracle's float64 result is within 1e-12 B of exact."""
    rng = np.random.default_rng(100 + M * 31 + N * 7 + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xb = _bf16(rng, (M, K))
    c, s = oracle.quantize_pack(W, 64)
    y, B = oracle.matmul_ref(xb, oracle.ternary_weights(K, 64, c, s))
    ye, Be = _exact_matmul(xb, _scalar_ternary_rows(c, s, K, 64))
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= Be[m][n] * Fraction(1, 10 ** 12)
            assert abs(Fraction(B[m, n]) - Be[m][n]) <= Be[m][n] * Fraction(1, 10 ** 12)


def test_two_plane_matmul_brute_force():
    rng = np.random.default_rng(101)
    W = (rng.standard_normal((5, 128)) * 0.02).astype(np.float32)
    xb = _bf16(rng, (3, 128))
    (c1, s1), (c2, s2) = oracle.two_plane(W, 64)
    y, B = oracle.matmul_ref(xb, oracle.ternary_weights(128, 64, c1, s1, c2, s2))
    r1 = _scalar_ternary_rows(c1, s1, 128, 64)
    r2 = _scalar_ternary_rows(c2, s2, 128, 64)
    rows = [[a + b for a, b in zip(p, q)] for p, q in zip(r1, r2)]
    ye, Be = _exact_matmul(xb, rows)
    for m in range(3):
        for n in range(5):
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= Be[m][n] * Fraction(1, 10 ** 12)


@pytest.mark.parametrize("with_rho,with_bias", [(False, False), (True, False), (True, True)])
def test_routeb_matmul_brute_force(with_rho, with_bias):
    rng = np.random.default_rng(102)
    a = np.array([1.0, 0.33, 0.115, 0.037, 0.012], np.float32)
    T = oracle.rb_table(a)
    N, K, M = 6, 40, 4
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    rho = rng.uniform(0.5, 1.5, N).astype(np.float16).view(np.uint16) if with_rho else None
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    xb = _bf16(rng, (M, K))
    y, B = oracle.matmul_ref(xb, oracle.rb_weights(codes, T, np.float32(0.02), rho), bias)
    rv = rho.view(np.float16) if with_rho else np.ones(N)
    rows = [[Fraction(float(np.float32(0.02))) * Fraction(float(T[codes[n, k]])) * Fraction(float(rv[n]))
             for k in range(K)] for n in range(N)]
    ye, Be = _exact_matmul(xb, rows, bias)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= Be[m][n] * Fraction(1, 10 ** 12)


def test_matmul_special_cases():
    """One-hot x picks a column of W_hat exactly; x = 0 gives 0; with
    integer-valued x and power-of-two scales every partial sum is exact."""
    rng = np.random.default_rng(103)
    W = (rng.standard_normal((9, 128)) * 0.02).astype(np.float32)
    c, s = oracle.quantize_pack(W, 64)
    w = oracle.ternary_weights(128, 64, c, s)
    import workloads
    eye = workloads.bf16_bits(np.eye(128, dtype=np.float32))
    y, _ = oracle.matmul_ref(eye, w)
    assert np.array_equal(y, w.T)
    y0, B0 = oracle.matmul_ref(np.zeros((2, 128), np.uint16), w)
    assert np.all(y0 == 0) and np.all(B0 == 0)


def test_grouped_reduces_to_dense():
    """Grouped matmul with every (token, slot) routed to one expert equals the
    dense matmul with that expert's weights, per slot."""
    rng = np.random.default_rng(104)
    Ws = [(rng.standard_normal((6, 64)) * 0.02).astype(np.float32) for _ in range(3)]
    pk = [oracle.quantize_pack(W, 64) for W in Ws]
    xb = _bf16(rng, (4, 64))
    ids = np.full((4, 2), 1, np.int32)
    y, B = oracle.grouped_ref(xb, ids, lambda e: oracle.ternary_weights(64, 64, *pk[e]))
    yd, Bd = oracle.matmul_ref(xb, oracle.ternary_weights(64, 64, *pk[1]))
    for j in range(2):
        assert np.array_equal(y[:, j], yd) and np.array_equal(B[:, j], Bd)
    ids = np.array([[0, 2], [1, 0], [2, 1], [0, 1]], np.int32)
    y, _ = oracle.grouped_ref(xb, ids, lambda e: oracle.ternary_weights(64, 64, *pk[e]))
    for t in range(4):
        for j in range(2):
            ye, _ = oracle.matmul_ref(xb[t:t + 1], oracle.ternary_weights(64, 64, *pk[ids[t, j]]))
            assert np.array_equal(y[t, j], ye[0])


def test_check_bound_logic():
    """The acceptance rule: |y - y_ref| <= 2e-3 B, no NaN/Inf, B = 0 needs equality."""
    yr = np.array([1.0, 0.0, -2.0])
    B = np.array([10.0, 0.0, 2.0])
    assert oracle.check_bound(yr + [0.0199, 0.0, 0.0039], yr, B)["ok"]
    assert not oracle.check_bound(yr + [0.0201, 0.0, 0.0], yr, B)["ok"]
    assert not oracle.check_bound(yr + [0.0, 1e-30, 0.0], yr, B)["ok"]
    assert not oracle.check_bound(np.array([np.nan, 0.0, -2.0]), yr, B)["ok"]


def test_check_bound_bf16_allowance():
    """bf16-stored results may also differ by half a bf16 spacing of y_ref:
    2^-8 at 1.0 <= |y| < 2, 2^-9 at 0.5 <= |y| < 1."""
    assert oracle.matmul.bf16_half_spacing(np.array([1.0, 1.99, 0.75]))[0] == 2.0 ** -8
    assert oracle.matmul.bf16_half_spacing(np.array([0.75]))[0] == 2.0 ** -9
    yr, B = np.array([1.5]), np.array([1.5])
    assert oracle.check_bound(yr + 0.0035, yr, B, stored="bf16")["ok"]
    assert not oracle.check_bound(yr + 0.0035, yr, B)["ok"]
    assert not oracle.check_bound(yr + 0.0075, yr, B, stored="bf16")["ok"]


# ---------------------------------------------------------- Route B encoder

def _balanced_ternary(n, digits=5):
    """Digits (most significant first) of the integer n in balanced ternary,
    by repeated division with remainders in {-1, 0, 1}."""
    out = []
    for _ in range(digits):
        r = n % 3
        if r == 2:
            r = -1
        out.append(r)
        n = (n - r) // 3
    assert n == 0
    return out[::-1]


def test_encode_worked_examples():
    """Hand-worked words of tests/golden/routeb_encode_example.txt (Route B,
    sections 3.1 and 3.2), including the tie at |r| = s_1 / 2 and the strict
    zero-bias test."""
    lad = _ladders()["S0"]
    W = np.array([[0.9, -0.5, 1.0, 0.0]], np.float32)
    for ln in _golden_lines("routeb_encode_example.txt"):
        x, zeta = float(ln[0]), float(ln[1])
        word, code = [int(v) for v in ln[2:7]], int(ln[7])
        assert sum((c + 1) * 3 ** (4 - i) for i, c in enumerate(word)) == code
        codes, alpha, rho = oracle.rb_encode(W, lad, zeta=zeta)
        assert alpha == np.float32(1.0) and rho is None
        k = int(np.flatnonzero(W[0] == np.float32(x))[0])
        assert int(codes[0, k]) == code, (x, zeta)
        assert list(oracle.code_words()[code]) == word


def test_encode_balanced_ladder_is_nearest_multiple_of_one_81st():
    """With S0 = (1, 1/3, 1/9, 1/27, 1/81) the greedy word of r in [-1, 1] is
    the balanced-ternary spelling of round(81 r) (away from the half-way
    points, where the fp32 ladder and float64 rounding may tip a step)."""
    lad = _ladders()["S0"]
    rng = np.random.default_rng(3)
    r = rng.uniform(-1, 1, 4000).astype(np.float32)
    r[0] = 1.0                                           # alpha = 1 exactly
    codes, alpha, _ = oracle.rb_encode(r[None, :], lad)
    assert alpha == 1.0
    cw = oracle.code_words()
    checked = 0
    for k in range(r.size):
        t = 81.0 * float(r[k])
        if abs(t - math.floor(t) - 0.5) < 1e-4:
            continue
        n = int(math.floor(t + 0.5))
        assert list(cw[codes[0, k]]) == _balanced_ternary(n), (r[k], n)
        checked += 1
    assert checked > 3900


def test_encode_greedy_residual_bound_and_decode():
    """Balanced ladder: every |r_0| <= 1 is reconstructed to within s_5 / 2
    (plus rounding), and alpha * T[code] is the decoded weight of section 3.2."""
    lad = _ladders()["S0"]
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((7, 300)) * 0.02).astype(np.float32)
    codes, alpha, _ = oracle.rb_encode(W, lad)
    assert alpha == np.abs(W).max()
    T = oracle.rb_table(lad).astype(np.float64)
    r0 = W.astype(np.float64) / float(alpha)
    assert np.all(np.abs(r0 - T[codes]) <= 0.5 / 81 + 1e-7)
    w_hat = oracle.rb_weights(codes, oracle.rb_table(lad), alpha)
    assert np.all(np.abs(W - w_hat) <= float(alpha) * (0.5 / 81 + 1e-7))


def test_encode_per_row_scale():
    """Section 3.3: r_0 = W / alpha_n, so each row's largest |W| spells
    (+-1, 0, 0, 0, 0) (codes 202 and 40 under S0); rho_n = fp16(alpha_n /
    alpha) against numpy's float64 -> float16 rounding; alpha = max |W|."""
    lad = _ladders()["S0"]
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((9, 70)) * rng.uniform(0.01, 1.0, (9, 1))).astype(np.float32)
    W[3, 5] = -np.abs(W[3]).max() * 1.5                  # a negative row maximum
    codes, alpha, rho = oracle.rb_encode(W, lad, per_row=True)
    a_n = np.abs(W).max(axis=1)
    assert alpha == np.abs(W).max()
    for n in range(W.shape[0]):
        k = int(np.argmax(np.abs(W[n])))
        assert int(codes[n, k]) == (202 if W[n, k] > 0 else 40)
    want = (a_n.astype(np.float64) / float(alpha)).astype(np.float16).view(np.uint16)
    assert np.array_equal(rho, want)
    # the row-normalised words equal the global encoding of W / alpha_n
    for n in range(W.shape[0]):
        row = (W[n].astype(np.float64) / float(a_n[n])).astype(np.float32)
        c_row, _, _ = oracle.rb_encode(row[None, :], lad)
        exact = np.all(W[n].astype(np.float64) / float(a_n[n]) == row.astype(np.float64))
        if exact:
            assert np.array_equal(c_row[0], codes[n])


def test_encode_zero_scale_and_errors():
    """Zero rows (and an all-zero matrix) give the all-zero word 121 and
    rho = 0; non-finite weights are rejected."""
    lad = _ladders()["S"]
    W = np.zeros((3, 10), np.float32)
    W[1, 2] = 0.5
    codes, alpha, rho = oracle.rb_encode(W, lad, per_row=True)
    assert alpha == 0.5
    assert np.all(codes[[0, 2]] == 121) and rho[0] == 0 and rho[2] == 0
    assert rho[1] == np.float16(1.0).view(np.uint16)
    codes, alpha, _ = oracle.rb_encode(np.zeros((2, 4), np.float32), lad)
    assert alpha == 0 and np.all(codes == 121)
    for bad in (np.nan, np.inf, -np.inf):
        W2 = W.copy()
        W2[0, 0] = bad
        with pytest.raises(ValueError):
            oracle.rb_encode(W2, lad)


def test_encode_zero_bias_below_one_half_changes_nothing():
    """|r| < s/2 already makes 0 the nearest step, so a zero-bias zeta <= 1/2
    leaves every word unchanged, while zeta = 1 only ever turns steps to 0
    where |r| < s_i."""
    lad = _ladders()["S"]
    rng = np.random.default_rng(6)
    W = rng.standard_normal((5, 400)).astype(np.float32)
    c0, _, _ = oracle.rb_encode(W, lad)
    for z in (0.1, 0.25, 0.5):
        cz, _, _ = oracle.rb_encode(W, lad, zeta=z)
        assert np.array_equal(c0, cz)
    c1, _, _ = oracle.rb_encode(W, lad, zeta=1.0)
    w0, w1 = oracle.code_words()[c0], oracle.code_words()[c1]
    assert np.count_nonzero(w1) < np.count_nonzero(w0)


def test_encode_head_blocks():
    """Section 8.2 per-head prosody as row blocks: one block equals the
    global encoding with rho = 1; blocks of one row equal the per-row scale;
    each block's largest |W| spells (+-1, 0, 0, 0, 0) under S0; rho_h is
    numpy's fp16 of alpha_h / alpha; a ragged last block works; and the
    decoded weight of row n uses rho_{n // b}."""
    lad = _ladders()["S0"]
    rng = np.random.default_rng(7)
    N, K, b = 10, 40, 4
    W = (rng.standard_normal((N, K)) * rng.uniform(0.05, 2.0, (N, 1))).astype(np.float32)
    cg, ag, _ = oracle.rb_encode(W, lad)
    c1, a1, r1 = oracle.rb_encode(W, lad, rho_rows=N)
    assert np.array_equal(c1, cg) and a1 == ag and list(r1) == [np.float16(1).view(np.uint16)]
    cr, _, rr = oracle.rb_encode(W, lad, per_row=True)
    cb, _, rb = oracle.rb_encode(W, lad, rho_rows=1)
    assert np.array_equal(cr, cb) and np.array_equal(rr, rb)
    codes, alpha, rho = oracle.rb_encode(W, lad, rho_rows=b)
    assert rho.shape == (3,)                           # rows 8, 9 form the last block
    a_h = oracle.rb_block_scales(W, b)
    for h in range(3):
        blk = np.abs(W[h * b:(h + 1) * b])
        assert a_h[h] == blk.max()
        n, k = np.unravel_index(int(np.argmax(blk)), blk.shape)
        n += h * b
        assert int(codes[n, k]) == (202 if W[n, k] > 0 else 40)
    want = (a_h.astype(np.float64) / float(alpha)).astype(np.float16).view(np.uint16)
    assert np.array_equal(rho, want)
    T = oracle.rb_table(lad)
    per_row_rho = np.repeat(rho, b)[:N]
    assert np.array_equal(oracle.rb_weights(codes, T, alpha, rho, rho_rows=b),
                          oracle.rb_weights(codes, T, alpha, per_row_rho))


def test_hot_prefix_weights():
    """FUCINA "The method": with the hot prefix covering every expert the
    experts are the two-plane sums, with an empty prefix the single planes,
    and in between expert e has its second plane exactly when e < n_hot;
    each expert's W_hat is also re-derived from the planes' exact rationals
    on one row."""
    rng = np.random.default_rng(105)
    E, N, K, G = 4, 3, 128, 64
    W = (rng.standard_normal((E * N, K)) * 0.02).astype(np.float32)
    (c1, s1), (c2, s2) = oracle.two_plane(W, G)
    for n_hot in range(E + 1):
        w_of = oracle.hot_prefix_weights(K, G, N, n_hot, c1, s1, c2[:n_hot * N], s2[:n_hot * N])
        for e in range(E):
            r = slice(e * N, (e + 1) * N)
            one = oracle.ternary_weights(K, G, c1[r], s1[r])
            two = oracle.ternary_weights(K, G, c1[r], s1[r], c2[r], s2[r])
            assert np.array_equal(w_of(e), two if e < n_hot else one)
    # one row by hand: trits times the fp16 scales, summed as fractions
    w_of = oracle.hot_prefix_weights(K, G, N, 1, c1, s1, c2[:N], s2[:N])
    t1 = oracle.unpack(c1[:1], np.full_like(s1[:1], 0x3c00), K, G)   # scale 1.0: the trits
    t2 = oracle.unpack(c2[:1], np.full_like(s2[:1], 0x3c00), K, G)
    sc1 = oracle.f16_bits_to_f64(s1[0])
    sc2 = oracle.f16_bits_to_f64(s2[0])
    for k in range(K):
        g = k // G
        exact = Fraction(float(t1[0, k])) * Fraction(float(sc1[g])) + \
            Fraction(float(t2[0, k])) * Fraction(float(sc2[g]))
        assert Fraction(float(w_of(0)[0, k])) == exact


# ------------------------------------------- Route B sections 8.1 and 8.3

def _pack7_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "routeb_pack7_example.txt")
    cases = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            left, right = line.split(":")
            nums = [int(v) for v in left.split()]
            K, idx = nums[0], nums[1:]
            assert len(idx) == K
            cases.append((K, idx, [int(v, 16) for v in right.split()]))
    return cases


def test_pack7_worked_example():
    """Section 8.1: 7-bit indices, packed bytes worked out by hand."""
    cases = _pack7_golden()
    assert len(cases) == 4
    for K, idx, want in cases:
        got = oracle.pack7(np.array([idx], np.uint8))
        assert got.shape == (1, -(-7 * K // 8))
        assert list(got[0]) == want
        assert list(oracle.unpack7(got, K)[0]) == idx


def test_pack7_single_bits():
    """One set bit q of index k lands on stream bit 7k + q, i.e. byte
    (7k+q) // 8, bit (7k+q) % 8; every other bit is zero."""
    for K in (1, 7, 8, 9, 33):
        for k in range(K):
            for q in range(7):
                idx = np.zeros((1, K), np.uint8)
                idx[0, k] = 1 << q
                got = oracle.pack7(idx)[0]
                p = 7 * k + q
                want = np.zeros(-(-7 * K // 8), np.uint8)
                want[p // 8] = 1 << (p % 8)
                assert np.array_equal(got, want), (K, k, q)


def test_pack7_round_trip_and_padding():
    rng = np.random.default_rng(81)
    for K in (1, 5, 8, 64, 100, 1024):
        idx = rng.integers(0, 128, (3, K), dtype=np.uint8)
        packed = oracle.pack7(idx)
        assert packed.shape == (3, -(-7 * K // 8))
        assert np.array_equal(oracle.unpack7(packed, K), idx)
        ones = oracle.pack7(np.full((1, K), 127, np.uint8))[0]
        bits = np.unpackbits(ones, bitorder="little")
        assert bits[:7 * K].all() and not bits[7 * K:].any()
    with pytest.raises(ValueError):
        oracle.pack7(np.array([[128]], np.uint8))


def test_truncate_alphabet():
    """Section 8.1: the used codes in increasing order, used[index] == codes,
    the list padded with the all-zero word 121, at most 128 codes."""
    rng = np.random.default_rng(82)
    alphabet = np.sort(rng.choice(243, 45, replace=False)).astype(np.uint8)
    codes = alphabet[rng.integers(0, 45, (40, 70))]
    codes[0, :45] = alphabet                        # every letter occurs
    used, n_used, index = oracle.rb_truncate(codes)
    assert n_used == 45
    assert np.array_equal(used[:45], alphabet)
    assert (used[45:] == 121).all()
    assert np.array_equal(used[index], codes)
    assert int(index.max()) == 44
    # one code; an empty matrix; all 128; too many; a non-code byte
    u1, n1, i1 = oracle.rb_truncate(np.full((2, 3), 200, np.uint8))
    assert n1 == 1 and u1[0] == 200 and (i1 == 0).all()
    u0, n0, _ = oracle.rb_truncate(np.zeros((0, 4), np.uint8))
    assert n0 == 0 and (u0 == 121).all()
    c128 = np.arange(115, 243).astype(np.uint8)[None, :]
    u, n, i = oracle.rb_truncate(c128)
    assert n == 128 and np.array_equal(u, c128[0]) and np.array_equal(i[0], np.arange(128))
    with pytest.raises(ValueError):
        oracle.rb_truncate(np.arange(114, 243).astype(np.uint8)[None, :])
    with pytest.raises(ValueError):
        oracle.rb_truncate(np.array([[3, 250]], np.uint8))


def test_rb_weights7_decodes_through_used_codes():
    """The 7-bit form decodes to the same weights as the code bytes, and an
    index past n_used (code 121) is a zero weight for any ladder."""
    rng = np.random.default_rng(83)
    lad = workloads_ladder(rng)
    T = oracle.rb_table(lad)
    assert T[121] == 0.0
    codes = rng.choice(np.array([3, 40, 121, 150, 202, 242], np.uint8), (6, 50))
    used, n_used, index = oracle.rb_truncate(codes)
    packed = oracle.pack7(index)
    rho = np.array([0.5, 1.0, 1.25, 0.75, 1.5, 2.0], np.float16).view(np.uint16)
    assert np.array_equal(oracle.rb_weights7(packed, 50, used, T, np.float32(0.02), rho),
                          oracle.rb_weights(codes, T, np.float32(0.02), rho))
    pad = np.full((1, 8), 100, np.uint8)             # index 100 >= n_used
    assert (oracle.rb_weights7(oracle.pack7(pad), 8, used, T, np.float32(1)) == 0).all()


def workloads_ladder(rng):
    u = rng.uniform(0.8, 1.2, 5).astype(np.float32)
    return (np.float32(0.5) ** np.arange(5, dtype=np.float32) * u).astype(np.float32)


def test_block_tables_closed_form():
    """Section 8.3: rows of block h read code book h.  Under the integer
    ladder (81, 27, 9, 3, 1) scaled by 2^h, T_h[b] = 2^h (b - 121) exactly,
    so every weight is alpha 2^(n // 32) (code - 121); a ragged last block
    works; equal tables reduce to the one-table call; swapping two blocks of
    rows together with their tables swaps the rows."""
    base = np.array([81, 27, 9, 3, 1], np.float32)
    N, K, b = 70, 9, 32                                  # blocks of 32, 32, 6 rows
    nb = 3
    tables = np.stack([oracle.rb_table(base * np.float32(2.0 ** h)) for h in range(nb)])
    for h in range(nb):
        assert np.array_equal(tables[h], (2.0 ** h * (np.arange(243) - 121)).astype(np.float32))
    rng = np.random.default_rng(84)
    codes = rng.integers(0, 243, (N, K), dtype=np.uint8)
    alpha = np.float32(0.375)
    w = oracle.rb_weights(codes, tables, alpha, table_rows=b)
    want = 0.375 * 2.0 ** (np.arange(N) // b)[:, None] * (codes.astype(np.float64) - 121)
    assert np.array_equal(w, want)
    same = np.stack([tables[1]] * nb)
    assert np.array_equal(oracle.rb_weights(codes, same, alpha, table_rows=b),
                          oracle.rb_weights(codes, tables[1], alpha))
    perm = np.r_[np.arange(32, 64), np.arange(0, 32), np.arange(64, 70)]
    w_sw = oracle.rb_weights(codes[perm], tables[[1, 0, 2]], alpha, table_rows=b)
    assert np.array_equal(w_sw, w[perm])
    with pytest.raises(ValueError):
        oracle.rb_weights(codes, tables[:2], alpha, table_rows=b)
