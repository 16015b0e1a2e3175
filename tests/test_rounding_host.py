"""Rounding identities the kernels rely on (host arithmetic, numpy).

The assembly kernel's bf16 keys: rounding an fp64 value to fp32 and then to bf16, both to
nearest even, gives the bf16 nearest to the fp64 value whenever the fp32
result is not exactly halfway between two bf16 values.  The kernel takes the
two hardware conversions except in that case, where it rounds once from the
fp64 bits.  Checked against an exact one-step rounding on random values over
a wide exponent range and on values placed within a few fp32 ulps of bf16
midpoints (where double rounding goes wrong when the midpoint case is not
set aside).

The band projection's folded data: the fp32 sum or difference u of two bf16
values splits exactly into hi = fp16(u) (to nearest even) and lo = fp16(u -
hi), apart from a remainder below fp16's normal range (rounded by at most
2^-25), with |lo| <= 2^-11 |u|; |u| >= 65520 gives an infinite hi.

The band projection's radix-4 form (transform lengths divisible by 128): bin
j of an nf-point transform from the four quarter sums y0, y2, a, b over nf/4
columns, with the tile mechanics the kernel uses (bins grouped by j mod 4, the
b products of classes 1 and 3 reading the tile's rows swapped, half of them
negated), checked against the transform's definition; and the fp16 hi + lo
pair of a four-term fp32 sum within 2^-22 of the sum plus the fp32 rounding
of its partial sums."""
import numpy as np


def _bf16_nearest_even(d):
    """bf16 bits of float64 values, one rounding: 8 significant bits by
    rint on the scaled significand (exact in fp64), normal range only."""
    m, e = np.frexp(d)
    v = np.ldexp(np.rint(m * 256.0) / 256.0, e)
    return v.astype(np.float32).view(np.uint32) >> 16


def _two_step(d):
    u = d.astype(np.float32).view(np.uint32)
    mid = (u & 0xFFFF) == 0x8000
    return (u + 0x7FFF + ((u >> 16) & 1)) >> 16, mid


def test_double_rounding_is_single_rounding_off_midpoints():
    rng = np.random.default_rng(5)
    n = 400_000
    d = rng.standard_normal(n) * np.exp(rng.uniform(-30, 30, n))
    mp = (rng.integers(0x3000, 0x4F00, n).astype(np.uint32) << 16 | 0x8000).view(np.float32).astype(np.float64)
    mp *= (1 + rng.integers(-40, 41, n) * 2.0 ** -33) * np.where(rng.random(n) < 0.5, -1, 1)
    d = np.concatenate([d, mp])
    want = _bf16_nearest_even(d)
    got, mid = _two_step(d)
    assert mid.sum() > 1000  # the constructed values do reach the midpoint case
    assert np.array_equal(got[~mid], want[~mid])
    # and the case set aside is real: some midpoint results do round differently
    assert (got[mid] != want[mid]).any()


def _bf16(x):
    """float32 values rounded to bf16 (nearest even), as float32."""
    u = x.astype(np.float32).view(np.uint32)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)


def test_fold_split_is_exact():
    rng = np.random.default_rng(11)
    n = 600_000
    # operands over a wide range of exponent gaps and both signs, up to the
    # fp16 limit; a quarter of the pairs within 2 binades of each other
    ea = rng.uniform(-20, 15.9, n)
    eb = np.where(rng.random(n) < 0.25, ea + rng.uniform(-2, 2, n), rng.uniform(-30, 15.9, n))
    a = _bf16(np.exp2(ea) * rng.choice([-1.0, 1.0], n) * rng.uniform(1, 2, n) / 2)
    b = _bf16(np.exp2(np.minimum(eb, 15.9)) * rng.choice([-1.0, 1.0], n) * rng.uniform(1, 2, n) / 2)
    for u in (a + b, a - b):  # float32 arithmetic, nearest even, as on the GPU
        with np.errstate(over="ignore"):
            hi = u.astype(np.float16)
        fin = np.abs(u) < 65520
        assert np.isinf(hi[~fin]).all() and np.isfinite(hi[fin]).all()
        u, hi = u[fin], hi[fin]
        r = u - hi.astype(np.float32)          # exact in fp32
        lo = r.astype(np.float16)
        err = np.abs(hi.astype(np.float64) + lo.astype(np.float64) - u.astype(np.float64))
        normal = (r == 0) | (np.abs(r) >= 2.0 ** -14)
        assert (err[normal] == 0).all()
        assert (err[~normal] <= 2.0 ** -25).all()
        assert (np.abs(lo.astype(np.float64)) <= 2.0 ** -11 * np.abs(u.astype(np.float64))).all()
        # the split is not trivial: remainders of both signs occur in the normal range
        assert ((r > 0) & normal & (u > 0)).sum() > 1000 and ((r < 0) & normal & (u > 0)).sum() > 1000


def _radix4_tiles(x, b0, kk):
    """Cosine and sine sums of bins b0 .. b0 + 63 (< kk) as the radix-4 band
    kernel forms them: four 32-row tiles, one per class k = j mod 4, rows
    i < 16 the cosine rows of bins b0 + 4i + k and rows 16 + i their sine
    rows, against the quarter sums over the first nf/4 columns."""
    nf = x.size
    M = nf // 4
    xq = x.reshape(4, M)
    terms = {"y0": (xq[0] + xq[2]) + (xq[1] + xq[3]), "y2": (xq[0] + xq[2]) - (xq[1] + xq[3]),
             "a": xq[0] - xq[2], "b": xq[1] - xq[3]}
    m = np.arange(M)
    R, S = {}, {}
    for k in range(4):
        i = np.arange(32)
        bins = b0 + 4 * (i & 15) + k
        ang = 2 * np.pi * np.outer(bins, m) / nf
        tile = np.where((i < 16)[:, None], np.cos(ang), np.sin(ang))
        tile[bins >= kk] = 0.0
        if k in (0, 2):
            acc = tile @ terms["y0" if k == 0 else "y2"]
        else:
            neg = (i < 16) if k == 1 else (i >= 16)
            swapped = tile[i ^ 16] * np.where(neg, -1.0, 1.0)[:, None]
            acc = tile @ terms["a"] + swapped @ terms["b"]
        for r in range(32):
            if bins[r] < kk:
                (R if r < 16 else S)[int(bins[r])] = acc[r]
    return R, S


def test_radix4_classes_give_the_dft():
    rng = np.random.default_rng(21)
    for nf, kk in ((256, 128), (512, 70), (128, 64)):
        x = rng.standard_normal(nf)
        n = np.arange(nf)
        for b0 in range(0, kk, 64):
            R, S = _radix4_tiles(x, b0, kk)
            assert sorted(R) == sorted(S) == list(range(b0, min(b0 + 64, kk)))
            for j in R:
                ang = 2 * np.pi * j * n / nf
                np.testing.assert_allclose(R[j], np.dot(np.cos(ang), x), atol=1e-9)
                np.testing.assert_allclose(S[j], np.dot(np.sin(ang), x), atol=1e-9)


def test_radix4_sum_split_bound():
    rng = np.random.default_rng(23)
    n = 400_000
    e = rng.uniform(-24, 13, (4, n))
    e = np.where(rng.random((4, n)) < 0.3, e[0] + rng.uniform(-1, 1, (4, n)), e)
    x = _bf16(np.exp2(e) * rng.choice([-1.0, 1.0], (4, n)) * rng.uniform(1, 2, (4, n)) / 2)
    exact = {"y0": (x[0].astype(np.float64) + x[2] + x[1] + x[3]),
             "y2": (x[0].astype(np.float64) + x[2] - x[1] - x[3])}
    s02, s13 = x[0] + x[2], x[1] + x[3]     # float32, as on the GPU
    for name, s in (("y0", s02 + s13), ("y2", s02 - s13)):
        with np.errstate(over="ignore"):
            hi = s.astype(np.float16)
        fin = np.abs(s) < 65520
        assert np.isfinite(hi[fin]).all() and np.isinf(hi[~fin]).all()
        r = s[fin] - hi[fin].astype(np.float32)  # exact in fp32
        lo = r.astype(np.float16)
        got = hi[fin].astype(np.float64) + lo.astype(np.float64)
        want = exact[name][fin]
        mag = np.abs(x[:, fin].astype(np.float64)).sum(axis=0)
        bound = 2.0 ** -22 * np.abs(want) + 2.0 ** -23 * mag + 2.0 ** -25
        assert (np.abs(got - want) <= bound).all()
