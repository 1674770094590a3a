"""The software 2^x behind fa_fwd_exp2_emulated (csrc/fa_exp2.h with the
coefficients of csrc/fa_exp2_coef.h, fitted by exact_attention_07_amd/exp2_fit.py),
checked on the CPU against the exponential it replaces.

"FlashAttention-4震撼发布：性能再攀新高", second algorithmic improvement:
part of the exponentials are computed by a polynomial on the FMA units.
The pins: the committed header is what the fit produces; the fit is the
minimax one (its error equioscillates at degree + 2 points with one
magnitude, the characterisation of a best uniform approximation); the
device routine, emulated step by step in fp32, stays within that error plus
fp32 rounding everywhere it is used, and maps masked scores to exactly 0.
"""
import math

import numpy as np

from exact_attention_07_amd import exp2_fit

FIT_ERR = 7.5e-5        # largest relative error of the cubic on [0, 1]


def test_header_matches_the_fit():
    assert exp2_fit.main(["--check"]) == 0


def test_fit_equioscillates():
    c, e = exp2_fit.remez()
    assert e < FIT_ERR
    f = np.linspace(0.0, 1.0, 200001)
    r = exp2_fit._rel_err(c, f)
    # the largest error is the levelled one (to the grid's resolution)
    assert abs(np.abs(r).max() - e) <= 1e-3 * e
    # degree + 2 = 5 alternating extrema of magnitude e: the endpoints and
    # three interior points
    sign = np.sign(r)
    runs = np.split(np.arange(f.size), np.nonzero(np.diff(sign))[0] + 1)
    ext = [run[np.argmax(np.abs(r[run]))] for run in runs]
    assert len(ext) == exp2_fit.DEGREE + 2
    for i in ext:
        assert abs(abs(r[i]) - e) <= 1e-3 * e
    signs = np.sign(r[ext])
    assert (signs[1:] == -signs[:-1]).all()
    assert ext[0] == 0 and ext[-1] == f.size - 1


def test_lower_degree_does_worse():
    # the cubic is the lowest degree that gets below 1e-4 (the bf16 rounding
    # of P is 2^-9 ~ 2e-3, the LSE bar 1e-3)
    _, e2 = exp2_fit.remez(degree=2)
    assert e2 > 1e-3


def _fma32(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(np.float32)


def device_exp2(x):
    """fa_exp2.h's exp2_poly step by step in fp32."""
    c0, c1, c2, c3 = (np.float32(v) for v in exp2_fit.read_header())
    x = np.fmax(np.asarray(x, np.float32), np.float32(-200.0))
    n = np.floor(x)
    f = (x - n).astype(np.float32)
    p = _fma32(c3, f, c2)
    p = _fma32(p, f, c1)
    p = _fma32(p, f, c0)
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)


def test_device_routine_relative_error():
    rng = np.random.default_rng(3)
    xs = np.concatenate([np.linspace(-126.0, 9.0, 400001), np.arange(-126, 10).astype(np.float64),
                         np.arange(-126, 10) - 2.0 ** -20, rng.uniform(-30, 9, 100000)]).astype(np.float32)
    got = device_exp2(xs).astype(np.float64)
    ref = np.exp2(xs.astype(np.float64))
    rel = np.abs(got / ref - 1.0)
    # the fit's error, plus the rounding of three FMAs and of f (a few 2^-24)
    assert rel.max() <= FIT_ERR + 8 * 2.0 ** -24, rel.max()


def test_masked_and_tiny_arguments_give_zero():
    out = device_exp2(np.array([-np.inf, np.nan, -200.0, -1e30, -151.0], np.float32))
    assert (out == 0.0).all() and not np.signbit(out).any()
    # just above the underflow the result is a positive subnormal, never 0
    assert device_exp2(np.array([-140.0], np.float32))[0] > 0


def test_probabilities_of_the_fast_path():
    # the kernel's arguments are at most tau = 8 above the reference: 2^8
    # within the fit's error, far below bf16's and e4m3's largest values
    v = float(device_exp2(np.array([8.0], np.float32))[0])
    assert abs(v / 256.0 - 1.0) <= FIT_ERR + 2.0 ** -22
    assert math.isfinite(v)
