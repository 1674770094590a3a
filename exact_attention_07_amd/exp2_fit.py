"""Coefficients of the software 2^x used by fa_fwd_exp2_emulated.

    python -m exact_attention_07_amd.exp2_fit          # rewrite csrc/fa_exp2_coef.h
    python -m exact_attention_07_amd.exp2_fit --check  # compare with the header

"FlashAttention-4震撼发布：性能再攀新高", second algorithmic improvement: part
of the exponentials are computed with a polynomial on the FMA units instead of
the hardware exponential unit.  Here 2^x is reduced to x = n + f with
n = floor(x), f in [0, 1), 2^x = 2^n * 2^f, and 2^f is approximated by the
cubic p(f) = c0 + c1 f + c2 f^2 + c3 f^3 whose largest relative error
|p(f) / 2^f - 1| over [0, 1] is smallest (minimax, found by the Remez
exchange below).  The coefficients are rounded to fp32 and written as a C
header; fa_exp2.h evaluates p by Horner's rule with fused multiply-adds.

Build tooling: plain numpy in fp64, no GPU.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

DEGREE = 3
HEADER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "fa_exp2_coef.h")


def _rel_err(c, f):
    return np.polynomial.polynomial.polyval(f, c) / np.exp2(f) - 1.0


def remez(degree: int = DEGREE, iters: int = 30, grid: int = 20001):
    """Minimax (relative error) polynomial of the given degree for 2^f on
    [0, 1]: returns (coefficients, lowest first, and the levelled error E)."""
    n = degree + 2
    # start from Chebyshev extrema mapped to [0, 1]
    x = 0.5 - 0.5 * np.cos(np.pi * np.arange(n) / (n - 1))
    dense = np.linspace(0.0, 1.0, grid)
    c, e = None, None
    for _ in range(iters):
        # p(x_i) - 2^x_i = (-1)^i E 2^x_i  for the n reference points
        a = np.zeros((n, n))
        for j in range(degree + 1):
            a[:, j] = x ** j
        a[:, -1] = -((-1.0) ** np.arange(n)) * np.exp2(x)
        sol = np.linalg.solve(a, np.exp2(x))
        c, e = sol[:-1], sol[-1]
        # new reference: the extrema of the error, one per sign run
        r = _rel_err(c, dense)
        sign = np.sign(r)
        sign[sign == 0] = 1
        runs = np.split(np.arange(grid), np.nonzero(np.diff(sign))[0] + 1)
        ext = np.array([run[np.argmax(np.abs(r[run]))] for run in runs])
        if ext.size != n:
            break
        new_x = dense[ext]
        if np.allclose(new_x, x, atol=1e-12):
            break
        x = new_x
    return c, abs(e)


def fp32_coefficients():
    c, e = remez()
    return [float(np.float32(v)) for v in c], float(e)


def header_text(coef, err) -> str:
    lines = ["// fa_exp2_coef.h -- coefficients of p(f) ~ 2^f on [0, 1), lowest first,",
             "// minimax in the relative error (Remez exchange, degree 3), rounded to",
             f"// fp32; levelled relative error of the exact-coefficient fit {err:.3e}.",
             "// Written by exact_attention_07_amd/exp2_fit.py; do not edit.",
             "#pragma once"]
    for i, v in enumerate(coef):
        lines.append(f"#define FA_EXP2_C{i} {float(np.float32(v)).hex()}f  /* {v!r} */")
    return "\n".join(lines) + "\n"


def read_header(path: str = HEADER):
    coef = {}
    for line in open(path):
        if line.startswith("#define FA_EXP2_C"):
            _, name, val = line.split()[:3]
            coef[int(name[len("FA_EXP2_C"):])] = float.fromhex(val.rstrip("f"))
    return [coef[i] for i in range(len(coef))]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--check", action="store_true")
    a = ap.parse_args(argv)
    coef, err = fp32_coefficients()
    if a.check:
        ok = read_header() == coef
        print("header matches the fit" if ok else "header differs from the fit")
        return 0 if ok else 1
    with open(HEADER, "w") as f:
        f.write(header_text(coef, err))
    print(HEADER, coef, err)
    return 0


if __name__ == "__main__":
    sys.exit(main())
