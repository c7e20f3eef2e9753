"""Writes tests/golden/gelu_table.txt: GELU(v) = v * Phi(v) at a few points,
Phi the standard normal CDF, to 20 significant digits.

Phi is summed here from its Maclaurin series in 80-digit decimal arithmetic,
independently of any libm erf / erfc (the oracle's GELU uses the C library's
erfc in double precision, which the table pins):
    Phi(v) = 1/2 + (1 / sqrt(2 pi)) * sum_{n >= 0} (-1)^n v^(2n+1) / (2^n n! (2n+1))
(term-by-term integration of the normal density's exponential series).  pi
comes from Machin's formula, pi = 16 atan(1/5) - 4 atan(1/239).  The series
converges for every v; at 80 digits the cancellation between its terms leaves
well over 40 correct digits for |v| <= 6.  Where mpmath is importable its
ncdf is asked for the same values as a second, separate check.

GELU is not on the pages; it is the activation between the two linears of
the DiT MLP workloads.

Run from the repository root:  python tests/golden/make_gelu_table.py
"""
import os
from decimal import Decimal, getcontext

getcontext().prec = 80

POINTS = ["0", "0.25", "0.5", "1", "1.5", "2", "2.5", "3", "4", "5",
          "-0.25", "-0.5", "-1", "-1.5", "-2", "-2.5", "-3", "-4", "-5", "-6"]


def atan_inv(k: int) -> Decimal:
    """atan(1/k) from its series sum (-1)^n / ((2n+1) k^(2n+1))."""
    x = Decimal(1) / k
    x2 = x * x
    term, total, n = x, Decimal(0), 0
    eps = Decimal(10) ** -(getcontext().prec + 2)
    while abs(term) > eps:
        total += term / (2 * n + 1) if n % 2 == 0 else -term / (2 * n + 1)
        term *= x2
        n += 1
    return total


def phi(v: Decimal, pi: Decimal) -> Decimal:
    v2 = v * v
    term = v            # v^(2n+1) / (2^n n!) for n = 0
    total, n = Decimal(0), 0
    eps = Decimal(10) ** -(getcontext().prec + 2)
    while n < 10 or abs(term) > eps:
        total += term / (2 * n + 1) if n % 2 == 0 else -term / (2 * n + 1)
        n += 1
        term = term * v2 / (2 * n)
    return Decimal("0.5") + total / (2 * pi).sqrt()


def main():
    pi = 16 * atan_inv(5) - 4 * atan_inv(239)
    try:
        import mpmath
        mpmath.mp.dps = 40
    except ImportError:
        mpmath = None
    lines = ["# GELU(v) = v * Phi(v), Phi = standard normal CDF, 20 significant digits.",
             "# Written by tests/golden/make_gelu_table.py: Phi summed from its Maclaurin",
             "# series in 80-digit decimal arithmetic (no libm erf/erfc involved).",
             "# GELU is not on the pages; it is the activation between the MLP layers of",
             "# the DiT workloads.",
             "# columns: v  Phi(v)  gelu(v)"]
    for p in POINTS:
        v = Decimal(p)
        ph = phi(v, pi)
        if mpmath is not None:
            ref = Decimal(str(mpmath.ncdf(mpmath.mpf(p))))
            assert abs(ph - ref) <= abs(ref) * Decimal("1e-35"), (p, ph, ref)
        g = v * ph
        gs = "0" if g == 0 else f"{g:.19E}"
        lines.append(f"{p:>5}  {ph:.19E}  {gs}")
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gelu_table.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


if __name__ == "__main__":
    main()
