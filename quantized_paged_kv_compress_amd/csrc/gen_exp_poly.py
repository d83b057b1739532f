"""Constants of the float64 exponential in kvq_device.hpp (exp_f64), reproducible.

    python quantized_paged_kv_compress_amd/csrc/gen_exp_poly.py

exp(d) = 2^k * exp(r) with k = rint(d / ln 2) and r = d - k ln 2, reduced in two steps
(Cody and Waite): ln 2 = LN2_HI + LN2_LO where LN2_HI keeps 32 significant bits, so
k * LN2_HI is exact for |k| < 2^21 and d - k * LN2_HI is exact as well.  exp(r) on
|r| <= ln(2)/2 (+ margin) is a degree-11 polynomial: the Chebyshev interpolant of exp on
[-0.35, 0.35], converted to monomial coefficients in 60-digit arithmetic and rounded to
float64.  Its error against exp is printed (relative, in units of 2^-53).
"""
import mpmath as mp

mp.mp.dps = 60
A = mp.mpf("0.35")
DEG = 11


def ln2_split():
    ln2 = mp.log(2)
    m, e = mp.frexp(ln2)                   # ln2 = m * 2^e, m in [0.5, 1)
    hi = mp.floor(m * 2 ** 32) / 2 ** 32 * mp.mpf(2) ** e
    lo = ln2 - hi
    return float(hi), float(lo)


def cheb_monomial():
    n = DEG + 1
    nodes = [A * mp.cos(mp.pi * (k + mp.mpf(1) / 2) / n) for k in range(n)]
    V = mp.matrix([[x ** j for j in range(n)] for x in nodes])
    y = mp.matrix([mp.exp(x) for x in nodes])
    c = mp.lu_solve(V, y)
    return [c[j] for j in range(n)]


def main():
    hi, lo = ln2_split()
    coef = cheb_monomial()
    cf = [float(c) for c in coef]
    worst = mp.mpf(0)
    for i in range(2001):
        r = -A + 2 * A * i / 2000
        p = mp.mpf(0)
        for c in reversed(cf):
            p = p * r + mp.mpf(c)
        worst = max(worst, abs(p / mp.exp(r) - 1))
    print(f"LN2_HI = {hi!r}  ({hi.hex()})")
    print(f"LN2_LO = {lo!r}  ({lo.hex()})")
    print(f"INV_LN2 = {float(1 / mp.log(2))!r}")
    for j, c in enumerate(cf):
        print(f"c{j} = {c.hex()}  // {c!r}")
    print(f"max relative error of the rounded polynomial on [-{A}, {A}]: "
          f"{mp.nstr(worst, 3)} = {mp.nstr(worst * 2 ** 53, 3)} x 2^-53")


if __name__ == "__main__":
    main()
