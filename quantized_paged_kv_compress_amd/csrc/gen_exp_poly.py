"""Constants of the float64 exponentials in kvq_device.hpp, reproducible.

    python quantized_paged_kv_compress_amd/csrc/gen_exp_poly.py          # exp_f64
    python quantized_paged_kv_compress_amd/csrc/gen_exp_poly.py --table  # exp_tab

exp_f64: exp(d) = 2^k * exp(r) with k = rint(d / ln 2) and r = d - k ln 2, reduced in
two steps (Cody and Waite): ln 2 = LN2_HI + LN2_LO where LN2_HI keeps 32 significant
bits, so k * LN2_HI is exact for |k| < 2^21.  exp(r) on |r| <= ln(2)/2 (+ margin) is a
degree-11 polynomial: the Chebyshev interpolant of exp on [-0.35, 0.35], converted to
monomial coefficients in 60-digit arithmetic and rounded to float64.

exp_tab: exp(d) = 2^(k >> 8) * 2^((k & 255) / 256) * exp(r) with k = rint(256 d / ln 2)
and r = d - k ln(2)/256 (|r| <= ln(2)/512), ln(2)/256 split with 33 significant bits in
the high part (k * hi exact for |k| < 2^20); 2^(j/256) comes from a 256-entry table of
correctly rounded float64 values and exp(r) - 1 from its Taylor terms up to r^4.
"""
import sys

import mpmath as mp

mp.mp.dps = 60


def split(c, bits):
    m, e = mp.frexp(c)
    hi = mp.floor(m * 2 ** bits) / 2 ** bits * mp.mpf(2) ** e
    return float(hi), float(c - hi)


def cheb_monomial(a, deg):
    n = deg + 1
    nodes = [a * mp.cos(mp.pi * (k + mp.mpf(1) / 2) / n) for k in range(n)]
    V = mp.matrix([[x ** j for j in range(n)] for x in nodes])
    y = mp.matrix([mp.exp(x) for x in nodes])
    c = mp.lu_solve(V, y)
    return [c[j] for j in range(n)]


def poly_constants():
    a = mp.mpf("0.35")
    hi, lo = split(mp.log(2), 32)
    cf = [float(c) for c in cheb_monomial(a, 11)]
    worst = mp.mpf(0)
    for i in range(2001):
        r = -a + 2 * a * i / 2000
        p = mp.mpf(0)
        for c in reversed(cf):
            p = p * r + mp.mpf(c)
        worst = max(worst, abs(p / mp.exp(r) - 1))
    return hi, lo, float(1 / mp.log(2)), cf, worst


def table_constants():
    tab = [float(mp.mpf(2) ** (mp.mpf(j) / 256)) for j in range(256)]
    hi, lo = split(mp.log(2) / 256, 33)
    tail = (mp.log(2) / 512) ** 5 / 120
    return tab, hi, lo, float(256 / mp.log(2)), tail


def main():
    if "--table" in sys.argv:
        tab, hi, lo, inv, tail = table_constants()
        print(f"256/ln2 = {inv.hex()}  ln2/256 hi = {hi.hex()}  lo = {lo.hex()}  "
              f"first dropped Taylor term {mp.nstr(tail, 3)}")
        for j in range(0, 256, 4):
            print("    " + ", ".join(t.hex() for t in tab[j:j + 4]) + ",")
        return
    hi, lo, inv, cf, worst = poly_constants()
    print(f"LN2_HI = {hi!r}  ({hi.hex()})")
    print(f"LN2_LO = {lo!r}  ({lo.hex()})")
    print(f"INV_LN2 = {inv!r}")
    for j, c in enumerate(cf):
        print(f"c{j} = {c.hex()}  // {c!r}")
    print(f"max relative error of the rounded polynomial on [-0.35, 0.35]: "
          f"{mp.nstr(worst, 3)} = {mp.nstr(worst * 2 ** 53, 3)} x 2^-53")


if __name__ == "__main__":
    main()
