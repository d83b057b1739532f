"""Soundness of the error bound that lets the ratio-2 and ratio-4 compressors keep a
float32 pooled value (CPU, no GPU).

The short-window kernel pools each channel in float32 with the hardware exp2 and
reciprocal, computes a bound E on the distance between its float32 result and the exact
softmax pool, and keeps the float32 result only where the bf16 rounding midpoint next to
it lies farther away than E (otherwise the channel is recomputed in float64).  If E were
too small, a kept value could round to the wrong bf16, an event so rare that random GPU
inputs would not show it.  This test replays the kernel's float32 sequence on the CPU
with the hardware's error allowances spent adversarially:
  - exp2: any float32 within 0.7827 ulp of 2^a (the largest error measured on gfx950 over
    every input in [-160, 1]), chosen to push the pooled value up, or down;
  - reciprocal: any float32 within 1 ulp of 1/l, chosen the same way (0.8818 ulp measured);
(both allowances are re-measured on the GPU under test by tests/test_gpu_hw_bounds.py)
and checks, on hard windows (huge score offsets, cancellation, wide spreads, values
placed next to bf16 midpoints), that wherever the kernel would keep its float32 value,
that value is within E of the exact pool (evaluated in 64-bit-mantissa long double) and
rounds to the same bf16.
"""
import numpy as np
import pytest

F32, LD = np.float32, np.longdouble
L32 = F32(1.4426950408889634)          # fl32(log2 e), the kernel's constant
U = 2.0 ** -24
EXP2_ULP = 0.7827
RCP_ULP = 1.0


def fma32(a, b, c):
    """fl32(a * b + c) with one rounding (the product is exact in long double)."""
    return (LD(a) * LD(b) + LD(c)).astype(F32)


def ulp32(v):
    """Spacing of float32 at |v| (normal range)."""
    return np.spacing(np.abs(v).astype(F32)).astype(LD)


def adversarial(exact, max_ulps, up):
    """The float32 farthest from `exact` (long double, positive) in direction `up` (bool
    array) that is still within max_ulps (<= 1) ulp of it: the grid value above exact if
    that one is close enough, else the one below (and the other way round for down)."""
    near = exact.astype(F32)
    lo = np.where(near.astype(LD) > exact, np.nextafter(near, F32(0)), near)          # grid value <= exact
    hi = np.where(lo.astype(LD) < exact, np.nextafter(lo, F32(np.inf)), lo)            # grid value >= exact
    u = ulp32(lo)
    best_up = np.where(hi.astype(LD) - exact <= max_ulps * u, hi, lo)
    best_dn = np.where(exact - lo.astype(LD) <= max_ulps * u, lo, hi)
    return np.where(up, best_up, best_dn)


def bf16_rne(v32):
    b = v32.astype(F32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint32)


def bf16_rne_exact(p):
    """bf16 bits of the long double p (|p| in the normal range), rounded to nearest even:
    the nearest of the three bf16 values around fl32(p), ties to the even one."""
    b = (p.astype(F32).view(np.uint32) & 0xFFFF0000).astype(np.int64)
    cands = np.stack([b - 0x10000, b, b + 0x10000]) & 0xFFFFFFFF
    vals = cands.astype(np.uint32).view(F32).astype(LD)
    d = np.abs(vals - p[None, :])
    best = d.min(axis=0)
    tied = d == best[None, :]
    even = ((cands >> 16) & 1) == 0
    pick = np.where((tied & even).any(axis=0), np.argmax(tied & even, axis=0), np.argmax(tied, axis=0))
    return (cands[pick, np.arange(p.size)] >> 16).astype(np.uint32)


def kernel_pool(s, x, up, p, shrink=1.0):
    """The kernel's float32 sequence for windows s, x [N, r] (float32); returns pc, E and
    the keep mask.  `up` [N] picks the direction of every adversarial rounding and p is
    the exact pool (rows whose kv lies above it get their weight pushed that way).  shrink
    scales the bound (1 in the kernel; the test's own check uses a smaller one)."""
    N, r = s.shape
    m = s.max(axis=1)
    mL = (m * L32).astype(F32)
    a = np.stack([fma32(s[:, j], np.full(N, L32), -mL) for j in range(r)], axis=1)
    exact_w = np.exp2(a.astype(LD))
    # push every weight whose kv lies above the pooled value up (or down), the others the
    # other way: that maximises the error of the weighted mean in direction `up`
    w_up = (x.astype(LD) >= p[:, None]) == up[:, None]
    w = adversarial(exact_w, EXP2_ULP, w_up)
    w = np.where(exact_w < 2.0 ** -126, F32(0), w)
    l = np.zeros(N, F32)
    acc = np.zeros(N, F32)
    A = np.zeros(N, F32)
    amin = np.zeros(N, F32)
    for j in range(r):
        l = (l + w[:, j]).astype(F32)
        acc = fma32(w[:, j], x[:, j], acc)
        A = fma32(w[:, j], np.abs(x[:, j]), A)
        amin = np.minimum(amin, a[:, j])
    rl = adversarial(1.0 / l.astype(LD), RCP_ULP, up == (acc >= 0))
    pc = (acc * rl).astype(F32)
    ap = np.abs(pc)
    dw = (F32(2.0 ** -23) + (F32(2.0 ** -23) * np.abs(mL) - amin) * (F32(0.6931472) * F32(1.25) * F32(U))).astype(F32)
    E = (F32(1.01) * ((dw + F32(r * U)) * fma32(ap, l, A) * rl + F32(3.0 * U) * ap)).astype(F32)
    E = (E * F32(shrink)).astype(F32)
    mid = ((pc.view(np.uint32) & 0xFFFF0000) | 0x8000).view(F32)
    keep = ((np.abs(pc - mid) > E) & (E < ap * F32(2.0 ** -10)) & (ap >= F32(2.0 ** -100)) &
            (amin >= F32(-126.0)) & (np.abs(mL) < F32(2.0 ** 20)))
    return pc, E, keep


def exact_pool(s, x):
    sl = s.astype(LD)
    w = np.exp(sl - sl.max(axis=1, keepdims=True))
    return (w * x.astype(LD)).sum(axis=1) / w.sum(axis=1)


def windows(kind, rng, N, r):
    if kind == "normal":
        s = rng.normal(0, 2, (N, r))
        x = rng.normal(0, 1, (N, r))
    elif kind == "offset":                       # large |m|: the mL term of the bound
        s = rng.normal(0, 2, (N, r)) + rng.choice([-1, 1], (N, 1)) * 10.0 ** rng.uniform(2, 5.5, (N, 1))
        x = rng.normal(0, 1, (N, r))
    elif kind == "wide":                         # weights down to 2^-120
        s = rng.uniform(-80, 0, (N, r))
        s[:, 0] = 0
        x = rng.normal(0, 1, (N, r)) * 10.0 ** rng.uniform(-3, 3, (N, r))
    elif kind == "cancel":                       # pooled value far below the kv scale
        s = rng.normal(0, 0.5, (N, r))
        x = rng.normal(0, 1, (N, r))
        x[:, -1] = -(x[:, :-1].sum(axis=1)) * (1 + rng.normal(0, 1e-3, N))
    elif kind == "tiny":                         # values near the bottom of the float32 range
        s = rng.normal(0, 2, (N, r))
        x = rng.normal(0, 1, (N, r)) * 2.0 ** -90
    else:
        raise ValueError(kind)
    return s.astype(F32), x.astype(F32)


def near_midpoint_windows(rng, N, r):
    """Windows whose exact pool lies within a few bound-widths of a bf16 midpoint: shift the
    last kv so that the float64 pool lands on a midpoint plus a small random offset."""
    s, x = windows("normal", rng, N, r)
    p = exact_pool(s, x).astype(np.float64)
    mid = (((np.float32(p).view(np.uint32) & 0xFFFF0000) | 0x8000).view(F32)).astype(np.float64)
    sl = s.astype(np.float64)
    w = np.exp(sl - sl.max(axis=1, keepdims=True))
    wl = w[:, -1] / w.sum(axis=1)
    target = mid * (1 + rng.normal(0, 1, N) * 2.0 ** -20)
    x[:, -1] = (x[:, -1].astype(np.float64) + (target - p) / wl).astype(F32)
    return s, x


@pytest.mark.parametrize("r", [2, 4])
@pytest.mark.parametrize("kind", ["normal", "offset", "wide", "cancel", "tiny", "near_midpoint"])
def test_bound_covers_adversarial_hardware_error(r, kind):
    rng = np.random.default_rng(7 + r * 10 + len(kind))
    N = 20000
    s, x = near_midpoint_windows(rng, N, r) if kind == "near_midpoint" else windows(kind, rng, N, r)
    p = exact_pool(s, x)
    for up in (np.ones(N, bool), np.zeros(N, bool)):
        pc, E, keep = kernel_pool(s, x, up, p)
        err = np.abs(pc.astype(LD) - p)
        assert np.all(err[keep] <= E[keep].astype(LD)), \
            f"{kind}, r {r}: {int((err[keep] > E[keep]).sum())} kept values outside the bound"
        idx = np.flatnonzero(keep)
        sub = idx[rng.permutation(idx.size)[:2000]]   # bf16 check on a sample (pure-Python rounding)
        assert np.array_equal(bf16_rne(pc[sub]), bf16_rne_exact(p[sub])), f"{kind}, r {r}: wrong bf16 kept"
        frac = 1 - keep.mean()
        print(f"[bound] {kind:14s} r {r}: {frac * 100:.3f} % of channels recomputed in float64, "
              f"max err/E {float((err[keep] / E[keep].astype(LD)).max()):.3f}")
    if kind == "near_midpoint":
        assert (~keep).mean() > 0.01, "the midpoint windows must exercise the fallback"


def test_bound_is_not_vacuous():
    """On the workloads' distribution almost every channel keeps its float32 value."""
    rng = np.random.default_rng(3)
    s, x = windows("normal", rng, 50000, 4)
    _, _, keep = kernel_pool(s, x, np.ones(50000, bool), exact_pool(s, x))
    assert keep.mean() > 0.99


def test_check_catches_a_bound_eight_times_too_small():
    """The replay has teeth: with E divided by 8, kept values fall outside it."""
    rng = np.random.default_rng(11)
    s, x = near_midpoint_windows(rng, 20000, 4)
    p = exact_pool(s, x)
    pc, E, keep = kernel_pool(s, x, np.ones(20000, bool), p, shrink=0.125)
    assert (np.abs(pc.astype(LD) - p)[keep] > E[keep].astype(LD)).any()
