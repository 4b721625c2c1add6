"""The two GELU forms the kernels evaluate (device_common.h), emulated in
float32 on the CPU from the coefficients in the source file itself, against
the exact erf form GELU(x) = x Phi(x) (scipy.special.erf, float64).

The activation is the erf GELU ('gelu' in AuTEncoderConfig, m-star API page).
The device forms are approximations of it:

* gelu_f, for results stored as fp32: the Abramowitz & Stegun 7.1.26 rational
  fit of erfc; bound 3.3e-7 absolute over [-12, 12] with a correctly rounded
  reciprocal and exp2, 3.33e-7 with either one unit off;
* gelu_bf16, for results stored as bf16 or MX-fp8: 2^P(t) with a degree-5
  polynomial P fitted to log2 of the upper tail on [0, 5] and evaluated
  unclamped; bound 2.25e-5 absolute over [-16, 16], and at most 0.081 of half
  a bf16 unit in the last place of the result wherever |GELU| > 1e-3.

The hardware reciprocal and exp2 are approximate to about one unit in the last
place, so every point is evaluated with each of them at the correctly rounded
value and at both float32 neighbours, and the worst of the nine is taken.
"""
import os
import re

import numpy as np
import pytest
from scipy.special import erf, erfc

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "packed_windowed_attention_amd", "csrc", "device_common.h")
F32 = np.float32
LIT = re.compile(r"(?<![\w.])-?\d+\.\d*(?:e[-+]?\d+)?f")


def literals(fn: str) -> list[float]:
    """Float literals of a device function's body, in source order."""
    text = open(SRC).read()
    m = re.search(r"float\s+" + fn + r"\(float x\)\s*\{(.*?)\n\}", text, re.S)
    assert m, f"{fn} not found in {SRC}"
    return [float(s[:-1]) for s in LIT.findall(m.group(1))]


def fma(a, b, c):
    """float32 fused multiply-add: the exact a * b (exact in float64 for
    float32 operands) plus c, rounded once to float32 (double rounding through
    float64 differs from one rounding only in far-off ties)."""
    return (np.float64(a) * np.float64(b) + np.float64(c)).astype(F32)


def neighbours(v):
    v = v.astype(F32)
    return [np.nextafter(v, F32(-np.inf)), v, np.nextafter(v, F32(np.inf))]


def exp2_f32(v):
    return np.exp2(v.astype(np.float64)).astype(F32)


def gelu_exact(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def emulate_gelu_f(x):
    c = literals("gelu_f")
    # p/sqrt2, 1, a5/2, a4/2, a3/2, a2/2, a1/2, -log2(e)/2, 0
    assert len(c) == 9 and c[1] == 1.0 and c[8] == 0.0, c
    x = x.astype(F32)
    ax = np.abs(x)
    r = (1.0 / fma(F32(c[0]), ax, F32(1.0)).astype(np.float64)).astype(F32)
    arg = ((x * F32(c[7])).astype(F32) * x).astype(F32)
    outs = []
    for t in neighbours(r):
        q = F32(c[2])
        for k in (3, 4, 5, 6):
            q = fma(q, t, F32(c[k]))
        q = (q * t).astype(F32)
        for e in neighbours(exp2_f32(arg)):
            outs.append(fma(-ax, (q * e).astype(F32), np.maximum(x, F32(0))))
    return outs


def emulate_gelu_bf16(x):
    c = literals("gelu_bf16")
    # polynomial coefficients from the highest degree down, 0 (no clamp: t = |x|)
    assert len(c) == 7 and c[6] == 0.0, c
    x = x.astype(F32)
    t = np.abs(x)
    p = fma(F32(c[0]), t, F32(c[1]))
    for k in (2, 3, 4, 5):
        p = fma(p, t, F32(c[k]))
    return [fma(-t, e, np.maximum(x, F32(0))) for e in neighbours(exp2_f32(p))]


def grid(lo, hi, n, seed):
    r = np.random.default_rng(seed)
    x = np.concatenate([np.linspace(lo, hi, n), r.uniform(lo, hi, n),
                        r.standard_normal(n) * 3.0, [0.0, -0.0, 1e-30, -1e-30, lo, hi]])
    return x[(x >= lo) & (x <= hi)].astype(F32)


def bf16_half_ulp(v):
    """Half the spacing of bf16 numbers at |v| (8 significant bits)."""
    _, E = np.frexp(np.abs(np.asarray(v, dtype=np.float64)))
    return np.ldexp(1.0, E - 8) / 2.0


def test_gelu_f_bound():
    x = grid(-12.0, 12.0, 200_000, 1)
    ref = gelu_exact(x)
    err = max(float(np.abs(o.astype(np.float64) - ref).max()) for o in emulate_gelu_f(x))
    print(f"gelu_f max abs error {err:.3e}")
    assert err <= 3.35e-7


def test_gelu_bf16_bound():
    x = grid(-16.0, 16.0, 200_000, 2)
    ref = gelu_exact(x)
    outs = emulate_gelu_bf16(x)
    err = max(float(np.abs(o.astype(np.float64) - ref).max()) for o in outs)
    big = np.abs(ref) > 1e-3
    frac = max(float((np.abs(o.astype(np.float64) - ref)[big] / bf16_half_ulp(ref[big])).max()) for o in outs)
    print(f"gelu_bf16 max abs error {err:.3e}; worst fraction of half a bf16 ulp {frac:.3f}")
    assert err <= 2.25e-5
    assert frac <= 0.081


def test_gelu_bf16_unclamped_tail():
    """gelu_bf16 evaluates its polynomial past the fitted range [0, 5]: there
    the tail term |x| 2^P(|x|) must stay negligible (P keeps falling), out to
    |x| = 1e6, so GELU(x) is x or 0 within far less than a bf16 step."""
    t = np.geomspace(5.0, 1e6, 20_000)
    x = np.concatenate([t, -t]).astype(F32)
    xd = x.astype(np.float64)
    # x Phi(x) through erfc, exact in float64 also where Phi(x) underflows 1 - erf
    ref = 0.5 * xd * erfc(-xd / np.sqrt(2.0))
    for o in emulate_gelu_bf16(x):
        o = o.astype(np.float64)
        # x > 0: x to float32 rounding; x < 0: a value of magnitude below 2e-6
        # (the true one is smaller still), far below any bf16 step of the output
        pos = x > 0
        assert float((np.abs(o - ref)[pos] / ref[pos]).max()) <= 2.0 ** -20
        assert float(np.abs(o[~pos]).max()) <= 2e-6 and float(np.abs(ref[~pos]).max()) <= 2e-6
    c = literals("gelu_bf16")
    p = np.polyval(np.array(c[:6], dtype=np.float64), t)
    assert float(p[t >= 5.5].max()) < -25.0


@pytest.mark.parametrize("fn", ["gelu_f", "gelu_bf16"])
def test_gelu_special_values(fn):
    """GELU(0) = 0 exactly, and far out the form is the identity (x > 0) or 0
    (x < 0) to within its bound."""
    emu = emulate_gelu_f if fn == "gelu_f" else emulate_gelu_bf16
    x = np.array([0.0, 30.0, -30.0], dtype=F32)
    for o in emu(x):
        assert o[0] == 0.0
        assert abs(float(o[1]) - 30.0) <= 3e-5 and abs(float(o[2])) <= 3e-5


def test_emulation_catches_a_wrong_coefficient(monkeypatch):
    """Planted: the linear coefficient of gelu_f's rational fit off by 1e-3
    breaks the bound, so the emulation really reads the source's values."""
    orig = literals

    def bad(fn):
        c = orig(fn)
        if fn == "gelu_f":
            c[6] += 1e-3
        return c

    monkeypatch.setattr(__import__(__name__), "literals", bad)
    x = grid(-12.0, 12.0, 20_000, 3)
    err = max(float(np.abs(o.astype(np.float64) - gelu_exact(x)).max()) for o in emulate_gelu_f(x))
    assert err > 3.35e-7
