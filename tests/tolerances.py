"""Tolerance rules for floating-point parity, shared by the CPU and GPU tests.

The oracle evaluates each stage exactly (fp64) and rounds once; any fp32
implementation differs from it by rounding.  The rules:

kv (wkv projection, fp32 accumulation, bf16 out):
  * at least 99.9 % of elements bit-equal to the oracle;
  * every element within 1 bf16 ulp, except where cancellation makes that
    impossible for any fp32 summation order: there the difference must stay
    within 2*sqrt(K)*2^-24*sum_k|a_k w_k| + 1/2 ulp (the standard bound for
    fp32 blocked summation of K terms, plus the final rounding); such
    elements are counted.
gate (fp32):
  * within 1e-5 relative of the oracle, except in the ill-conditioned band
    |a| < 1e-4 (a = the normalised weighted dot) where the sign of a is
    rounding noise: there g must lie in [sigmoid(-0.01), sigmoid(0.01)].
out (bf16):
  * within 2 bf16 ulp of the oracle, plus the propagated gate difference
    |g - g_ref|*|v| and fp32 rounding of h + g*v (2^-23*(|h| + |g v|));
    the count beyond a plain 2 ulp is reported and bounded.
"""
from __future__ import annotations

import math

import numpy as np

SIG_LO = 1.0 / (1.0 + math.exp(0.01))
SIG_HI = 1.0 / (1.0 + math.exp(-0.01))
BAND = 1e-4


def bf16_value(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (2^-133 in the subnormal range)."""
    a = np.abs(np.asarray(x, np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def check_kv(kv, ref, abs_dot=None, K=None, min_equal=0.999):
    """kv, ref: bf16 bits of the same shape; abs_dot = sum_k |a_k w_k| (fp64),
    needed only where elements differ by more than 1 ulp."""
    kv = np.asarray(kv, np.uint16)
    ref = np.asarray(ref, np.uint16)
    eq = kv == ref
    frac = float(eq.mean()) if eq.size else 1.0
    v, r = bf16_value(kv), bf16_value(ref)
    diff = np.abs(v - r)
    over = diff > ulp_bf16(r) * (1 + 1e-12)
    n_over = int(over.sum())
    if n_over:
        assert abs_dot is not None and K is not None, "kv beyond 1 ulp and no bound given"
        bound = 2 * math.sqrt(K) * 2.0 ** -24 * np.asarray(abs_dot)[over] + 0.5 * ulp_bf16(r[over])
        worst = diff[over] / bound
        assert np.all(worst <= 1.0), "kv beyond the cancellation bound: %r" % float(worst.max())
    assert frac >= min_equal, "kv bit-equal fraction %.6f < %.4f" % (frac, min_equal)
    return dict(bit_equal=frac, beyond_1ulp=n_over)


def check_gate(g, g_ref, a_ref, rtol=1e-5):
    g = np.asarray(g, np.float64)
    g_ref = np.asarray(g_ref, np.float64)
    a_ref = np.asarray(a_ref, np.float64)
    band = np.abs(a_ref) < BAND
    live = ~band
    rel = np.abs(g - g_ref) / np.maximum(np.abs(g_ref), 1e-300)
    ok = np.where(live, rel <= rtol, (g >= SIG_LO - 1e-7) & (g <= SIG_HI + 1e-7))
    # masked positions have g_ref == 0 exactly and must be exactly 0
    zero = g_ref == 0
    ok = np.where(zero, g == 0, ok)
    assert np.all(ok), "gate outside tolerance at %d places (max rel %.3g)" % (
        int((~ok).sum()), float(rel[live & ~zero].max()) if np.any(live & ~zero) else 0.0)
    return dict(max_rel=float(rel[live & ~zero].max()) if np.any(live & ~zero) else 0.0,
                band=int(band.sum()))


def check_out(out, ref, h, v, g, g_ref, max_frac_beyond=1e-3):
    """out, ref: bf16 bits [tok, hc, dim]; h bits [tok, hc, dim]; v bits [tok, dim];
    g, g_ref [tok, hc]."""
    o, r = bf16_value(out), bf16_value(ref)
    hv = bf16_value(h)
    vv = bf16_value(v)[:, None, :]
    gg = np.asarray(g_ref, np.float64)[:, :, None]
    dg = np.abs(np.asarray(g, np.float64) - np.asarray(g_ref, np.float64))[:, :, None]
    diff = np.abs(o - r)
    two = 2 * ulp_bf16(r) * (1 + 1e-12)
    bound = two + dg * np.abs(vv) + 2.0 ** -23 * (np.abs(hv) + np.abs(gg * vv))
    bad = diff > bound
    assert not np.any(bad), "out beyond bound at %d places" % int(bad.sum())
    beyond = float((diff > two).mean())
    assert beyond <= max_frac_beyond, "out beyond 2 ulp at a fraction %.3g" % beyond
    return dict(bit_equal=float((np.asarray(out) == np.asarray(ref)).mean()), beyond_2ulp=beyond)
