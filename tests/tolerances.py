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
    the count beyond a plain 2 ulp is reported and bounded.  End to end,
    where the value comes out of the projection, g*ulp(v) is added for a
    value one ulp away.
"""
from __future__ import annotations

import math

import numpy as np

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


def key_ulp_da(x_bits, key_bits, q_bits, k_bits, eps):
    """End to end the key comes out of the tested projection and may sit one
    bf16 ulp from the oracle's key in any element.  Returns a first-order
    bound on the resulting |a - a_ref| per (token, stream), from the oracle's
    own inputs: x [tok, hc, dim], key [tok, hc, dim], q/k [hc, dim] bits."""
    h = bf16_value(x_bits)
    key = bf16_value(key_bits)
    w = bf16_value(q_bits) * bf16_value(k_bits)
    u = ulp_bf16(key)
    D = h.shape[-1]
    shh = np.sum(h * h, -1)
    skk = np.sum(key * key, -1)
    shwk = np.sum(h * w[None] * key, -1)
    rstd = 1.0 / np.sqrt(shh / D + eps) / np.sqrt(skk / D + eps)
    d_hwk = np.sum(np.abs(h * w[None]) * u, -1)
    d_kk = np.sum(2 * np.abs(key) * u + u * u, -1)
    a = shwk * rstd / math.sqrt(D)
    return 2.0 * (d_hwk * rstd / math.sqrt(D) + np.abs(a) * 0.5 * (d_kk / D) / (skk / D + eps))


def check_gate(g, g_ref, a_ref, rtol=1e-5, da=None, min_tight=0.5):
    """da: optional bound on |a - a_ref| from inputs that differ (end to end);
    it widens the bound by its first-order effect on g and the band by da,
    and then at least `min_tight` of the live gates must still meet rtol.
    (End to end, a key of dim elements is bit-identical to the oracle's with
    probability about p^dim, p = the kv bit-equal fraction: ~0.97 at dim 256,
    ~0.6 at dim 5120 for p = 0.9999; the gates of the other keys are held to
    the propagated bound.)"""
    g = np.asarray(g, np.float64)
    g_ref = np.asarray(g_ref, np.float64)
    a_ref = np.asarray(a_ref, np.float64)
    extra = 0.0
    band_w = BAND
    if da is not None:
        da = np.asarray(da, np.float64)
        s = np.sqrt(np.maximum(np.abs(a_ref), 1e-6))
        extra = g_ref * (1 - g_ref) * da / (2 * s) / np.maximum(g_ref, 1e-300)
        band_w = BAND + da
    band = np.abs(a_ref) < band_w
    live = ~band
    rel = np.abs(g - g_ref) / np.maximum(np.abs(g_ref), 1e-300)
    # in the band, g may be sigmoid of anything in [-sqrt(band), +sqrt(band)]
    half = 1.0 / (1.0 + np.exp(-np.sqrt(np.maximum(band_w, 1e-6)))) - 0.5
    in_band = np.abs(g - 0.5) <= half + 1e-7
    ok = np.where(live, rel <= rtol + extra, in_band)
    # masked positions have g_ref == 0 exactly and must be exactly 0
    zero = g_ref == 0
    ok = np.where(zero, g == 0, ok)
    if not np.all(ok):
        bad = np.nonzero(~ok)
        raise AssertionError("gate outside tolerance at %d places (max rel %.3g); first: g=%r "
                             "g_ref=%r a_ref=%r" % (
                                 int((~ok).sum()),
                                 float(rel[live & ~zero].max()) if np.any(live & ~zero) else 0.0,
                                 g[bad][:4].tolist(), g_ref[bad][:4].tolist(),
                                 a_ref[bad][:4].tolist()))
    live_nz = live & ~zero
    tight = float((rel[live_nz] <= rtol).mean()) if np.any(live_nz) else 1.0
    if da is not None:
        assert tight >= min_tight, "only %.4f of live gates within %g" % (tight, rtol)
    return dict(max_rel=float(rel[live_nz].max()) if np.any(live_nz) else 0.0,
                band=int(band.sum()), tight=tight)


def check_out(out, ref, h, v, g, g_ref, max_frac_beyond=1e-3, v_ulps=0):
    """out, ref: bf16 bits [tok, hc, dim]; h bits [tok, hc, dim]; v bits [tok, dim]
    (the oracle's value); g, g_ref [tok, hc].  v_ulps > 0 admits a value that
    itself differs by that many bf16 ulp (end-to-end runs, where the value
    comes out of the tested projection)."""
    o, r = bf16_value(out), bf16_value(ref)
    hv = bf16_value(h)
    vv = bf16_value(v)[:, None, :]
    gg = np.asarray(g_ref, np.float64)[:, :, None]
    dg = np.abs(np.asarray(g, np.float64) - np.asarray(g_ref, np.float64))[:, :, None]
    diff = np.abs(o - r)
    two = 2 * ulp_bf16(r) * (1 + 1e-12)
    bound = two + dg * np.abs(vv) + 2.0 ** -23 * (np.abs(hv) + np.abs(gg * vv))
    if v_ulps:
        bound = bound + gg * v_ulps * ulp_bf16(vv)
    bad = diff > bound
    assert not np.any(bad), "out beyond bound at %d places" % int(bad.sum())
    beyond = float((diff > two).mean())
    assert beyond <= max_frac_beyond, "out beyond 2 ulp at a fraction %.3g" % beyond
    return dict(bit_equal=float((np.asarray(out) == np.asarray(ref)).mean()), beyond_2ulp=beyond)
