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
end to end (the key and value come out of the tested projection):
  * each key and value element may differ from the oracle's by what the kv
    rule admits (kv_err_bound); key_da turns that into a rigorous bound on
    |a - a_ref| (first-order terms with their exact remainder), check_gate
    admits the exact spread of g over that interval, check_out the value's
    error times g;
  * floors on the observed rates (the fraction of live gates within 1e-5
    without that widening, the fraction of outputs beyond 2 ulp, the kv
    elements beyond 1 ulp) are asserted per workload by the tests.
"""
from __future__ import annotations

import math

import numpy as np

BAND = 1e-4


def bf16_value(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # signalling NaNs widen to quiet ones
        return b.view(np.float32).astype(np.float64)


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (2^-133 in the subnormal range)."""
    a = np.abs(np.asarray(x, np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def check_kv(kv, ref, abs_dot=None, K=None, min_equal=0.999, max_beyond=None):
    """kv, ref: bf16 bits of the same shape [M, N]; abs_dot = sum_k |a_k w_k|
    (fp64) per element, or a function of row indices returning it for those
    rows; needed only where elements differ by more than 1 ulp.
    max_beyond: optional ceiling on the count of elements beyond 1 ulp (a
    floor on the observed rate)."""
    kv = np.asarray(kv, np.uint16)
    ref = np.asarray(ref, np.uint16)
    eq = kv == ref
    frac = float(eq.mean()) if eq.size else 1.0
    v, r = bf16_value(kv), bf16_value(ref)
    diff = np.abs(v - r)
    over = diff > ulp_bf16(r) * (1 + 1e-12)
    n_over = int(over.sum())
    worst_all = 0.0
    if n_over:
        assert abs_dot is not None and K is not None, "kv beyond 1 ulp and no bound given"
        if callable(abs_dot):
            rows = np.nonzero(over.reshape(over.shape[0], -1).any(-1))[0]
            ad = np.asarray(abs_dot(rows)).reshape((len(rows),) + over.shape[1:])[over[rows]]
        else:
            ad = np.asarray(abs_dot)[over]
        bound = 2 * math.sqrt(K) * 2.0 ** -24 * ad + 0.5 * ulp_bf16(r[over])
        worst = diff[over] / bound
        worst_all = float(worst.max())
        assert np.all(worst <= 1.0), "kv beyond the cancellation bound: %r" % worst_all
    assert frac >= min_equal, "kv bit-equal fraction %.6f < %.4f" % (frac, min_equal)
    if max_beyond is not None:
        assert n_over <= max_beyond, "kv beyond 1 ulp at %d places (ceiling %d)" % (
            n_over, max_beyond)
    return dict(bit_equal=frac, beyond_1ulp=n_over, worst_vs_bound=worst_all)


def kv_err_bound(ref_bits, abs_dot=None, K=None) -> np.ndarray:
    """Per-element bound on |kv - kv_ref| that check_kv admits: one bf16 ulp
    of the oracle's element, or, where cancellation makes that impossible
    for an fp32 sum, 2*sqrt(K)*2^-24*sum|a*w| + 1/2 ulp (whichever is
    larger).  abs_dot = sum_k |a_k w_k| per element (fp64)."""
    u = ulp_bf16(bf16_value(ref_bits))
    if abs_dot is None:
        return u
    return np.maximum(u, 2 * math.sqrt(K) * 2.0 ** -24 * np.asarray(abs_dot) + 0.5 * u)


def key_da(x_bits, key_bits, q_bits, k_bits, eps, key_err=None):
    """End to end, the key the gate sees comes out of the tested projection
    and differs from the oracle's key by at most key_err per element (default
    one bf16 ulp; kv_err_bound gives the full rule).  Returns, per (token,
    stream), a rigorous bound on |a(key') - a(key)| over every such key'.

    With S_hwk = sum h*w*key, S = mean(key^2) + eps, c = rsqrt(mean(h^2)+eps)/sqrt(D),
    a = S_hwk * c / sqrt(S).  A change e_f per element moves S_hwk by at most
    d1 = sum |h*w|*e_f and S by at most x*S, x = sum(2|key|*e_f + e_f^2)/D/S,
    so for x < 1 (mean value theorem on t^-1/2):
      |a' - a| <= d1*c/sqrt(S) / sqrt(1-x) + |a| * x/2 / (1-x)^1.5.
    x: [tok, hc, dim] bits; key: [tok, hc, dim] bits; q/k: [hc, dim] bits."""
    h = bf16_value(x_bits)
    key = bf16_value(key_bits)
    w = bf16_value(q_bits) * bf16_value(k_bits)
    e = ulp_bf16(key) if key_err is None else np.asarray(key_err, np.float64)
    D = h.shape[-1]
    shh = np.sum(h * h, -1)
    skk = np.sum(key * key, -1)
    shwk = np.sum(h * w[None] * key, -1)
    S = skk / D + eps
    c = 1.0 / np.sqrt(shh / D + eps) / math.sqrt(D)
    d1 = np.sum(np.abs(h * w[None]) * e, -1)
    x = np.sum(2 * np.abs(key) * e + e * e, -1) / D / S
    assert np.all(x < 0.5), "key error bound too wide for a first-order bound"
    a = shwk * c / np.sqrt(S)
    return d1 * c / np.sqrt(S) / np.sqrt(1 - x) + np.abs(a) * 0.5 * x / (1 - x) ** 1.5


def gate_of(a):
    """g(a) = sigmoid(copysign(sqrt(max(|a|, fp32(1e-6))), a)) in fp64: the
    gate as a function of a, non-decreasing in a."""
    a = np.asarray(a, np.float64)
    s = np.copysign(np.sqrt(np.maximum(np.abs(a), float(np.float32(1e-6)))), a)
    return 1.0 / (1.0 + np.exp(-s))


def check_gate(g, g_ref, a_ref, rtol=1e-5, da=None, min_tight=None):
    """g within rtol of g_ref where |a_ref| >= BAND; inside the band, where
    the sign of a is rounding noise, g in [sigmoid(-sqrt(band)), sigmoid(+sqrt(band))].
    da: optional bound on |a - a_ref| from inputs that differ (end to end,
    the key comes out of the tested projection): every a' within da of
    a_ref is admitted, which widens the relative bound by the exact spread
    of g over [a_ref - da, a_ref + da] (g is monotonic in a) and the band
    by da.  min_tight: the least fraction of live gates that must still
    meet rtol without that widening (a floor on the observed rate)."""
    g = np.asarray(g, np.float64)
    g_ref = np.asarray(g_ref, np.float64)
    a_ref = np.asarray(a_ref, np.float64)
    extra = 0.0
    band_w = BAND
    if da is not None:
        da = np.asarray(da, np.float64)
        g0 = gate_of(a_ref)
        spread = np.maximum(gate_of(a_ref + da) - g0, g0 - gate_of(a_ref - da))
        extra = spread / np.maximum(g_ref, 1e-300)
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
    if min_tight is not None:
        assert tight >= min_tight, "only %.4f of live gates within %g (floor %.4f)" % (
            tight, rtol, min_tight)
    return dict(max_rel=float(rel[live_nz].max()) if np.any(live_nz) else 0.0,
                band=int(band.sum()), tight=tight)


def check_out(out, ref, h, v, g, g_ref, max_frac_beyond=1e-3, v_err=None):
    """out, ref: bf16 bits [tok, hc, dim]; h bits [tok, hc, dim]; v bits [tok, dim]
    (the oracle's value); g, g_ref [tok, hc].  v_err [tok, dim] (end-to-end
    runs, where the value comes out of the tested projection): a bound on
    |v - v_ref| per element (kv_err_bound), which the bound then admits."""
    o, r = bf16_value(out), bf16_value(ref)
    hv = bf16_value(h)
    vv = bf16_value(v)[:, None, :]
    gg = np.asarray(g_ref, np.float64)[:, :, None]
    dg = np.abs(np.asarray(g, np.float64) - np.asarray(g_ref, np.float64))[:, :, None]
    diff = np.abs(o - r)
    two = 2 * ulp_bf16(r) * (1 + 1e-12)
    bound = two + dg * np.abs(vv) + 2.0 ** -23 * (np.abs(hv) + np.abs(gg * vv))
    if v_err is not None:
        ve = np.asarray(v_err, np.float64)[:, None, :]
        bound = bound + gg * ve + dg * ve
    bad = diff > bound
    assert not np.any(bad), "out beyond bound at %d places" % int(bad.sum())
    beyond = float((diff > two).mean())
    assert beyond <= max_frac_beyond, "out beyond 2 ulp at a fraction %.3g" % beyond
    return dict(bit_equal=float((np.asarray(out) == np.asarray(ref)).mean()), beyond_2ulp=beyond)


def check_end_to_end(out_bits, gate, x_bits, ref, rows_bits, w_bits, q_bits, k_bits, eps,
                     min_tight=None, max_frac_beyond=1e-3, max_rel=None, chunk=256):
    """Gate and out of a whole forward against the oracle's, for n positions.
    out_bits, x_bits [n, hc, dim]; gate [n, hc]; ref: the oracle's kv [n, N],
    out, gate and a; rows_bits [n, K] the oracle's gathered rows; w_bits
    [N, K]; q_bits, k_bits [hc, dim].  Each key and value element is allowed
    what the kv rule allows (kv_err_bound, from sum|a*w| per element): a
    worst-case admission (every element off by its whole allowance, all
    errors aligned), far wider than what a projection that rounds correctly
    almost everywhere produces.  The discriminating checks are the floors
    on the whole set: min_tight (fraction of live gates within 1e-5 of the
    oracle with no widening), max_rel (ceiling on the largest relative gate
    difference outside the band) and max_frac_beyond (fraction of outputs
    beyond 2 ulp).  Works in chunks of positions."""
    n, hc, dim = x_bits.shape
    K = rows_bits.shape[1]
    hd = hc * dim
    wabs = np.abs(bf16_value(w_bits))
    n_live = n_tight = 0
    max_rel_seen = 0.0
    n_band = 0
    n_beyond = 0
    bit_equal = 0
    for i0 in range(0, n, chunk):
        sl = slice(i0, min(n, i0 + chunk))
        m = sl.stop - sl.start
        absdot = np.abs(bf16_value(rows_bits[sl])) @ wabs.T
        err = kv_err_bound(ref["kv"][sl], absdot, K)
        da = key_da(x_bits[sl], ref["kv"][sl, :hd].reshape(m, hc, dim), q_bits, k_bits, eps,
                    err[:, :hd].reshape(m, hc, dim))
        gs = check_gate(gate[sl], ref["gate"][sl], ref["a"][sl], da=da)
        os_ = check_out(out_bits[sl], ref["out"][sl], x_bits[sl], ref["kv"][sl, hd:], gate[sl],
                        ref["gate"][sl], max_frac_beyond=1.0, v_err=err[:, hd:])
        live = int(np.sum((np.abs(ref["a"][sl]) >= BAND + da) & (ref["gate"][sl] != 0)))
        n_live += live
        n_tight += int(round(gs["tight"] * live))
        max_rel_seen = max(max_rel_seen, gs["max_rel"])
        n_band += gs["band"]
        n_beyond += int(round(os_["beyond_2ulp"] * m * hd))
        bit_equal += int(round(os_["bit_equal"] * m * hd))
    tight = n_tight / n_live if n_live else 1.0
    beyond = n_beyond / (n * hd)
    if min_tight is not None:
        assert tight >= min_tight, "only %.5f of live gates within 1e-5 (floor %.5f)" % (
            tight, min_tight)
    if max_rel is not None:
        assert max_rel_seen <= max_rel, "largest relative gate difference %.3g (ceiling %.3g)" % (
            max_rel_seen, max_rel)
    assert beyond <= max_frac_beyond, "out beyond 2 ulp at a fraction %.3g (ceiling %.3g)" % (
        beyond, max_frac_beyond)
    return dict(gate_tight=tight, gate_max_rel=max_rel_seen, gate_band=n_band,
                out_bit_equal=bit_equal / (n * hd), out_beyond_2ulp=beyond)
