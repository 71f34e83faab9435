"""Pins for the oracle's gate-and-add (stage 4).

Closed forms that follow from the gate equations on the "Gate per stream" page
and the Engram block's `forward`, written in terms of the inputs rather than
the oracle's steps:
  * key = c*x, unit weights:  a = c*sqrt(D)*m / sqrt((m+eps)(c^2 m+eps)),
    m = mean(x^2)  ->  a = sign(c)*sqrt(D) as eps -> 0;
  * eps = 0, unit weights:    a = sqrt(D) * cos(h, key)  (cosine similarity);
  * key = x, eps = 0:         a = sqrt(D) * sum(w x^2) / sum(x^2);
  * zero dot:                 g = sigmoid(+sqrt(fp32(1e-6)));
  * masked positions pass x through bit-exactly, gate 0.
"""
import json
import math
import os

import numpy as np
import torch

import oracle
import synth

from tests import tolerances

GOLD = os.path.join(os.path.dirname(__file__), "golden")
CLAMP = float(np.float32(1e-6))


def bf(a):
    return torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def val(b):
    return oracle.bf16_value(b)


def sig(s):
    return 1.0 / (1.0 + math.exp(-s))


def kv_from(key, value):
    """key [tok, hc, dim], value [tok, dim] -> kv [tok, dim*(hc+1)] (bits)."""
    tok, hc, dim = key.shape
    return np.concatenate([key.reshape(tok, hc * dim), value], axis=1)


def test_key_proportional_to_stream_closed_form():
    rng = np.random.default_rng(0)
    D, hc = 256, 4
    x = bf(rng.standard_normal((3, hc, D)))
    cs = np.array([0.5, -2.0, 0.25, -1.0])              # powers of two: c*x exact in bf16
    key = bf(val(x) * cs[None, :, None])
    v = bf(rng.standard_normal((3, D)))
    ones = bf(np.ones((hc, D)))
    xv = val(x)
    m = np.mean(xv * xv, axis=-1)
    for eps in (1e-6, 0.0, 0.25):
        e = float(np.float32(eps))
        _, gate, a = oracle.gate_and_add(x, kv_from(key, v), ones, ones, eps)
        c = cs[None, :]
        exp_a = c * math.sqrt(D) * m / np.sqrt((m + e) * (c * c * m + e))
        assert np.allclose(a, exp_a, rtol=1e-12, atol=0)
    # eps -> 0: a = sign(c) sqrt(D), g = sigmoid(sign(c) D^(1/4))
    _, gate, a = oracle.gate_and_add(x, kv_from(key, v), ones, ones, 0.0)
    assert np.allclose(a, np.sign(cs)[None, :] * math.sqrt(D), rtol=1e-13)
    assert abs(gate[0, 0] - 0.98201376) < 1e-7 and abs(gate[0, 1] - 0.017986210) < 1e-8


def test_dim_5120_gate_extremes():
    rng = np.random.default_rng(1)
    D = 5120
    x = bf(rng.standard_normal((1, 2, D)))
    key = bf(val(x) * np.array([1.0, -1.0])[None, :, None])
    v = bf(np.zeros((1, D)))
    ones = bf(np.ones((2, D)))
    out, gate, a = oracle.gate_and_add(x, kv_from(key, v), ones, ones, 0.0)
    assert abs(gate[0, 0] - 0.99978811) < 1e-7 and abs(gate[0, 1] - 2.1194536e-4) < 1e-10
    assert np.array_equal(out, x)                        # zero value adds nothing


def test_streams_normalised_separately():
    rng = np.random.default_rng(2)
    D, hc = 128, 4
    base = rng.standard_normal((2, 1, D))
    scale = np.array([1.0, 4.0, 1 / 16, 64.0])[None, :, None]
    x = bf(base * scale)
    key = bf(val(x) * 2.0)
    v = bf(rng.standard_normal((2, D)))
    ones = bf(np.ones((hc, D)))
    _, _, a = oracle.gate_and_add(x, kv_from(key, v), ones, ones, 0.0)
    # joint normalisation over the copies would make these differ by stream
    assert np.allclose(a, math.sqrt(D), rtol=1e-13)


def test_cosine_identity():
    rng = np.random.default_rng(3)
    D, hc, tok = 200, 3, 5
    x = bf(rng.standard_normal((tok, hc, D)))
    key = bf(rng.standard_normal((tok, hc, D)) + 0.3 * val(x))
    v = bf(rng.standard_normal((tok, D)))
    ones = bf(np.ones((hc, D)))
    _, gate, a = oracle.gate_and_add(x, kv_from(key, v), ones, ones, 0.0)
    h, k = val(x), val(key)
    cos = np.sum(h * k, -1) / (np.linalg.norm(h, axis=-1) * np.linalg.norm(k, axis=-1))
    assert np.allclose(a, math.sqrt(D) * cos, rtol=1e-12)
    s = np.sign(a) * np.sqrt(np.maximum(np.abs(a), CLAMP))
    assert np.allclose(gate, 1 / (1 + np.exp(-s)), rtol=1e-7)


def test_weight_is_elementwise_product_of_q_and_k():
    rng = np.random.default_rng(4)
    D, hc = 64, 2
    x = bf(rng.standard_normal((4, hc, D)))
    q = bf(1 + rng.uniform(-0.5, 0.5, (hc, D)))
    k = bf(1 + rng.uniform(-0.5, 0.5, (hc, D)))
    v = bf(rng.standard_normal((4, D)))
    _, _, a = oracle.gate_and_add(x, kv_from(x, v), q, k, 0.0)
    h, w = val(x), val(q) * val(k)
    expect = math.sqrt(D) * np.sum(w[None] * h * h, -1) / np.sum(h * h, -1)
    assert np.allclose(a, expect, rtol=1e-12)
    # constant q = 2, k = 3: a = 6 sqrt(D) (a sum q + k would give 5 sqrt(D))
    two, three = bf(np.full((hc, D), 2.0)), bf(np.full((hc, D), 3.0))
    _, _, a = oracle.gate_and_add(x, kv_from(x, v), two, three, 0.0)
    assert np.allclose(a, 6 * math.sqrt(D), rtol=1e-13)


def test_zero_dot_takes_positive_clamp():
    rng = np.random.default_rng(5)
    D, hc = 64, 3
    x = bf(rng.standard_normal((1, hc, D)))
    key = np.zeros((1, hc, D), np.uint16)
    xv = val(x)
    # stream 0: zero key; stream 1: zero stream (x row zero);
    # stream 2: exactly orthogonal pair key_i = x_j, key_j = -x_i (equal weights)
    x[0, 1] = 0
    key[0, 1] = bf(rng.standard_normal(D))
    key[0, 2, 3] = x[0, 2, 7]
    key[0, 2, 7] = x[0, 2, 3] ^ 0x8000
    v = bf(rng.standard_normal((1, D)))
    ones = bf(np.ones((hc, D)))
    out, gate, a = oracle.gate_and_add(x, kv_from(key, v), ones, ones, 1e-6)
    assert np.all(a == 0) and np.all(np.copysign(1.0, a) == 1.0)
    g0 = sig(math.sqrt(CLAMP))
    assert np.all(gate == np.float32(g0))
    assert abs(g0 - 0.50024999998) < 1e-10   # sigmoid(0.001) = 1/2 + 1/4000 - ...


def test_tiny_negative_dot_is_clamped_with_its_sign():
    D = 8
    x = np.zeros((1, 1, D), np.float32)
    x[0, 0, 0] = 1.0
    key = np.zeros((1, 1, D), np.float32)
    key[0, 0, 0] = -(2.0 ** -24)
    key[0, 0, 1] = 1.0
    v = bf(np.ones((1, D)))
    ones = bf(np.ones((1, D)))
    _, gate, a = oracle.gate_and_add(bf(x), kv_from(bf(key), v), ones, ones, 0.0)
    assert -CLAMP < a[0, 0] < 0
    assert gate[0, 0] == np.float32(sig(-math.sqrt(CLAMP)))
    assert abs(gate[0, 0] - 0.49975000002) < 3e-8  # fp32 of sigmoid(-0.001)


def test_mask_and_zero_value_pass_through():
    cfg = synth.config("tiny")
    x = synth.activations(cfg, 16, "cpu")
    q, k = synth.qk_weights(cfg, "cpu")
    kv = torch.randn(16, cfg.dim * 5).to(torch.bfloat16)
    b = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    mask = np.ones(16, bool)
    mask[[0, 5, 6, 15]] = False
    out, gate, _ = oracle.gate_and_add(b(x), b(kv), b(q), b(k), 1e-6, mask)
    assert np.array_equal(out[~mask], b(x)[~mask])
    assert np.all(gate[~mask] == 0) and np.all(gate[mask] > 0)
    kv0 = kv.clone()
    kv0[:, 4 * cfg.dim:] = 0
    out, _, _ = oracle.gate_and_add(b(x), b(kv0), b(q), b(k), 1e-6)
    assert np.array_equal(out, b(x))


def test_output_is_one_rounding_of_h_plus_g_v():
    # key = 2x, unit weights, eps 0, D = 256: g = sigmoid(4) exactly known
    rng = np.random.default_rng(6)
    D = 256
    x = bf(rng.standard_normal((2, 1, D)))
    key = bf(val(x) * 2.0)
    v = bf(rng.standard_normal((2, D)) * 3)
    ones = bf(np.ones((1, D)))
    out, gate, _ = oracle.gate_and_add(x, kv_from(key, v), ones, ones, 0.0)
    g = sig(4.0)
    expect = oracle.bf16_round(val(x)[:, 0] + g * val(v))
    assert np.array_equal(out[:, 0], expect)


def test_agrees_with_fp32_torch_evaluation_of_the_gate_equations():
    # A semantics cross-check of the oracle (which stream a key belongs to,
    # the sign convention, the weight, masking, the final cast) against an
    # independent fp32 evaluation in torch on the CPU, in its own summation
    # order, of the "Gate per stream" page's two equations: a_k as the
    # weighted dot of stream k with its key over the product of the two RMS
    # values and sqrt(dim) (eps inside each RMS, as the block's code has it),
    # and g as the sigmoid of the signed square root of |a_k| clamped at
    # 1e-6.  The value is the last dim columns of kv, added to every stream.
    cfg = synth.config("tiny")
    g = torch.Generator().manual_seed(1)
    T, hc, D = 64, cfg.hc_mult, cfg.dim
    x = torch.randn(T, hc, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(T, D * (hc + 1), generator=g).to(torch.bfloat16)
    kv[:, :hc * D] += (x.float() * torch.rand(T, hc, 1, generator=g) * 2 - 1).reshape(T, -1).to(torch.bfloat16)
    q, k = synth.qk_weights(cfg, "cpu")
    live = torch.rand(T, generator=g) > 0.2
    eps = cfg.norm_eps
    X = x.float()
    value = kv[:, hc * D:].float()
    gate_t = torch.zeros(T, hc)
    out_t = torch.empty(T, hc, D)
    for s in range(hc):
        keys = kv[:, s * D:(s + 1) * D].float()          # [T, D], stream s's key
        wk = q[s].float() * k[s].float() * keys          # w_{k,f} * key_{k,f}
        num = torch.linalg.vecdot(X[:, s], wk)           # sum over f
        rms_x = torch.sqrt(torch.mean(X[:, s] ** 2, dim=1) + eps)
        rms_k = torch.sqrt(torch.mean(keys ** 2, dim=1) + eps)
        a_s = num / (rms_x * rms_k * math.sqrt(D))
        root = torch.sqrt(torch.clamp(a_s.abs(), min=1e-6))
        g_s = torch.sigmoid(torch.where(a_s < 0, -root, root))
        gate_t[:, s] = torch.where(live, g_s, torch.zeros_like(g_s))
        out_t[:, s] = X[:, s] + gate_t[:, s, None] * value
    out_t = out_t.to(torch.bfloat16)
    b = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    out, gate, a = oracle.gate_and_add(b(x), b(kv), b(q), b(k), eps, live.numpy())
    tolerances.check_gate(gate_t.numpy(), gate, a)
    tolerances.check_out(b(out_t), out, b(x), b(kv[:, hc * D:]), gate_t.numpy(), gate)
    assert np.array_equal(out[~live.numpy()], b(x)[~live.numpy()])


def test_non_finite_inputs_follow_the_blocks_clamp():
    # The block's forward clamps |a| with an elementwise clamp on a tensor,
    # which keeps a NaN ("DeepSeek V4.1" Engram block, forward): a NaN in a
    # stream or in its key makes that stream's a, g and every out element
    # NaN; a NaN in the value spoils that feature only; an infinite value
    # gives an infinite out (g > 0).  The oracle must show exactly the pattern
    # an fp32 torch evaluation of the block's expression shows, with every
    # NaN output as the canonical 0x7FC0 (reading R9).
    T, hc, D = 6, 4, 64
    g = torch.Generator().manual_seed(5)
    x = torch.randn(T, hc, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(T, D * (hc + 1), generator=g).to(torch.bfloat16)
    q = (1 + 0.1 * torch.rand(hc, D, generator=g)).to(torch.bfloat16)
    k = (1 + 0.1 * torch.rand(hc, D, generator=g)).to(torch.bfloat16)
    xi, kvi = x.view(torch.int16), kv.view(torch.int16)
    xi[0, 1, 7] = 0x7FA5                      # a signalling NaN in stream 1 of token 0
    kvi[1, hc * D + 9] = 0x7F80               # +inf in the value of token 1
    kvi[1, hc * D + 10] = 0xFF80 - 0x10000    # -inf
    kvi[2, hc * D + 4] = 0xFFD3 - 0x10000     # a negative NaN with a payload in the value
    kvi[3, 2 * D + 5] = 0x7FC0                # NaN in the key of stream 2 of token 3
    X, value = x.float(), kv[:, hc * D:].float()
    gate_t = torch.empty(T, hc)
    out_t = torch.empty(T, hc, D)
    for s_ in range(hc):
        keys = kv[:, s_ * D:(s_ + 1) * D].float()
        dot = (X[:, s_] * (q[s_].float() * k[s_].float()) * keys).sum(1)
        dot = dot * torch.rsqrt((X[:, s_] ** 2).mean(1) + 1e-6) * torch.rsqrt((keys ** 2).mean(1) + 1e-6)
        dot = dot / math.sqrt(D)
        # g of the gate page: the sigmoid of the square root of |a| held at
        # 1e-6 from below, carrying the sign of a; torch.clamp on a tensor
        # keeps a NaN, as the block's clamp does
        root = torch.sqrt(torch.clamp(dot.abs(), min=1e-6))
        gate_t[:, s_] = 1.0 / (1.0 + torch.exp(-torch.where(dot < 0, -root, root)))
        out_t[:, s_] = X[:, s_] + gate_t[:, s_, None] * value
    b = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    ob_t = b(out_t.to(torch.bfloat16))
    out, gate, _ = oracle.gate_and_add(b(x), b(kv), b(q), b(k), 1e-6)
    assert np.array_equal(np.isnan(gate), torch.isnan(gate_t).numpy())
    assert np.isnan(gate[0, 1]) and np.isnan(gate[3, 2]) and np.isnan(gate).sum() == 2
    special = lambda v: (v & 0x7F80) == 0x7F80
    nan = lambda v: special(v) & ((v & 0x007F) != 0)
    assert np.array_equal(special(out), special(ob_t)) and np.array_equal(nan(out), nan(ob_t))
    assert nan(out)[0, 1].all() and nan(out)[3, 2].all() and nan(out)[2, :, 4].all()
    assert np.all(out[nan(out)] == 0x7FC0)
    inf = special(out) & ~nan(out)
    assert np.array_equal(out[inf], ob_t[inf]) and inf.sum() == 2 * hc


def test_page_counts():
    gold = json.load(open(os.path.join(GOLD, "page_counts.json")))
    cfg = synth.config("prefill")
    assert synth.n_hash_cols(cfg) == gold["rows_per_position"]
    t = synth.hash_tables(cfg)
    geom = synth.geometry_dict(cfg, t["num_embeddings"])
    ids = synth.token_ids(cfg, 1, 8)
    h = oracle.hash_ids(t, geom, oracle.HashState(1, 16), ids)
    assert h.shape[-1] == gold["rows_per_position"]
    q, k = synth.qk_weights(cfg, "cpu")
    assert q.numel() == gold["q_weight"] and k.numel() == gold["k_weight"]
    assert q.numel() + k.numel() == gold["gate_parameters"]
    assert tuple(q.shape) == (gold["streams"], gold["dim"])
    # gate in/out shapes: [T, 4, 5120] x2 in, [T, 4] out
    x = synth.activations(cfg, 2, "cpu")
    kv = torch.zeros(2, cfg.dim * (cfg.hc_mult + 1), dtype=torch.bfloat16)
    b = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    out, gate, _ = oracle.gate_and_add(b(x), b(kv), b(q), b(k), cfg.norm_eps)
    assert gate.shape == (2, gold["streams"]) and out.shape == (2, gold["streams"], gold["dim"])
