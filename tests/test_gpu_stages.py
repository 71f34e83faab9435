"""GPU parity, stage by stage, at sizes the oracle finishes in seconds.

Each stage gets the same input bytes on both sides (hash ids for the gather
come from the oracle's hash, rows for the projection from the generator or
the oracle), so each stage's rounding is isolated; the end-to-end forward is
checked on top.  Bars: hash ids and gathered rows bit-exact; kv, gate and out
per tests/tolerances.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import tolerances
from tests.gpu_util import Workload, bits, device_tables, from_bits, geometry, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    import gram_memory_layer_amd as ge
    ge.load()
    return ge


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def tiny(ge, dev):
    return Workload(ge, "tiny", dev)


# ------------------------------------------------------------------ stage 1: hash
@pytest.mark.parametrize("B,T", [(1, 16), (4, 200), (3, 1), (2, 2), (5, 1000)])
def test_hash_fresh_bit_exact(ge, dev, tiny, B, T):
    say("hash fresh", B, T)
    ids = synth.token_ids(tiny.cfg, B, T, name="h%d_%d" % (B, T))
    ref = oracle.hash_ids(tiny.t, tiny.geom, oracle.HashState(B, T + 4), ids)
    got = ge.engram_hash(tiny.g, tiny.tables, torch.from_numpy(ids).to(dev))
    assert np.array_equal(got.cpu().numpy(), ref)


def test_hash_state_carries_across_calls(ge, dev, tiny):
    say("hash split")
    B, T = 3, 40
    ids = synth.token_ids(tiny.cfg, B, T, name="split")
    ref = oracle.hash_ids(tiny.t, tiny.geom, oracle.HashState(B, T + 4), ids)
    for k in (0, 1, 2, 5, 39):
        state = torch.full((B, tiny.cfg.max_ngram_size - 1), tiny.cfg.pad_id, dtype=torch.int32,
                           device=dev)
        parts = []
        if k:
            parts.append(ge.engram_hash(tiny.g, tiny.tables, torch.from_numpy(ids[:, :k]).to(dev),
                                        state=state))
        for s in range(k, T):
            parts.append(ge.engram_hash(tiny.g, tiny.tables,
                                        torch.from_numpy(ids[:, s:s + 1].copy()).to(dev),
                                        state=state))
        got = torch.cat(parts, dim=1).cpu().numpy()
        assert np.array_equal(got, ref), k
        # the state holds the last n-1 compressed ids
        assert np.array_equal(state.cpu().numpy(), tiny.t["token_map"][ids[:, -2:]])


# The state is read only by a sequence's first max_ngram_size-1 positions,
# which the hash kernel gives to workgroups that own whole sequences and
# rewrite the state after they have read it.  Chunks shorter than the state
# (the new state then keeps old entries), a sequence count that does not
# fill the last such workgroup, and more head items per sequence than one
# workgroup pass (n_cols 300).
@pytest.mark.parametrize("mx,nh,B,chunks", [(5, 2, 7, (1, 3, 2, 4, 1, 9, 5)),
                                            (3, 150, 5, (1, 2, 7, 1)),
                                            (2, 1, 9, (1, 1, 3, 1))])
def test_hash_state_split_geometries(ge, dev, mx, nh, B, chunks):
    import dataclasses
    cfg = dataclasses.replace(synth.config("tiny"), max_ngram_size=mx, n_heads=nh,
                              prime_limit=100003)
    say("hash split geometry", mx, nh, B, chunks)
    wl = Workload(ge, cfg, dev, with_table=False, with_weights=False)
    T = sum(chunks)
    ids = synth.token_ids(cfg, B, T, name="splitg")
    ref = oracle.hash_ids(wl.t, wl.geom, oracle.HashState(B, T + 4), ids)
    state = torch.full((B, mx - 1), cfg.pad_id, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    parts, s0 = [], 0
    for c in chunks:
        parts.append(ge.engram_hash(wl.g, wl.tables, torch.from_numpy(ids[:, s0:s0 + c].copy()).to(dev),
                                    state=state, err=err))
        s0 += c
    got = torch.cat(parts, dim=1).cpu().numpy()
    assert np.array_equal(got, ref)
    assert int(err.item()) == 0
    # the state holds the last n-1 compressed ids
    assert np.array_equal(state.cpu().numpy(), wl.t["token_map"][ids[:, T - (mx - 1):]])


# Several layers in one launch: each layer's block of the output equals the
# single-layer call with that layer's tables, table size and state (the
# single-layer call is pinned to the oracle above).
@pytest.mark.parametrize("n_layers,B,chunks,with_state", [(3, 5, (7, 1, 2), True),
                                                          (4, 2, (300,), False),
                                                          (32, 3, (5, 1), True)])
def test_hash_layers_equal_single_calls(ge, dev, n_layers, B, chunks, with_state):
    import dataclasses
    base = dataclasses.replace(synth.config("tiny"), max_ngram_size=4, n_heads=3)
    say("hash layers", n_layers, B, chunks, with_state)
    cfgs = [dataclasses.replace(base, index=100 + l, prime_limit=1009 + 500 * l)
            for l in range(n_layers)]
    wls = [Workload(ge, c, dev, with_table=False, with_weights=False) for c in cfgs]
    assert len({w.num_emb for w in wls}) > 1
    T = sum(chunks)
    ids = synth.token_ids(base, B, T, name="layers")
    ids[0, 0] = base.vocab + 9                                # a bad token: flagged once
    st_multi = [torch.full((B, 3), base.pad_id, dtype=torch.int32, device=dev) + l
                for l in range(n_layers)] if with_state else None
    st_single = [s.clone() for s in st_multi] if with_state else None
    err_m = torch.zeros(1, dtype=torch.int32, device=dev)
    err_s = torch.zeros(1, dtype=torch.int32, device=dev)
    got, want, s0 = [], [], 0
    for c in chunks:
        part = torch.from_numpy(ids[:, s0:s0 + c].copy()).to(dev)
        got.append(ge.engram_hash_layers([w.g for w in wls], [w.tables for w in wls], part,
                                         states=st_multi, err=err_m))
        want.append(torch.stack([ge.engram_hash(w.g, w.tables, part,
                                                state=st_single[l] if with_state else None,
                                                err=err_s)
                                 for l, w in enumerate(wls)]))
        s0 += c
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(got, dim=2), torch.cat(want, dim=2))
    assert int(err_m.item()) == int(err_s.item()) == ge.ERRBIT_TOKEN
    if with_state:
        for a, b in zip(st_multi, st_single):
            assert torch.equal(a, b)


def _oracle_state(B, cap, seed_ids=None):
    """An oracle HashState whose history starts with the given compressed
    ids [B, n] (the look-back a carried state holds), or empty (fresh)."""
    st = oracle.HashState(B, cap)
    if seed_ids is not None:
        n = seed_ids.shape[1]
        st.hist[:, :n] = seed_ids
        st.length[:] = n
    return st


# Several layers in one launch against the oracle, layer by layer: layer l's
# block must equal oracle.hash_ids run with layer l's own tables (token map,
# multipliers, primes, offsets; the table sizes differ, as the block's
# constructor picks num_embeddings by the layer's hash index) and its own
# NgramHashState, carried over a prefill chunk and then one-token decode
# steps.  Covers the decode workload's geometry (24 columns, primes near
# 2^20, the full vocabulary) and the 32-layer maximum.
@pytest.mark.parametrize("n_layers,geo,B,chunks,seeded", [
    (3, "full", 4, (96, 1, 1, 1, 1), False),
    (5, "full", 64, (512, 1, 1, 1), True),
    (32, "small", 3, (9, 1, 1, 1, 1, 1), True),
    (32, "small", 2, (1, 1, 40), False)])
def test_hash_layers_vs_oracle(ge, dev, n_layers, geo, B, chunks, seeded):
    import dataclasses
    if geo == "full":
        base = synth.config("decode")
        cfgs = [dataclasses.replace(base, index=200 + l, prime_limit=(1 << 20) - 7919 * l)
                for l in range(n_layers)]
    else:
        base = dataclasses.replace(synth.config("tiny"), max_ngram_size=4, n_heads=3)
        cfgs = [dataclasses.replace(base, index=300 + l, prime_limit=1009 + 701 * l)
                for l in range(n_layers)]
    say("hash layers vs oracle", n_layers, geo, B, chunks, seeded)
    wls = [Workload(ge, c, dev, with_table=False, with_weights=False) for c in cfgs]
    assert len({w.num_emb for w in wls}) == n_layers
    nm1 = base.max_ngram_size - 1
    T = sum(chunks)
    ids = synth.token_ids(base, B, T, name="layers_vs_oracle")
    rng = np.random.default_rng(n_layers * 1000 + B)
    seeds = [rng.integers(0, base.n_compressed, (B, nm1)).astype(np.int32) if seeded else None
             for _ in range(n_layers)]
    ost = [_oracle_state(B, T + nm1 + 4, seeds[l]) for l in range(n_layers)]
    states = [torch.from_numpy(seeds[l] if seeded else
                               np.full((B, nm1), base.pad_id, np.int32)).to(dev)
              for l in range(n_layers)]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    s0 = 0
    for c in chunks:
        part = ids[:, s0:s0 + c].copy()
        got = ge.engram_hash_layers([w.g for w in wls], [w.tables for w in wls],
                                    torch.from_numpy(part).to(dev), states=states,
                                    err=err).cpu().numpy()
        for l, w in enumerate(wls):
            ref = oracle.hash_ids(w.t, w.geom, ost[l], part)
            assert np.array_equal(got[l], ref), (l, s0, c)
            # every id lies in its own column's slot of this layer's table
            col_lo = w.t["offset"].astype(np.int64)
            col_hi = col_lo + w.t["prime"].astype(np.int64)
            assert np.all((got[l] >= col_lo) & (got[l] < col_hi))
        s0 += c
    assert int(err.item()) == 0
    # each layer's state holds its last n-1 compressed ids
    for l, w in enumerate(wls):
        assert np.array_equal(states[l].cpu().numpy(), w.t["token_map"][ids[:, T - nm1:]])


def test_hash_bad_token_flags_and_stays_in_range(ge, dev, tiny):
    say("hash bad token")
    ids = synth.token_ids(tiny.cfg, 1, 16, name="bad")
    ids[0, 5] = tiny.cfg.vocab + 3
    ids[0, 9] = -1
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    got = ge.engram_hash(tiny.g, tiny.tables, torch.from_numpy(ids).to(dev), err=err).cpu().numpy()
    assert int(err.item()) & ge.ERRBIT_TOKEN
    lo = tiny.t["offset"].astype(np.int64)
    assert np.all(got >= lo) and np.all(got < lo + tiny.t["prime"].astype(np.int64))


def test_hash_inconsistent_tables_flag(ge, dev, tiny):
    say("hash bad table")
    t = dict(tiny.t)
    t["offset"] = t["offset"] + np.uint64(tiny.num_emb)      # every slot past the table
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ids = torch.from_numpy(synth.token_ids(tiny.cfg, 1, 8)).to(dev)
    got = ge.engram_hash(tiny.g, device_tables(t, dev), ids, err=err).cpu().numpy()
    assert int(err.item()) & ge.ERRBIT_HASH
    assert np.all(got == -1)


# ------------------------------------------------------------------ stage 2: rows
def test_gather_every_code_and_scale_pair(ge, dev):
    say("gather exhaustive")
    vc, sc = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    order = np.lexsort((vc.reshape(-1), sc.reshape(-1)))
    table = vc.reshape(-1)[order].reshape(-1, 64).astype(np.uint8)
    scales = sc.reshape(-1)[order].astype(np.uint8).reshape(-1, 32)[:, 0].reshape(-1, 2).copy()
    rows = table.shape[0]
    g = ge.Geometry.make(dim=64, hc_mult=1, max_ngram_size=2, n_heads=1, head_dim=64,
                         num_embeddings=rows, vocab=1)
    rng = np.random.default_rng(0)
    ids = np.concatenate([np.arange(rows), rng.integers(0, rows, 333)]).astype(np.int32)[:, None]
    ref = oracle.embed_rows(table, scales, ids[:, 0])
    got = ge.engram_gather(g, torch.from_numpy(table).to(dev), torch.from_numpy(scales).to(dev),
                           torch.from_numpy(ids).to(dev))
    assert np.array_equal(bits(got).reshape(ref.shape), ref)


def test_gather_tiny_bit_exact(ge, dev, tiny):
    say("gather tiny")
    ids = synth.token_ids(tiny.cfg, 2, 50, name="g")
    hid = oracle.hash_ids(tiny.t, tiny.geom, oracle.HashState(2, 64), ids).reshape(100, -1)
    ref = oracle.embed_rows(tiny.table.cpu().numpy(), tiny.scales.cpu().numpy(), hid)
    got = ge.engram_gather(tiny.g, tiny.table, tiny.scales, torch.from_numpy(hid).to(dev))
    assert np.array_equal(bits(got).reshape(ref.shape), ref)


def test_gather_bad_id_gives_zero_row(ge, dev, tiny):
    say("gather bad id")
    hid = np.array([[0, 5, tiny.num_emb, -7]], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    got = bits(ge.engram_gather(tiny.g, tiny.table, tiny.scales, torch.from_numpy(hid).to(dev),
                                err=err)).reshape(4, -1)
    assert int(err.item()) & ge.ERRBIT_ROW
    assert np.all(got[2:] == 0)
    ref = oracle.embed_rows(tiny.table.cpu().numpy(), tiny.scales.cpu().numpy(), hid[0, :2])
    assert np.array_equal(got[:2], ref)


# ------------------------------------------------------------------ stage 3: wkv
def _abs_dot(a_bits, w_bits):
    a = np.abs(tolerances.bf16_value(a_bits))
    w = np.abs(tolerances.bf16_value(w_bits))
    return a @ w.T


def _wkv_case(ge, dev, g, M, seed, kind="randn"):
    gen = torch.Generator(device=dev).manual_seed(seed)
    if kind == "randn":
        a = torch.randn((M, g.K), generator=gen, device=dev).to(torch.bfloat16)
        w = (torch.randn((g.N, g.K), generator=gen, device=dev) * g.K ** -0.5).to(torch.bfloat16)
    else:  # small integers: every partial sum exact in fp32
        a = torch.randint(-8, 9, (M, g.K), generator=gen, device=dev).to(torch.bfloat16)
        w = torch.randint(-8, 9, (g.N, g.K), generator=gen, device=dev).to(torch.bfloat16)
    kv = ge.engram_wkv(g, a, w)
    ab, wb = bits(a), bits(w)
    ref = oracle.linear(ab, wb)
    return bits(kv), ref, ab, wb


@pytest.mark.parametrize("M", [1, 16, 63, 64, 65, 300, 1024, 1100])
def test_wkv_tiny_geometry(ge, dev, tiny, M):
    say("wkv tiny M", M)
    kv, ref, ab, wb = _wkv_case(ge, dev, tiny.g, M, seed=M)
    st = tolerances.check_kv(kv, ref, _abs_dot(ab, wb), tiny.g.K)
    say("  ", st)


@pytest.mark.parametrize("M", [7, 300, 1500])
def test_wkv_ragged_n_and_k(ge, dev, M):
    # N = 200*5 = 1000 (not a multiple of any tile), K = 5*32 = 160 (a half k-tile)
    g = ge.Geometry.make(dim=200, hc_mult=4, max_ngram_size=6, n_heads=1, head_dim=32,
                         num_embeddings=1, vocab=1)
    say("wkv ragged M", M, "N", g.N, "K", g.K)
    kv, ref, ab, wb = _wkv_case(ge, dev, g, M, seed=100 + M)
    tolerances.check_kv(kv, ref, _abs_dot(ab, wb), g.K)


@pytest.mark.parametrize("M", [1030, 2600])
def test_wkv_ragged_n_main_kernel(ge, dev, M):
    # K = 2*32 = 64 (a whole k-tile), N = 1000: large-M kernel with a ragged N and M edge
    g = ge.Geometry.make(dim=200, hc_mult=4, max_ngram_size=3, n_heads=1, head_dim=32,
                         num_embeddings=1, vocab=1)
    say("wkv ragged main M", M, "N", g.N, "K", g.K)
    kv, ref, ab, wb = _wkv_case(ge, dev, g, M, seed=200 + M)
    tolerances.check_kv(kv, ref, _abs_dot(ab, wb), g.K)


@pytest.mark.parametrize("M", [50, 1030])
def test_wkv_small_integers_exact(ge, dev, tiny, M):
    say("wkv small ints", M)
    kv, ref, _, _ = _wkv_case(ge, dev, tiny.g, M, seed=7, kind="int")
    assert np.array_equal(kv, ref)


@pytest.mark.parametrize("M", [128, 1280])
def test_wkv_one_hot_rows_are_weight_columns(ge, dev, tiny, M):
    say("wkv one-hot", M)
    K = tiny.g.K
    a = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    r = torch.arange(M, device=dev)
    a[r, r % K] = 1.0
    w = synth.wkv_weight(tiny.cfg, dev)
    kv = ge.engram_wkv(tiny.g, a, w)
    expect = w.t()[(r % K)]
    assert torch.equal(kv.view(torch.int16), expect.contiguous().view(torch.int16))


# ------------------------------------------------------------------ stage 4: gate
def _gate_inputs(cfg, n_tok, dev, name="kvg"):
    x = synth.activations(cfg, n_tok, dev, name="x" + name)
    q, k = synth.qk_weights(cfg, dev)
    kv, cat = synth.gate_stress_kv(cfg, x, q, k, name=name)
    return x, kv, q, k, cat


def _gate_check(ge, g, x, kv, q, k, mask=None, inplace=False):
    n_tok = x.shape[0]
    gate = torch.empty((n_tok, g.hc_mult), dtype=torch.float32, device=x.device)
    xb = bits(x)
    if inplace:
        out = x.clone()
        ge.engram_gate_add(g, out, kv, q, k, mask=mask, out=out, gate=gate)
    else:
        out = ge.engram_gate_add(g, x, kv, q, k, mask=mask, gate=gate)
    m = None if mask is None else mask.cpu().numpy()
    ref_out, ref_g, ref_a = oracle.gate_and_add(xb, bits(kv), bits(q), bits(k), g.norm_eps, m)
    gs = tolerances.check_gate(gate.cpu().numpy(), ref_g, ref_a)
    os_ = tolerances.check_out(bits(out), ref_out, xb, bits(kv)[:, g.hc_mult * g.dim:],
                               gate.cpu().numpy(), ref_g)
    if m is not None:
        assert np.array_equal(bits(out)[~m.astype(bool)], xb[~m.astype(bool)])
    return gs, os_, out, gate


def test_gate_tiny(ge, dev, tiny):
    say("gate tiny")
    x, kv, q, k, _ = _gate_inputs(tiny.cfg, 64, dev)
    say("  ", _gate_check(ge, tiny.g, x, kv, q, k)[:2])


def test_gate_full_width_stress_recipe(ge, dev):
    cfg = synth.config("gate_stress")
    t = synth.hash_tables(cfg)
    g = geometry(ge, cfg, t["num_embeddings"])
    say("gate dim 5120, 96 tokens")
    x, kv, q, k, cat = _gate_inputs(cfg, 96, dev)
    gs, os_, out, gate = _gate_check(ge, g, x, kv, q, k)
    say("  ", gs, os_)
    # exactly orthogonal keys: dot is +0 -> g = sigmoid(+sqrt(fp32(1e-6)))
    orth = cat.cpu().numpy() == 0
    assert orth.any()
    g0 = np.float32(1.0 / (1.0 + np.exp(-np.sqrt(np.float64(np.float32(1e-6))))))
    gv = gate.cpu().numpy()[orth]
    assert np.all(np.abs(gv - g0) <= np.spacing(g0)), gv[:4]


def test_gate_small_batches_equal_large(ge, dev):
    # batches under four tokens per compute unit run one workgroup per
    # (token, stream) instead of one per token: the same sums in the same
    # order, so both layouts must agree bit for bit (both gate forms)
    cfg = synth.config("gate_stress")
    t = synth.hash_tables(cfg)
    g = geometry(ge, cfg, t["num_embeddings"])
    say("gate small vs large batch")
    n_big, n_small = 1100, 64
    x, kv, q, k, _ = _gate_inputs(cfg, n_big, dev, name="split")
    x = x.reshape(n_big, cfg.hc_mult, cfg.dim)
    mask = torch.from_numpy(synth.token_ids(cfg, 1, n_big, name="splitm")[0] % 5 != 0).to(dev)
    gen = torch.Generator(device=dev).manual_seed(77)
    nq = cfg.dim // 128
    part = torch.randn((n_big, cfg.hc_mult, nq, 2), generator=gen, device=dev)
    part[..., 0] = part[..., 0].abs() * 40.0
    v = kv[:, cfg.hc_mult * cfg.dim:].contiguous()
    for form in ("kv", "partials"):
        outs, gates = [], []
        for n in (n_big, n_small):
            gate = torch.empty((n, cfg.hc_mult), dtype=torch.float32, device=dev)
            if form == "kv":
                o = ge.engram_gate_add(g, x[:n], kv[:n], q, k, mask=mask[:n], gate=gate)
            else:
                o = ge.engram_gate_from_partials(g, x[:n], v[:n], part[:n], mask=mask[:n],
                                                 gate=gate)
            outs.append(o)
            gates.append(gate)
        torch.cuda.synchronize()
        assert torch.equal(outs[0][:n_small].view(torch.int16), outs[1].view(torch.int16)), form
        assert torch.equal(gates[0][:n_small], gates[1]), form


@pytest.mark.parametrize("hc,dim,n_tok", [(3, 16384, 6), (8, 32768, 3), (1, 8, 50), (2, 1000, 33)])
def test_gate_other_geometries(ge, dev, hc, dim, n_tok):
    # streaming variant (x and value re-read), tiny dims, odd chunk counts
    g = ge.Geometry.make(dim=dim, hc_mult=hc, max_ngram_size=2, n_heads=1, head_dim=32,
                         num_embeddings=1, vocab=1)
    say("gate hc", hc, "dim", dim)
    gen = torch.Generator(device=dev).manual_seed(hc * 7 + dim)
    x = torch.randn((n_tok, hc, dim), generator=gen, device=dev).to(torch.bfloat16)
    key = x.float() * torch.rand((n_tok, hc, 1), generator=gen, device=dev) * 2 - x.float() * 0.5
    key = key + 0.3 * torch.randn((n_tok, hc, dim), generator=gen, device=dev)
    v = torch.randn((n_tok, dim), generator=gen, device=dev)
    kv = torch.cat([key.reshape(n_tok, hc * dim), v], dim=1).to(torch.bfloat16)
    q = (1 + 0.1 * torch.rand((hc, dim), generator=gen, device=dev)).to(torch.bfloat16)
    k = (1 + 0.1 * torch.rand((hc, dim), generator=gen, device=dev)).to(torch.bfloat16)
    mask = torch.ones(n_tok, dtype=torch.bool, device=dev)
    mask[n_tok // 2] = False
    _gate_check(ge, g, x, kv, q, k, mask=mask)


# NaN and infinity in the inputs, in the form with one workgroup per token
# (1100 tokens) and one per (token, stream) (6 tokens): out must carry the
# oracle's bits wherever either is not finite (a NaN always as the canonical
# 0x7FC0, reading R9, whatever the input NaN's sign and payload), gates must
# be NaN exactly where the oracle's are, and every finite value must meet the
# usual tolerances.
@pytest.mark.parametrize("n_tok", [6, 1100])
def test_gate_special_values(ge, dev, n_tok):
    hc, dim = 4, 256
    g = ge.Geometry.make(dim=dim, hc_mult=hc, max_ngram_size=2, n_heads=1, head_dim=32,
                         num_embeddings=1, vocab=1)
    say("gate special values, tokens", n_tok)
    gen = torch.Generator(device=dev).manual_seed(31 + n_tok)
    x = torch.randn((n_tok, hc, dim), generator=gen, device=dev).to(torch.bfloat16)
    key = x.float() * (torch.rand((n_tok, hc, 1), generator=gen, device=dev) * 2 - 1)
    key = key + 0.3 * torch.randn((n_tok, hc, dim), generator=gen, device=dev)
    v = torch.randn((n_tok, dim), generator=gen, device=dev)
    kv = torch.cat([key.reshape(n_tok, hc * dim), v], dim=1).to(torch.bfloat16)
    q = (1 + 0.1 * torch.rand((hc, dim), generator=gen, device=dev)).to(torch.bfloat16)
    k = (1 + 0.1 * torch.rand((hc, dim), generator=gen, device=dev)).to(torch.bfloat16)
    xi, kvi = x.view(torch.int16), kv.view(torch.int16)
    vo = hc * dim
    xi[0, 1, 7] = 0x7FA5                      # a signalling NaN in h: stream 1 of token 0
    kvi[1, vo + 9] = 0x7F80                   # +inf in the value
    kvi[1, vo + 10] = 0xFF80 - 0x10000        # -inf in the value
    kvi[2, vo + 4] = 0xFFD3 - 0x10000         # NaN with sign and payload in the value
    kvi[3, 2 * dim + 5] = 0x7FC0              # NaN in the key of stream 2 of token 3
    gate = torch.empty((n_tok, hc), dtype=torch.float32, device=dev)
    out = ge.engram_gate_add(g, x, kv, q, k, gate=gate)
    xb, kvb = bits(x), bits(kv)
    ref_out, ref_g, ref_a = oracle.gate_and_add(xb, kvb, bits(q), bits(k), g.norm_eps)
    ob, gg = bits(out), gate.cpu().numpy()
    special = lambda b: (b & 0x7F80) == 0x7F80  # NaN or infinity (bf16 bits)
    sp = special(ref_out)
    assert np.array_equal(special(ob), sp)
    assert np.array_equal(ob[sp], ref_out[sp])
    assert np.all(ob[np.isnan(tolerances.bf16_value(ob))] == 0x7FC0)
    assert np.array_equal(np.isnan(gg), np.isnan(ref_g))
    assert np.isnan(ref_g[0, 1]) and np.isnan(ref_g[3, 2]) and sp[1, :, 9].all() and sp[2, :, 4].all()
    # the finite rest, with the non-finite places zeroed on both sides
    gz, rgz = np.where(np.isnan(gg), 0.0, gg), np.where(np.isnan(ref_g), 0.0, ref_g)
    raz = np.where(np.isnan(ref_a), 0.0, ref_a)
    tolerances.check_gate(gz, rgz, raz)
    vb = kvb[:, vo:].copy()
    vb[special(vb)] = 0
    tolerances.check_out(np.where(sp, 0, ob), np.where(sp, 0, ref_out), xb, vb, gz, rgz)


def test_gate_mask_and_in_place(ge, dev, tiny):
    say("gate mask in place")
    x, kv, q, k, _ = _gate_inputs(tiny.cfg, 40, dev, name="m")
    mask = torch.ones(40, dtype=torch.bool, device=dev)
    mask[[0, 3, 4, 39]] = False
    _, _, out, gate = _gate_check(ge, tiny.g, x, kv, q, k, mask=mask, inplace=True)
    assert torch.all(gate[~mask] == 0)


def test_gate_deterministic(ge, dev):
    cfg = synth.config("prefill")
    g = geometry(ge, cfg, 1)
    say("gate determinism")
    x, kv, q, k, _ = _gate_inputs(cfg, 128, dev, name="d")
    g1 = torch.empty((128, 4), device=dev)
    g2 = torch.empty((128, 4), device=dev)
    o1 = ge.engram_gate_add(g, x, kv, q, k, gate=g1)
    o2 = ge.engram_gate_add(g, x, kv, q, k, gate=g2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(g1, g2)


# ------------------------------------------------------------------ end to end
def test_forward_tiny_end_to_end(ge, dev, tiny):
    say("forward tiny")
    cfg = tiny.cfg
    for B, T in ((1, 16), (3, 37)):
        ids = synth.token_ids(cfg, B, T, name="f%d" % T)
        x = synth.activations(cfg, B * T, dev, name="xf%d" % T).reshape(B, T, cfg.hc_mult, cfg.dim)
        mask = torch.from_numpy(synth.token_ids(cfg, B, T, name="mk") % 5 != 0).to(dev)
        gate = torch.empty((B, T, cfg.hc_mult), dtype=torch.float32, device=dev)
        state = torch.full((B, cfg.max_ngram_size - 1), cfg.pad_id, dtype=torch.int32, device=dev)
        out = ge.engram_forward(tiny.g, tiny.tables, tiny.table, tiny.scales, tiny.w, tiny.q,
                                tiny.k, x, torch.from_numpy(ids).to(dev), mask=mask, state=state,
                                gate=gate)
        ref = oracle.forward(tiny.t, tiny.geom, oracle.HashState(B, T + 4), ids,
                             tiny.table.cpu().numpy(), tiny.scales.cpu().numpy(), bits(tiny.w),
                             bits(tiny.q), bits(tiny.k), bits(x), mask.cpu().numpy())
        n = B * T
        tolerances.check_end_to_end(bits(out).reshape(n, cfg.hc_mult, cfg.dim),
                                    gate.cpu().numpy().reshape(n, -1),
                                    bits(x).reshape(n, cfg.hc_mult, cfg.dim), ref, ref["rows"],
                                    bits(tiny.w), bits(tiny.q), bits(tiny.k), cfg.norm_eps)
        mk = mask.cpu().numpy().reshape(-1)
        assert np.array_equal(bits(out).reshape(n, -1)[~mk], bits(x).reshape(n, -1)[~mk])
        assert np.array_equal(state.cpu().numpy(), tiny.t["token_map"][ids[:, -2:]])
