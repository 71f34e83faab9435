"""Parity of the fused gather + projection (engram_wkv_gathered) with the
oracle's embed_rows followed by linear, and with the library's own two-stage
path (engram_gather then engram_wkv), which takes every product and every
fp32 sum in the same order, so the two must agree bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import tolerances
from tests.gpu_util import bits, geometry, say, Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    import gram_memory_layer_amd as m
    m.load()
    return m


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def _small(dim, hc, max_ngram, n_heads, rows, scale_codes=(120, 132)):
    base = synth.config("tiny")
    return dataclasses.replace(base, dim=dim, hc_mult=hc, max_ngram_size=max_ngram,
                               n_heads=n_heads, head_dim=64, scale_codes=scale_codes), rows


def _check_against_oracle_and_two_stage(ge, g, cfg, table, scales, hid, w, sample=None):
    dev = hid.device
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv = ge.engram_wkv_gathered(g, table, scales, hid, w, err=err)
    two = ge.engram_wkv(g, ge.engram_gather(g, table, scales, hid), w)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(kv.view(torch.int16), two.view(torch.int16)), "fused != gather + wkv"
    h = hid.reshape(-1, g.n_hash_cols).cpu().numpy()
    pos = np.arange(h.shape[0]) if sample is None else sample
    # the oracle sees only the table rows these positions reference
    uniq, inv = np.unique(h[pos].reshape(-1), return_inverse=True)
    idx = torch.from_numpy(uniq.astype(np.int64)).to(dev)
    tab = table.index_select(0, idx).cpu().numpy()
    sc = scales.index_select(0, idx).cpu().numpy()
    rows = oracle.embed_rows(tab, sc, inv.reshape(len(pos), -1).astype(np.int32))
    rows = rows.reshape(len(pos), -1)
    wb = bits(w)
    ref = oracle.linear(rows, wb)
    absdot = np.abs(tolerances.bf16_value(rows)) @ np.abs(tolerances.bf16_value(wb)).T
    got = bits(kv[torch.from_numpy(np.asarray(pos)).to(dev)])
    return tolerances.check_kv(got, ref, absdot, g.K)


# (dim, hc, max_ngram, n_heads): K = 64 * (max_ngram-1) * n_heads covers 1..12
# and 17 k-tiles: every prologue and drain sequence of the 3-stage ring, with
# and without passes of the steady loop; N = dim*(hc+1) covers whole and
# ragged 256-, 128- and 64-wide tiles.
GEOMS = [(256, 3, 2, 1), (200, 4, 3, 1), (256, 1, 2, 3), (512, 2, 3, 2), (96, 4, 5, 1),
         (128, 2, 6, 1), (320, 4, 4, 2), (64, 1, 8, 1), (256, 3, 5, 2), (64, 2, 4, 3),
         (128, 1, 6, 2), (64, 1, 12, 1), (96, 2, 5, 3), (64, 1, 2, 17)]


@pytest.mark.parametrize("shape", GEOMS)
@pytest.mark.parametrize("M", [1, 37, 300, 1100])
def test_fused_small_geometries(ge, dev, shape, M):
    dim, hc, mx, nh = shape
    cfg, rows = _small(dim, hc, mx, nh, rows=5000)
    g = geometry(ge, cfg, rows)
    say("fused small", shape, "M", M, "N", g.N, "K", g.K)
    table, scales = synth.embedding_table(cfg, rows, dev)
    w = synth.wkv_weight(cfg, dev)
    rng = np.random.default_rng(1000 * M + dim)
    hid = torch.from_numpy(rng.integers(0, rows, (M, g.n_hash_cols)).astype(np.int32)).to(dev)
    st = _check_against_oracle_and_two_stage(ge, g, cfg, table, scales, hid, w)
    say("   kv", st)


# Shapes that take the persistent 256x256 kernel (nk % 3 == 0 and at least two
# tiles per compute unit): nk = 3 and 6, an uneven number of tiles per
# workgroup, and a ragged last M-tile.
@pytest.mark.parametrize("dim,hc,mx,nh,M", [(2048, 4, 2, 3, 4096), (2048, 4, 3, 3, 4000),
                                            (1024, 4, 4, 2, 8192)])
def test_fused_persistent_shapes(ge, dev, dim, hc, mx, nh, M):
    cfg, rows = _small(dim, hc, mx, nh, rows=100000)
    g = geometry(ge, cfg, rows)
    say("fused persistent", (dim, hc, mx, nh), "M", M, "N", g.N, "K", g.K)
    table, scales = synth.embedding_table(cfg, rows, dev)
    w = synth.wkv_weight(cfg, dev)
    rng = np.random.default_rng(M + dim)
    hid = torch.from_numpy(rng.integers(0, rows, (M, g.n_hash_cols)).astype(np.int32)).to(dev)
    pos = np.unique(np.concatenate([[0, 255, 256, M - 257, M - 256, M - 1],
                                    rng.integers(0, M, 10)]))
    st = _check_against_oracle_and_two_stage(ge, g, cfg, table, scales, hid, w, sample=pos)
    say("   kv", st)


def test_fused_every_scale_code(ge, dev):
    # all 256 e8m0 codes (NaN and the subnormal 2^-127 included) on rows that
    # every position references; kv must match the two-stage path bit for bit
    cfg, rows = _small(128, 1, 2, 2, rows=256)
    g = geometry(ge, cfg, rows)
    say("fused scale codes")
    table, _ = synth.embedding_table(cfg, rows, dev)
    sc = np.stack([np.arange(256), (np.arange(256) * 7 + 3) % 256], axis=1).astype(np.uint8)
    scales = torch.from_numpy(sc).to(dev)
    w = synth.wkv_weight(cfg, dev)
    M = 1280
    hid = torch.from_numpy((np.arange(M * 2) % rows).astype(np.int32).reshape(M, 2)).to(dev)
    kv = ge.engram_wkv_gathered(g, table, scales, hid, w)
    two = ge.engram_wkv(g, ge.engram_gather(g, table, scales, hid), w)
    torch.cuda.synchronize()
    # a NaN result's sign and payload are unspecified: NaN-ness must agree,
    # everything else bit for bit
    nan_f, nan_t = torch.isnan(kv), torch.isnan(two)
    assert torch.equal(nan_f, nan_t)
    assert int(nan_f.sum()) > 0 and int((~nan_f).sum()) > 0
    assert torch.equal(kv.view(torch.int16)[~nan_f], two.view(torch.int16)[~nan_t])


# both row forms: decode-sized batches (table rows at offsets) and larger
# ones (rows copied per hash column)
@pytest.mark.parametrize("M", [100, 1100])
def test_fused_bad_ids_read_zero_rows(ge, dev, M):
    cfg, rows = _small(256, 3, 3, 1, rows=3000)
    g = geometry(ge, cfg, rows)
    say("fused bad ids M", M)
    table, scales = synth.embedding_table(cfg, rows, dev)
    w = synth.wkv_weight(cfg, dev)
    rng = np.random.default_rng(5)
    h = rng.integers(0, rows, (M, g.n_hash_cols)).astype(np.int32)
    h[3, 0], h[M // 2, 1], h[M - 1, 0] = -1, rows, 1 << 30
    hid = torch.from_numpy(h).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv = ge.engram_wkv_gathered(g, table, scales, hid, w, err=err)
    two = ge.engram_wkv(g, ge.engram_gather(g, table, scales, hid), w)
    torch.cuda.synchronize()
    assert int(err.item()) & ge.ERRBIT_ROW
    assert torch.equal(kv.view(torch.int16), two.view(torch.int16))


def test_fused_unsupported_head_dim(ge, dev):
    tiny = synth.config("tiny")  # head_dim 32
    g = geometry(ge, tiny, 100)
    hid = torch.zeros((4, g.n_hash_cols), dtype=torch.int32, device=dev)
    with pytest.raises(ge.EngramError):
        ge.engram_wkv_gathered(g, torch.zeros((100, 32), dtype=torch.uint8, device=dev),
                               torch.zeros((100, 1), dtype=torch.uint8, device=dev), hid,
                               torch.zeros((g.N, g.K), dtype=torch.bfloat16, device=dev))


@pytest.fixture(scope="module")
def prefill(ge, dev):
    return Workload(ge, "prefill", dev)


@pytest.mark.parametrize("M", [4096, 2048, 1000])
def test_fused_full_size(ge, dev, prefill, M):
    # the full table (25.2 M rows) and the full 25600 x 1536 weight; hash ids
    # uniform over the table.  Whole kv against the two-stage path, sampled
    # rows (tile edges included) against the oracle.
    wl = prefill
    say("fused full M", M)
    rng = np.random.default_rng(M)
    hid = torch.from_numpy(rng.integers(0, wl.num_emb, (M, wl.g.n_hash_cols)).astype(np.int32))
    hid = hid.to(dev)
    edges = [0, 127, 128, 255, 256, M - 129, M - 128, M - 1]
    pos = np.unique(np.concatenate([[e for e in edges if 0 <= e < M],
                                    rng.integers(0, M, 8)]))
    st = _check_against_oracle_and_two_stage(ge, wl.g, wl.cfg, wl.table, wl.scales, hid, wl.w,
                                             sample=pos)
    say("   kv", st)


# ------------------------------------------------------------------ fully fused prefill
@pytest.fixture(scope="module")
def gp_case(ge, dev):
    # dim 2048, hc 4, 6 hash columns, M = 4096: 640 tiles of 256x256, the
    # persistent kernel with every key column reduced in its epilogue
    cfg, rows = _small(2048, 4, 3, 3, rows=200000)
    g = geometry(ge, cfg, rows)
    M = 4096
    assert ge.engram_gate_partials_supported(g, M)
    table, scales = synth.embedding_table(cfg, rows, dev)
    w = synth.wkv_weight(cfg, dev)
    q, k = synth.qk_weights(cfg, dev)
    x = synth.activations(cfg, M, dev).reshape(M, cfg.hc_mult, cfg.dim)
    rng = np.random.default_rng(77)
    hid = torch.from_numpy(rng.integers(0, rows, (M, g.n_hash_cols)).astype(np.int32)).to(dev)
    kv = ge.engram_wkv_gathered(g, table, scales, hid, w)
    v, part = ge.engram_wkv_gate_partials(g, table, scales, hid, w, x, q, k)
    torch.cuda.synchronize()
    return dict(cfg=cfg, g=g, M=M, q=q, k=k, x=x, kv=kv, v=v, part=part)


def test_gate_partials_value_and_sums(ge, dev, gp_case):
    c = gp_case
    g, M, cfg = c["g"], c["M"], c["cfg"]
    hd = cfg.hc_mult * cfg.dim
    say("gate partials: value columns bit for bit")
    assert torch.equal(c["v"].view(torch.int16), c["kv"][:, hd:].contiguous().view(torch.int16))
    say("gate partials: sums against fp64 over the stored keys")
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(3).integers(0, M, 28)]))
    key = tolerances.bf16_value(bits(c["kv"][torch.from_numpy(rows).to(dev)][:, :hd]))
    key = key.reshape(len(rows), cfg.hc_mult, cfg.dim // 128, 128)
    h = tolerances.bf16_value(bits(c["x"][torch.from_numpy(rows).to(dev)]))
    h = h.reshape(key.shape)
    wq = (tolerances.bf16_value(bits(c["q"])) * tolerances.bf16_value(bits(c["k"])))
    wq = wq.reshape(1, cfg.hc_mult, cfg.dim // 128, 128)
    t_kk = key * key
    t_hwk = (h * wq) * key
    ref = np.stack([t_kk.sum(-1), t_hwk.sum(-1)], -1)
    bound = 128 * 2.0 ** -23 * np.stack([np.abs(t_kk).sum(-1), np.abs(t_hwk).sum(-1)], -1) + 1e-30
    got = c["part"][torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= bound), "partial sums off by %r of the bound" % float((err / bound).max())


def test_gate_from_partials_against_oracle(ge, dev, gp_case):
    # the gate from the partial sums against the oracle's gate_and_add on the
    # same kv (the GPU's), with a mask
    c = gp_case
    g, M, cfg = c["g"], c["M"], c["cfg"]
    mask = torch.from_numpy((np.random.default_rng(9).random(M) > 0.25).astype(np.uint8)).to(dev)
    gate = torch.empty((M, cfg.hc_mult), dtype=torch.float32, device=dev)
    out = ge.engram_gate_from_partials(g, c["x"], c["v"], c["part"], mask=mask, gate=gate)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, M - 1], np.random.default_rng(4).integers(0, M, 40)]))
    ri = torch.from_numpy(rows).to(dev)
    xb, kvb = bits(c["x"][ri]), bits(c["kv"][ri])
    mk = mask.cpu().numpy()[rows]
    ref_out, ref_gate, ref_a = oracle.gate_and_add(xb, kvb, bits(c["q"]), bits(c["k"]),
                                                   cfg.norm_eps, mk)
    gs = tolerances.check_gate(gate.cpu().numpy()[rows], ref_gate, ref_a)
    os_ = tolerances.check_out(bits(out[ri]), ref_out, xb, kvb[:, cfg.hc_mult * cfg.dim:],
                               gate.cpu().numpy()[rows], ref_gate)
    say("   gate", gs, "out", os_)


# ------------------------------------------------------------------ forward = its stages
# The forward hashes straight into the fused projections' row offsets and
# scales.  It must give the same out, gate, state and error bits, bit for bit,
# as the stage calls it stands for, also with bad token ids (flagged, read as
# the pad id) and a hash column whose slots all fall past the table (flagged,
# its rows read as zeros).  Cases: the 64-wide fused tiles (n_tok <= 256), the
# 256-wide fused tiles (300, 700 and 1100 positions), and the fully fused path
# with the gate's sums in the projection.
FWD_CASES = [((256, 3, 3, 2), 1, 37), ((256, 3, 3, 2), 3, 100), ((256, 3, 3, 2), 1, 1100),
             ((256, 3, 3, 2), 2, 350),
             ((2048, 4, 3, 3), 1, 4096), ((256, 3, 3, 2), 5, 1), ((256, 3, 5, 2), 3, 2)]


@pytest.mark.parametrize("shape,B,T", FWD_CASES)
def test_forward_equals_stage_calls(ge, dev, shape, B, T):
    dim, hc, mx, nh = shape
    cfg = dataclasses.replace(synth.config("tiny"), dim=dim, hc_mult=hc, max_ngram_size=mx,
                              n_heads=nh, head_dim=64, scale_codes=(120, 132))
    wl = Workload(ge, cfg, dev)
    g = wl.g
    n = B * T
    say("forward vs stages", shape, "B", B, "T", T)
    t = dict(wl.t)
    t["offset"] = t["offset"].copy()
    t["offset"][1] += np.uint64(wl.num_emb)          # column 1: every slot past the table
    tables = {k2: torch.from_numpy(np.ascontiguousarray(t[k2])).to(dev)
              for k2 in ("token_map", "mult", "prime", "offset")}
    ids_np = synth.token_ids(cfg, B, T, name="fs")
    ids_np[0, min(5, T - 1)] = cfg.vocab + 7
    ids_np[-1, T // 2] = -3                           # (the same position when T = 1, B = 1)
    ids = torch.from_numpy(ids_np).to(dev)
    x = synth.activations(cfg, n, dev, name="fsx").reshape(B, T, hc, dim)
    mask = torch.from_numpy(synth.token_ids(cfg, B, T, name="fsm") % 4 != 0).to(dev)
    st0 = torch.from_numpy(synth.token_ids(cfg, B, mx - 1, name="fss") % 500).to(dev)

    state_a, err_a = st0.clone(), torch.zeros(1, dtype=torch.int32, device=dev)
    gate_a = torch.empty((B, T, hc), dtype=torch.float32, device=dev)
    out_a = ge.engram_forward(g, tables, wl.table, wl.scales, wl.w, wl.q, wl.k, x, ids, mask=mask,
                              state=state_a, gate=gate_a, err=err_a)

    state_b, err_b = st0.clone(), torch.zeros(1, dtype=torch.int32, device=dev)
    gate_b = torch.empty((B, T, hc), dtype=torch.float32, device=dev)
    hid = ge.engram_hash(g, tables, ids, state=state_b, err=err_b).reshape(n, -1)
    xf = x.reshape(n, hc, dim)
    if ge.engram_gate_partials_supported(g, n):
        v, part = ge.engram_wkv_gate_partials(g, wl.table, wl.scales, hid, wl.w, xf, wl.q, wl.k,
                                              err=err_b)
        out_b = ge.engram_gate_from_partials(g, xf, v, part, mask=mask.reshape(-1), gate=gate_b)
    else:
        kv = ge.engram_wkv_gathered(g, wl.table, wl.scales, hid, wl.w, err=err_b)
        out_b = ge.engram_gate_add(g, xf, kv, wl.q, wl.k, mask=mask.reshape(-1), gate=gate_b)
    torch.cuda.synchronize()
    bits_err = int(err_a.item())
    assert bits_err == int(err_b.item())
    assert bits_err & ge.ERRBIT_TOKEN and bits_err & ge.ERRBIT_HASH and bits_err & ge.ERRBIT_ROW
    assert torch.equal(state_a, state_b)
    assert torch.equal(out_a.view(torch.int16).reshape(-1), out_b.view(torch.int16).reshape(-1))
    assert torch.equal(gate_a.reshape(-1), gate_b.reshape(-1))


# ------------------------------------------------------------------ masked prefill, compacted
# Under a mask the fully fused forward projects only the live positions,
# packed in order; the projection's tiles past the live count are skipped.
# Its out, gate and state must equal, bit for bit, the dense stage calls
# (every row projected) followed by the masked gate.  Mask patterns: spans
# of 256..1024 positions (30% masked), everything masked, one live
# position, every other position, a live count that leaves most
# workgroups of the persistent kernel with no tile or one, and no position
# masked.
MASKS = ["spans", "none_live", "one_live", "alternate", "head300", "all_live"]


def _mask(kind, cfg, T):
    if kind == "spans":
        return synth.token_mask(dataclasses.replace(cfg, mask_frac=0.3), 1, T)[0]
    m = np.zeros(T, dtype=bool)
    if kind == "one_live":
        m[T // 3] = True
    elif kind == "alternate":
        m[::2] = True
    elif kind == "head300":
        m[:300] = True
    elif kind == "all_live":
        m[:] = True
    return m


# Layouts: one sequence with the mask 16-byte aligned (the hash kernel counts
# the live positions itself, 16 bytes a load), 4-byte aligned (4 bytes a
# load), or at an odd address, and two sequences with a state (those two take
# the one-workgroup scan before the hash).
@pytest.mark.parametrize("kind,T,layout", [(k, 4096, "b1") for k in MASKS] +
                         [("spans", 9000, "b1"), ("alternate", 9000, "b1"),
                          ("spans", 4096, "b2"), ("alternate", 4096, "off1"),
                          ("spans", 9000, "off4"), ("spans", 40000, "b1")])
def test_forward_masked_compaction(ge, dev, kind, T, layout):
    # T = 9000: a ragged last 256-row block; T = 40000: past the positions
    # the hash kernel counts itself
    B = 2 if layout == "b2" else 1
    Tb = T // B
    cfg = dataclasses.replace(synth.config("tiny"), dim=2048, hc_mult=4, max_ngram_size=3,
                              n_heads=3, head_dim=64, scale_codes=(120, 132), T=T)
    wl = Workload(ge, cfg, dev)
    g = wl.g
    assert ge.engram_gate_partials_supported(g, T)
    say("masked compaction", kind, T, layout)
    mask_np = _mask(kind, cfg, T)
    ids_np = synth.token_ids(cfg, 1, T, name="mc").reshape(B, Tb)
    masked = np.nonzero(~mask_np)[0]
    if len(masked):
        ids_np.reshape(-1)[masked[len(masked) // 2]] = cfg.vocab + 5   # bad token, masked position
    ids = torch.from_numpy(ids_np).to(dev)
    off = {"off1": 1, "off4": 4}.get(layout, 0)
    mbuf = torch.zeros(T + 16, dtype=torch.uint8, device=dev)
    mbuf[off:off + T] = torch.from_numpy(mask_np.astype(np.uint8)).to(dev)
    mask = mbuf[off:off + T].view(B, Tb)
    x = synth.activations(cfg, T, dev, name="mcx").reshape(B, Tb, cfg.hc_mult, cfg.dim)
    st0 = torch.from_numpy(synth.token_ids(cfg, B, 2, name="mcs") % 500).to(dev)

    state_a, err_a = st0.clone(), torch.zeros(1, dtype=torch.int32, device=dev)
    gate_a = torch.full((B, Tb, cfg.hc_mult), -1.0, dtype=torch.float32, device=dev)
    out_a = ge.engram_forward(g, wl.tables, wl.table, wl.scales, wl.w, wl.q, wl.k, x, ids,
                              mask=mask, state=state_a, gate=gate_a, err=err_a)

    state_b, err_b = st0.clone(), torch.zeros(1, dtype=torch.int32, device=dev)
    gate_b = torch.full((T, cfg.hc_mult), -1.0, dtype=torch.float32, device=dev)
    hid = ge.engram_hash(g, wl.tables, ids, state=state_b, err=err_b).reshape(T, -1)
    xf = x.reshape(T, cfg.hc_mult, cfg.dim)
    v, part = ge.engram_wkv_gate_partials(g, wl.table, wl.scales, hid, wl.w, xf, wl.q, wl.k,
                                          err=err_b)
    out_b = ge.engram_gate_from_partials(g, xf, v, part, mask=mask.reshape(-1).contiguous(),
                                         gate=gate_b)
    torch.cuda.synchronize()
    assert int(err_a.item()) == int(err_b.item()) == (ge.ERRBIT_TOKEN if len(masked) else 0)
    assert torch.equal(state_a, state_b)
    assert torch.equal(out_a.view(torch.int16).reshape(-1), out_b.view(torch.int16).reshape(-1))
    assert torch.equal(gate_a.reshape(-1), gate_b.reshape(-1))
    # masked positions: x itself and gate 0
    mk = torch.from_numpy(~mask_np).to(dev)
    assert torch.equal(out_a.reshape(T, -1)[mk].view(torch.int16),
                       x.reshape(T, -1)[mk].view(torch.int16))
    assert torch.all(gate_a.reshape(T, -1)[mk] == 0).item()


# ------------------------------------------------------------------ forward from hash ids
# The block's own signature (x, hash_ids, token_mask): the same outputs, bit
# for bit, as the forward from token ids, on every path (64-wide fused tiles,
# 256-wide fused tiles for mid-sized and larger batches, fully fused with and
# without a mask); and two layers hashed in one launch, then each layer's forward from
# its block of ids, equal to each layer's forward from token ids.
@pytest.mark.parametrize("shape,T,masked", [((256, 3, 3, 2), 37, True), ((256, 3, 3, 2), 300, True),
                                            ((256, 3, 3, 2), 1100, False),
                                            ((2048, 4, 3, 3), 4096, False),
                                            ((2048, 4, 3, 3), 4096, True)])
def test_forward_hashed_equals_forward(ge, dev, shape, T, masked):
    dim, hc, mx, nh = shape
    say("forward from hash ids", shape, T, masked)
    layers = []
    for l in range(2):
        cfg = dataclasses.replace(synth.config("tiny"), dim=dim, hc_mult=hc, max_ngram_size=mx,
                                  n_heads=nh, head_dim=64, scale_codes=(120, 132), index=300 + l)
        layers.append(Workload(ge, cfg, dev))
    cfg = layers[0].cfg
    ids = torch.from_numpy(synth.token_ids(cfg, 1, T, name="fh")).to(dev)
    x = synth.activations(cfg, T, dev, name="fhx").reshape(1, T, hc, dim)
    mask = None
    if masked:
        mask = torch.from_numpy(synth.token_ids(cfg, 1, T, name="fhm") % 3 != 0).to(dev)
    hid_all = ge.engram_hash_layers([w.g for w in layers], [w.tables for w in layers], ids)
    for l, wl in enumerate(layers):
        gate_a = torch.empty((1, T, hc), dtype=torch.float32, device=dev)
        gate_b = torch.empty_like(gate_a)
        err_a = torch.zeros(1, dtype=torch.int32, device=dev)
        err_b = torch.zeros(1, dtype=torch.int32, device=dev)
        out_a = ge.engram_forward(wl.g, wl.tables, wl.table, wl.scales, wl.w, wl.q, wl.k, x, ids,
                                  mask=mask, gate=gate_a, err=err_a)
        out_b = ge.engram_forward_hashed(wl.g, wl.table, wl.scales, wl.w, wl.q, wl.k, x,
                                         hid_all[l], mask=mask, gate=gate_b, err=err_b)
        torch.cuda.synchronize()
        assert int(err_a.item()) == int(err_b.item()) == 0
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), l
        assert torch.equal(gate_a, gate_b), l
