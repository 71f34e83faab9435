"""Pins for the oracle's n-gram hash (stage 1 of the "Module engram" docs).

Each part of the definition is isolated by a multiplier choice that reduces the
hash to a closed form: which lookback a multiplier belongs to, the XOR fold,
wrapping 64-bit products, the unsigned modulus, the per-column prime and
offset, the size-major column order, the pad before position 0 and the
token_map compression.  Invariants cover the rest: range, prefill/decode split
invariance (the NgramHashState cache) and locality of the window.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth

U64 = np.uint64


def geom(max_ngram=3, n_heads=2, vocab=6, pad=0):
    return dict(max_ngram_size=max_ngram, n_heads=n_heads, vocab=vocab, pad_id=pad,
                dim=8, hc_mult=1, head_dim=32, norm_eps=0.0, num_embeddings=0)


def tables(token_map, mult, prime, offset):
    return dict(token_map=np.asarray(token_map, np.int32), mult=np.asarray(mult, U64),
                prime=np.asarray(prime, U64), offset=np.asarray(offset, U64))


def run(g, t, ids, cap=64):
    ids = np.atleast_2d(np.asarray(ids, np.int32))
    st = oracle.HashState(ids.shape[0], cap)
    return oracle.hash_ids(t, g, st, ids)


# --------------------------------------------------------------- closed forms
def test_single_lookback_multipliers_select_that_token():
    g = geom(max_ngram=3, n_heads=1, vocab=10, pad=7)
    tm = np.arange(10) * 3 + 1          # compressed ids 1, 4, 7, ...
    prime = [1_000_003, 999_983]
    offset = [5, 17]
    seq = [2, 9, 0, 5, 5]
    c = [int(tm[s]) for s in seq]
    for k in range(3):
        m = np.zeros((2, 3), U64)
        m[:, k] = 1
        h = run(g, tables(tm, m, prime, offset), seq)[0]
        for t in range(len(seq)):
            ck = c[t - k] if t - k >= 0 else 7      # pad id, used as is
            # column 0 is the size-2 column: it only sees lookbacks 0 and 1
            exp0 = (ck if k < 2 else 0) % prime[0] + offset[0]
            exp1 = ck % prime[1] + offset[1]
            assert h[t, 0] == exp0 and h[t, 1] == exp1, (k, t)


def test_xor_fold_not_sum():
    g = geom(max_ngram=2, n_heads=1, vocab=16)
    tm = np.arange(16)                   # identity compression
    m = np.array([[1, 1]], U64)
    prime, offset = [65521], [0]
    # equal tokens cancel under XOR
    h = run(g, tables(tm, m, prime, offset), [5, 5, 5])[0]
    assert h[1, 0] == 0 and h[2, 0] == 0
    assert h[0, 0] == 5                  # 5 ^ pad(0)
    # 3 ^ 5 = 6 (a sum would give 8)
    h = run(g, tables(tm, m, prime, offset), [3, 5])[0]
    assert h[1, 0] == 6
    # the same multiplier on both lookbacks cancels whatever it is
    m2 = np.array([[0x9E3779B97F4A7C15, 0x9E3779B97F4A7C15]], U64)
    h = run(g, tables(tm, m2, prime, offset), [11, 11])[0]
    assert h[1, 0] == 0


def test_products_wrap_mod_2_64_and_modulus_is_unsigned():
    g = geom(max_ngram=2, n_heads=1, vocab=4)
    tm = [0, 1, 2, 3]
    p = 997
    # 2 * (2^63 + 1) = 2^64 + 2 -> wraps to 2
    h = run(g, tables(tm, [[(1 << 63) + 1, 0]], [p], [0]), [2])[0]
    assert h[0, 0] == 2
    # 1 * (2^64 - 1): top bit set; unsigned modulus of 2^64-1
    h = run(g, tables(tm, [[(1 << 64) - 1, 0]], [p], [0]), [1])[0]
    assert h[0, 0] == ((1 << 64) - 1) % p
    # 3 * (2^64 - 1) = 2^64*3 - 3 -> wraps to 2^64 - 3
    h = run(g, tables(tm, [[(1 << 64) - 1, 0]], [p], [0]), [3])[0]
    assert h[0, 0] == ((1 << 64) - 3) % p


def test_offset_and_prime_per_column_in_size_major_order():
    g = geom(max_ngram=3, n_heads=2, vocab=8)
    tm = np.arange(8) + 100
    m = np.zeros((4, 3), U64)
    m[:, 2] = 1                          # only lookback 2 (the oldest of a 3-gram)
    prime = [11, 13, 17, 19]
    offset = [0, 11, 24, 41]
    seq = [1, 2, 3, 4]
    h = run(g, tables(tm, m, prime, offset), seq)[0]
    for t in range(4):
        c2 = tm[seq[t - 2]] if t >= 2 else 0
        # columns 0, 1 are n = 2 (lookbacks 0..1): mix = 0 -> the offset
        assert h[t, 0] == 0 and h[t, 1] == 11
        # columns 2, 3 are n = 3 heads 0 and 1
        assert h[t, 2] == c2 % 17 + 24 and h[t, 3] == c2 % 19 + 41


def test_pad_is_a_compressed_id_not_mapped():
    g = geom(max_ngram=2, n_heads=1, vocab=5, pad=3)
    tm = [4, 4, 4, 4, 4]                 # every raw id compresses to 4
    h = run(g, tables(tm, [[0, 1]], [101], [0]), [0, 1])[0]
    assert h[0, 0] == 3                  # pad id itself, not token_map[3]
    assert h[1, 0] == 4


# --------------------------------------------------------------- invariants
def _tiny_tables():
    cfg = synth.config("tiny")
    return cfg, synth.hash_tables(cfg), synth.geometry_dict(cfg, 3948)


def test_range_and_counts_on_tiny_workload():
    cfg, t, g = _tiny_tables()
    assert t["prime"].tolist() == [997, 991, 983, 977]
    assert t["offset"].tolist() == [0, 997, 1988, 2971]
    assert t["num_embeddings"] == 3948
    ids = synth.token_ids(cfg, 4, 200)
    st = oracle.HashState(4, 256)
    h = oracle.hash_ids(t, g, st, ids)
    assert h.shape == (4, 200, 4)
    lo = t["offset"].astype(np.int64)
    hi = lo + t["prime"].astype(np.int64)
    assert np.all(h >= lo) and np.all(h < hi)


def test_prefill_decode_split_invariance():
    cfg, t, g = _tiny_tables()
    ids = synth.token_ids(cfg, 3, 24, name="split")
    full = oracle.hash_ids(t, g, oracle.HashState(3, 64), ids)
    for k in range(0, 25):
        st = oracle.HashState(3, 64)
        parts = [oracle.hash_ids(t, g, st, ids[:, :k])] if k else []
        for s in range(k, 24):
            parts.append(oracle.hash_ids(t, g, st, ids[:, s:s + 1]))
        assert np.array_equal(np.concatenate(parts, axis=1), full), k


def test_token_map_invariance():
    cfg, t, g = _tiny_tables()
    tm = t["token_map"]
    # two raw ids with the same compressed id hash identically in any context
    vals, first = np.unique(tm, return_index=True)
    dup = [i for i in range(len(tm)) if i not in set(first.tolist())][:20]
    ids = synth.token_ids(cfg, 1, 40, name="tm")
    base = oracle.hash_ids(t, g, oracle.HashState(1, 64), ids)
    for d in dup:
        twin = int(first[np.searchsorted(vals, tm[d])])
        a = ids.copy()
        a[0, 10] = d
        b = ids.copy()
        b[0, 10] = twin
        ha = oracle.hash_ids(t, g, oracle.HashState(1, 64), a)
        hb = oracle.hash_ids(t, g, oracle.HashState(1, 64), b)
        assert np.array_equal(ha, hb)
        # positions outside the window of position 10 are untouched
        assert np.array_equal(ha[0, :10], base[0, :10]) and np.array_equal(ha[0, 13:], base[0, 13:])


def test_window_locality_brute_force():
    # vocab of 6 raw ids compressed onto 3; all 6^4 sequences of length 4.
    # The size-n column at position t depends only on the last n compressed ids:
    # it equals the same column at the last position of the suffix of length n
    # (and a suffix shorter than n sees pad ids, like position n-2 of a fresh
    # sequence).
    g = geom(max_ngram=3, n_heads=2, vocab=6)
    rng = np.random.default_rng(11)
    tm = np.array([0, 1, 2, 0, 1, 2], np.int32)
    mult = (rng.integers(0, 1 << 63, (4, 3), dtype=np.uint64) << U64(1)) | U64(1)
    t = tables(tm, mult, [997, 991, 983, 977], [0, 997, 1988, 2971])
    seqs = np.array(list(itertools.product(range(6), repeat=4)), np.int32)
    h = oracle.hash_ids(t, g, oracle.HashState(len(seqs), 8), seqs)
    h2 = oracle.hash_ids(t, g, oracle.HashState(len(seqs), 8), seqs[:, 2:])
    h3 = oracle.hash_ids(t, g, oracle.HashState(len(seqs), 8), seqs[:, 1:])
    assert np.array_equal(h[:, 3, :2], h2[:, 1, :2])   # n = 2 columns
    assert np.array_equal(h[:, 3, 2:], h3[:, 2, 2:])   # n = 3 columns
    # compressed-equal sequences collide; the distinct compressed 4-grams
    # (3^4 = 81 of them) give the distinct hash rows
    comp = tm[seqs]
    key = comp @ np.array([27, 9, 3, 1])
    for kval in np.unique(key)[:10]:
        rows = h[key == kval]
        assert np.all(rows == rows[0])


def test_bad_token_is_reported():
    g = geom(max_ngram=2, n_heads=1, vocab=4)
    t = tables([0, 1, 2, 3], [[1, 1]], [7], [0])
    with pytest.raises(ValueError):
        run(g, t, [1, 4])
    with pytest.raises(ValueError):
        run(g, t, [-1])
