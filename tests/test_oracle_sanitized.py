"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and run through all four stages on the tiny workload
and on a ragged variant of it (masked positions, several sequences, a 64-wide
table row, unit and non-unit scales).  Every buffer the driver hands the
oracle has exactly the size the stage reads, so a read or write past any of
them, an uninitialised history slot, a signed overflow or an out-of-range
shift aborts the run.  The sanitized build must also write exactly what the
normal build computes."""
import dataclasses
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("eo_san")
    exe = str(d / "eo_sanitized")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wno-unknown-pragmas",
                           os.path.join(ROOT, "oracle", "engram_oracle.c"),
                           os.path.join(HERE, "oracle_sanitize_main.c"), "-lm", "-o", exe])
    return exe


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("variant", ["tiny", "ragged"])
def test_oracle_under_sanitizers(sanitized, tmp_path, variant):
    cfg = synth.config("tiny")
    B, T = cfg.B, cfg.T
    if variant == "ragged":
        cfg = dataclasses.replace(cfg, head_dim=64, n_heads=3, scale_codes=(120, 134))
        B, T = 3, 11
    t = synth.hash_tables(cfg)
    rows = t["num_embeddings"]
    geom = synth.geometry_dict(cfg, rows)
    ids = synth.token_ids(cfg, B, T)
    table, scales = synth.embedding_table(cfg, rows, "cpu")
    w = synth.wkv_weight(cfg, "cpu")
    q, k = synth.qk_weights(cfg, "cpu")
    x = synth.activations(cfg, B * T, "cpu")
    mask = np.ones(B * T, np.uint8)
    if variant == "ragged":
        mask[[1, 5, 6, 20]] = 0
    d = str(tmp_path)
    with open(os.path.join(d, "geom.txt"), "w") as f:
        f.write("%d %d %d %d %d %d %d %d %.9g %d %d\n" % (
            cfg.dim, cfg.hc_mult, cfg.max_ngram_size, cfg.n_heads, cfg.head_dim, cfg.vocab,
            cfg.pad_id, rows, cfg.norm_eps, B, T))
    files = dict(token_map=t["token_map"].astype(np.int32), mult=t["mult"].astype(np.uint64),
                 prime=t["prime"].astype(np.uint64), offset=t["offset"].astype(np.uint64),
                 ids=ids.astype(np.int32), table=table.numpy(), scales=scales.numpy(),
                 w=_bits(w), q=_bits(q), k=_bits(k), x=_bits(x), mask=mask)
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(os.path.join(d, name + ".bin"))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    r = subprocess.run([sanitized, d], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, "sanitized oracle failed (%d):\n%s" % (r.returncode, r.stderr[-4000:])
    assert "runtime error" not in r.stderr, r.stderr[-4000:]

    ref = oracle.forward(t, geom, oracle.HashState(B, T + 4), ids, table.numpy(), scales.numpy(),
                         _bits(w), _bits(q), _bits(k), _bits(x), mask.astype(bool))
    n = B * T
    n_cols = synth.n_hash_cols(cfg)
    got = lambda nm, dt: np.fromfile(os.path.join(d, "out_%s.bin" % nm), dt)
    assert np.array_equal(got("hash", np.int32), ref["hash_ids"].reshape(-1))
    assert np.array_equal(got("rows", np.uint16), ref["rows"].reshape(-1))
    assert np.array_equal(got("kv", np.uint16), ref["kv"].reshape(-1))
    assert np.array_equal(got("out", np.uint16), ref["out"].reshape(-1))
    assert np.array_equal(got("gate", np.float32), ref["gate"].reshape(-1))
    assert got("hash", np.int32).size == n * n_cols
