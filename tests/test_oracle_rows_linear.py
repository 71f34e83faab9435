"""Pins for the oracle's row gather (stage 2) and wkv projection (stage 3).

Rows: torch's own fp8 / e8m0 casts, fp32 multiply and bf16 cast (library
routines) over every (value code, scale code) pair; unit scales reduce the
stage to the e4m3 decode ("Module engram" docs, stage 2 and embed_rows).
Linear: one-hot rows and small integers make every accumulation order exact,
so the expected values are integer matmuls from numpy; random inputs are
checked against numpy's fp64 BLAS.
"""
import numpy as np
import torch

import oracle


def _torch_dequant(codes, scode):
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    s = torch.from_numpy(scode).view(torch.float8_e8m0fnu).float()
    return (v * s).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_rows_all_pairs_exhaustive():
    # the full 256 x 256 (value code, scale code) space, one pair per element:
    # sorted by scale code, each 32-block holds one scale and 32 value codes
    vc, sc = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    order = np.lexsort((vc.reshape(-1), sc.reshape(-1)))
    table = vc.reshape(-1)[order].reshape(-1, 64).astype(np.uint8)
    sflat = sc.reshape(-1)[order].astype(np.uint8)
    scales = sflat.reshape(-1, 32)[:, 0].reshape(-1, 2)
    assert np.all(sflat.reshape(-1, 32) == sflat.reshape(-1, 32)[:, :1])
    ids = np.arange(table.shape[0], dtype=np.int32)
    ours = oracle.embed_rows(table, scales, ids)
    ref = _torch_dequant(table, sflat.reshape(table.shape))
    nan = np.isnan(oracle.bf16_value(ref))
    assert np.array_equal(np.isnan(oracle.bf16_value(ours)), nan)
    assert np.all(ours[nan] == 0x7FC0)            # canonical NaN
    assert np.array_equal(ours[~nan], ref[~nan])  # bit-exact, signed zeros too


def test_unit_scales_give_e4m3_values_and_gather_by_id():
    rng = np.random.default_rng(5)
    table = rng.integers(0, 256, (50, 32), dtype=np.uint8)
    table[table == 0x7F] = 0
    table[table == 0xFF] = 0
    scales = np.full((50, 1), 127, np.uint8)
    ids = rng.integers(0, 50, 37).astype(np.int32)
    out = oracle.embed_rows(table, scales, ids)
    expect = torch.from_numpy(table[ids]).view(torch.float8_e4m3fn).to(torch.bfloat16)
    assert np.array_equal(out, expect.view(torch.int16).numpy().view(np.uint16))


def test_linear_one_hot_rows_pick_weight_columns():
    rng = np.random.default_rng(1)
    K, N = 48, 40
    w = torch.randn(N, K).to(torch.bfloat16)
    wb = w.view(torch.int16).numpy().view(np.uint16)
    a = np.zeros((K, K), np.float32)
    np.fill_diagonal(a, 1.0)
    a[3, 3] = -2.0
    ab = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = oracle.linear(ab, wb)
    expect = (torch.from_numpy(a) @ w.float().T).to(torch.bfloat16)
    assert np.array_equal(out, expect.view(torch.int16).numpy().view(np.uint16))
    # row m of the output is weight column m: the weight is [out, in]
    assert np.array_equal(out[5], wb[:, 5])


def test_linear_small_integers_exact():
    rng = np.random.default_rng(2)
    M, N, K = 17, 33, 128
    a = rng.integers(-8, 9, (M, K))
    w = rng.integers(-8, 9, (N, K))
    exact = a @ w.T                      # int64, exact
    ab = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wb = torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = oracle.linear(ab, wb)
    # |exact| <= 8192 is an exact fp32; one bf16 rounding of it
    expect = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(out, expect.view(torch.int16).numpy().view(np.uint16))


def test_linear_random_against_blas():
    g = torch.Generator().manual_seed(9)
    M, N, K = 64, 96, 1536
    a = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, generator=g) * K ** -0.5).to(torch.bfloat16)
    out = oracle.linear(a.view(torch.int16).numpy().view(np.uint16),
                        w.view(torch.int16).numpy().view(np.uint16))
    exact = a.double().numpy() @ w.double().numpy().T
    ref = oracle.bf16_round(exact)
    # fp64 sums in two different orders: equal unless the exact value sits
    # within ~1e-13 relative of a bf16 rounding boundary
    assert np.mean(out == ref) > 0.9999
    diff = np.abs(out.astype(np.int64) - ref.astype(np.int64))
    assert diff.max() <= 1
