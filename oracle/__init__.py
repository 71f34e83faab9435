"""CPU oracle for the Engram forward path -- TEST INFRASTRUCTURE ONLY.

Plain fp64 C (``engram_oracle.c``) behind a thin ctypes wrapper taking numpy
arrays.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
use this package; the HIP library never imports, links or calls it.

Each function follows the pages it cites in ``engram_oracle.c``:
  e4m3 / e8m0 codecs ........ "Module engram" docs, Functions
  hash ...................... "Module engram" docs, stage 1 and NgramHashState
  embed_rows ................ "Module engram" docs, stage 2 / embed_rows / regen_table
  linear .................... "Module engram" docs, stage 3 / linear_bf16
  gate_and_add .............. Engram block `forward`; "Gate per stream" equations
bf16 tensors travel as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "engram_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BAD_TOKEN, BAD_HASH, HISTORY_FULL, BAD_ID = 1, 2, 3, 4


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i64, i32 = C.c_int64, C.c_int32
        L.eo_num_threads.restype = C.c_int
        L.eo_set_num_threads.restype = None
        L.eo_set_num_threads.argtypes = [C.c_int]
        L.eo_bf16_value.restype = C.c_double
        L.eo_bf16_value.argtypes = [C.c_uint16]
        L.eo_bf16_round.restype = C.c_uint16
        L.eo_bf16_round.argtypes = [C.c_double]
        L.eo_e4m3_decode.restype = C.c_double
        L.eo_e4m3_decode.argtypes = [C.c_uint]
        L.eo_e4m3_encode.restype = C.c_uint
        L.eo_e4m3_encode.argtypes = [C.c_float]
        L.eo_e8m0_decode.restype = C.c_double
        L.eo_e8m0_decode.argtypes = [C.c_uint]
        L.eo_e8m0_encode.restype = C.c_uint
        L.eo_e8m0_encode.argtypes = [C.c_float]
        for nm in ("eo_e4m3_decode_n", "eo_e4m3_encode_n", "eo_e8m0_encode_n", "eo_bf16_round_n"):
            getattr(L, nm).argtypes = [P, i64, P]
            getattr(L, nm).restype = None
        L.eo_hash.restype = C.c_int
        L.eo_hash.argtypes = [C.c_int, C.c_int, i32, i64, P, P, P, P, C.c_int, i64, P,
                              P, i64, P, P]
        L.eo_embed_rows.restype = C.c_int
        L.eo_embed_rows.argtypes = [C.c_int, i64, P, P, P, i64, P]
        L.eo_linear.restype = None
        L.eo_linear.argtypes = [i64, i64, i64, P, P, P]
        L.eo_gate_and_add.restype = None
        L.eo_gate_and_add.argtypes = [i64, C.c_int, C.c_int, C.c_float, P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().eo_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only)."""
    lib().eo_set_num_threads(int(n))


# ------------------------------------------------------------------ codecs
def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().eo_e4m3_decode_n(_p(c), c.size, _p(out))
    return out


def e4m3_encode(values) -> np.ndarray:
    v = _c(values, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().eo_e4m3_encode_n(_p(v), v.size, _p(out))
    return out


def e8m0_decode(code: int) -> float:
    return lib().eo_e8m0_decode(int(code))


def e8m0_encode(values) -> np.ndarray:
    v = _c(values, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().eo_e8m0_encode_n(_p(v), v.size, _p(out))
    return out


def bf16_round(values) -> np.ndarray:
    v = _c(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().eo_bf16_round_n(_p(v), v.size, _p(out))
    return out


def bf16_value(bits) -> np.ndarray:
    b = _c(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ stage 1: hash
class HashState:
    """The page's NgramHashState: every compressed id seen, per sequence."""

    def __init__(self, B: int, capacity: int):
        self.hist = np.zeros((B, capacity), np.int32)
        self.length = np.zeros(B, np.int64)

    @property
    def B(self) -> int:
        return self.hist.shape[0]


def hash_ids(tables: dict, geom: dict, state: HashState, ids) -> np.ndarray:
    """ids int32 [B, T] -> hash_ids int32 [B, T, n_cols]; appends to `state`."""
    L = lib()
    ids = _c(ids, np.int32)
    B, T = ids.shape
    assert B == state.B
    n_cols = (geom["max_ngram_size"] - 1) * geom["n_heads"]
    out = np.empty((B, T, n_cols), np.int32)
    tm = _c(tables["token_map"], np.int32)
    mult = _c(tables["mult"], np.uint64)
    prime = _c(tables["prime"], np.uint64)
    offset = _c(tables["offset"], np.uint64)
    rc = L.eo_hash(geom["max_ngram_size"], geom["n_heads"], geom["pad_id"], geom["vocab"],
                   _p(tm), _p(mult), _p(prime), _p(offset), B, T, _p(ids),
                   _p(state.hist), state.hist.shape[1], _p(state.length), _p(out))
    if rc != 0:
        raise ValueError("oracle hash failed with code %d" % rc)
    return out


# ------------------------------------------------------------------ stage 2: rows
def embed_rows(table, scales, ids) -> np.ndarray:
    """table uint8 [rows, hd], scales uint8 [rows, hd/32], ids int32 [...] ->
    bf16 bits uint16 [..., hd]."""
    t = _c(table, np.uint8)
    s = _c(scales, np.uint8)
    i = _c(ids, np.int32)
    rows, hd = t.shape
    assert s.shape == (rows, hd // 32)
    out = np.empty(i.shape + (hd,), np.uint16)
    rc = lib().eo_embed_rows(hd, rows, _p(t), _p(s), _p(i), i.size, _p(out))
    if rc != 0:
        raise ValueError("oracle embed_rows failed with code %d" % rc)
    return out


# ------------------------------------------------------------------ stage 3: wkv
def linear(a, w) -> np.ndarray:
    """a bf16 bits [M, K], w bf16 bits [N, K] -> bf16 bits [M, N]."""
    a = _c(a, np.uint16)
    w = _c(w, np.uint16)
    M, K = a.shape
    N, K2 = w.shape
    assert K == K2
    out = np.empty((M, N), np.uint16)
    lib().eo_linear(M, N, K, _p(a), _p(w), _p(out))
    return out


# ------------------------------------------------------------------ stage 4: gate
def gate_and_add(x, kv, q, k, eps: float, mask=None):
    """x bf16 bits [tok, hc, dim], kv [tok, dim*(hc+1)], q/k [hc, dim], mask bool/uint8 [tok]
    -> (out bf16 bits [tok, hc, dim], gate fp32 [tok, hc], a fp64 [tok, hc])."""
    x = _c(x, np.uint16)
    kv = _c(kv, np.uint16)
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    n_tok, hc, dim = x.shape
    assert kv.shape == (n_tok, dim * (hc + 1)) and q.shape == (hc, dim) and k.shape == (hc, dim)
    m = None if mask is None else _c(mask, np.uint8).reshape(-1)
    out = np.empty_like(x)
    gate = np.empty((n_tok, hc), np.float32)
    a = np.empty((n_tok, hc), np.float64)
    lib().eo_gate_and_add(n_tok, hc, dim, float(eps), _p(x), _p(kv), _p(q), _p(k), _p(m),
                          _p(out), _p(gate), _p(a))
    return out, gate, a


# ------------------------------------------------------------------ whole path
def forward(tables: dict, geom: dict, state: HashState, ids, table, scales, w, q, k, x,
            mask=None) -> dict:
    """All four stages in order: hash -> rows -> wkv -> gate_and_add."""
    hid = hash_ids(tables, geom, state, ids)
    B, T, nc = hid.shape
    rows = embed_rows(table, scales, hid.reshape(B * T, nc))
    a = rows.reshape(B * T, nc * table.shape[1])
    kv = linear(a, w)
    xx = np.asarray(x).reshape(B * T, geom["hc_mult"], geom["dim"])
    m = None if mask is None else np.asarray(mask).reshape(B * T)
    out, gate, av = gate_and_add(xx, kv, q, k, geom["norm_eps"], m)
    return dict(hash_ids=hid, rows=a, kv=kv, out=out, gate=gate, a=av)
