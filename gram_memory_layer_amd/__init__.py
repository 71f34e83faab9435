"""Python binding for libengram, the Engram forward path on MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libengram.so``.  PyTorch provides device memory and the current stream;
the functions below check dtypes, devices and shapes, pass raw device
pointers through the C ABI declared in ``include/engram.h`` and raise
``EngramError`` on a non-zero status.  There is no CPU fallback: if the
library is not built, every call raises.

Functions carry the C names:
    engram_hash, engram_gather, engram_wkv, engram_wkv_gathered, engram_gate_add,
    engram_forward, engram_forward_workspace_size, engram_wkv_gathered_scratch_size,
    engram_gate_partials_supported, engram_wkv_gate_partials, engram_gate_from_partials,
    engram_check_geometry
plus ``Geometry`` / ``HashTables`` (the C structs) and ``EngramLayer``, a
holder for one layer's device tables, weights and workspace.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "Geometry", "HashTables", "EngramError", "EngramLayer", "load", "library_path",
    "engram_check_geometry", "engram_hash", "engram_hash_layers", "engram_gather", "engram_wkv",
    "engram_wkv_gathered", "engram_wkv_gathered_scratch_size",
    "engram_gate_partials_supported", "engram_wkv_gate_partials", "engram_gate_from_partials",
    "engram_gate_add", "engram_forward", "engram_forward_hashed", "engram_forward_workspace_size",
    "ERRBIT_TOKEN", "ERRBIT_HASH", "ERRBIT_ROW",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libengram.so")

ERRBIT_TOKEN, ERRBIT_HASH, ERRBIT_ROW = 0x1, 0x2, 0x4
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported geometry",
           3: "workspace missing or too small", 4: "HIP runtime error",
           5: "call needs more than the fixed scratch array holds"}
ERR_TOO_LARGE = 5


class EngramError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (status %d)" % (fn, _STATUS.get(status, "?"), status))
        self.status = status


class Geometry(C.Structure):
    _fields_ = [("dim", C.c_int32), ("hc_mult", C.c_int32), ("max_ngram_size", C.c_int32),
                ("n_heads", C.c_int32), ("head_dim", C.c_int32), ("vocab", C.c_int32),
                ("pad_id", C.c_int32), ("reserved", C.c_int32), ("num_embeddings", C.c_int64),
                ("norm_eps", C.c_float), ("reserved2", C.c_int32)]

    @classmethod
    def make(cls, dim, hc_mult, max_ngram_size, n_heads, head_dim, num_embeddings, vocab,
             pad_id=0, norm_eps=1e-6) -> "Geometry":
        return cls(dim, hc_mult, max_ngram_size, n_heads, head_dim, vocab, pad_id, 0,
                   num_embeddings, norm_eps, 0)

    @property
    def n_hash_cols(self) -> int:
        return (self.max_ngram_size - 1) * self.n_heads

    @property
    def K(self) -> int:
        return self.n_hash_cols * self.head_dim

    @property
    def N(self) -> int:
        return self.dim * (self.hc_mult + 1)


class HashTables(C.Structure):
    _fields_ = [("token_map", C.c_void_p), ("mult", C.c_void_p), ("prime", C.c_void_p),
                ("offset", C.c_void_p)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libengram.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libengram.so is not built; run `python -m gram_memory_layer_amd.build`")
    L = C.CDLL(_LIB_PATH)
    P, G, HT = C.c_void_p, C.POINTER(Geometry), C.POINTER(HashTables)
    i32, i64 = C.c_int32, C.c_int64
    L.engram_status_string.restype = C.c_char_p
    L.engram_status_string.argtypes = [C.c_int]
    L.engram_check_geometry.restype = C.c_int
    L.engram_check_geometry.argtypes = [G]
    L.engram_hash.restype = C.c_int
    L.engram_hash.argtypes = [G, HT, P, P, i32, i32, P, P, P]
    L.engram_hash_layers.restype = C.c_int
    L.engram_hash_layers.argtypes = [G, HT, i32, P, P, i32, i32, P, P, P]
    L.engram_gather.restype = C.c_int
    L.engram_gather.argtypes = [G, P, P, P, i64, P, P, P]
    L.engram_wkv.restype = C.c_int
    L.engram_wkv.argtypes = [G, P, P, i64, P, P]
    L.engram_wkv_gathered_scratch_size.restype = C.c_size_t
    L.engram_wkv_gathered_scratch_size.argtypes = [G, i64]
    L.engram_wkv_gathered.restype = C.c_int
    L.engram_wkv_gathered.argtypes = [G, P, P, P, i64, P, P, P, C.c_size_t, P, P]
    L.engram_gate_partials_supported.restype = C.c_int
    L.engram_gate_partials_supported.argtypes = [G, i64]
    L.engram_wkv_gate_partials.restype = C.c_int
    L.engram_wkv_gate_partials.argtypes = [G, P, P, P, i64, P, P, P, P, P, P, P, C.c_size_t, P, P]
    L.engram_gate_from_partials.restype = C.c_int
    L.engram_gate_from_partials.argtypes = [G, P, P, P, P, i64, P, P, P]
    L.engram_gate_add.restype = C.c_int
    L.engram_gate_add.argtypes = [G, P, P, P, P, P, i64, P, P, P]
    L.engram_forward_hashed.restype = C.c_int
    L.engram_forward_hashed.argtypes = [G, P, P, P, P, P, P, P, P, i64, P, P, P, C.c_size_t, P, P]
    L.engram_forward_workspace_size.restype = C.c_size_t
    L.engram_forward_workspace_size.argtypes = [G, i64]
    L.engram_forward.restype = C.c_int
    L.engram_forward.argtypes = [G, HT, P, P, P, P, P, P, P, P, P, i32, i32, P, P, P, C.c_size_t,
                                 P, P]
    L.engram_fixed_scratch_bytes.restype = C.c_size_t
    L.engram_fixed_scratch_bytes.argtypes = []
    L.engram_forward_noalloc.restype = C.c_int
    L.engram_forward_noalloc.argtypes = [G, HT, P, P, P, P, P, P, P, P, P, i32, i32, P, P, P, P]
    _lib = L
    return L


# ------------------------------------------------------------------ helpers
def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor (got %s)" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    return t


def _check(fn, status):
    if status != 0:
        raise EngramError(fn, status)


def _tables(tables: dict, g: Geometry, device) -> HashTables:
    nc = g.n_hash_cols
    tm = _dev(tables["token_map"], "token_map", torch.int32, (g.vocab,), device)
    mult = _dev(tables["mult"], "mult", torch.uint64, (nc, g.max_ngram_size), device)
    prime = _dev(tables["prime"], "prime", torch.uint64, (nc,), device)
    offset = _dev(tables["offset"], "offset", torch.uint64, (nc,), device)
    return HashTables(tm.data_ptr(), mult.data_ptr(), prime.data_ptr(), offset.data_ptr())


# ------------------------------------------------------------------ C entry points
def engram_check_geometry(g: Geometry) -> int:
    return load().engram_check_geometry(C.byref(g))


def engram_forward_workspace_size(g: Geometry, n_tok: int) -> int:
    return load().engram_forward_workspace_size(C.byref(g), int(n_tok))


def engram_hash(g: Geometry, tables: dict, ids: torch.Tensor, state=None, hash_ids=None, err=None):
    """ids int32 [B, T] -> hash_ids int32 [B, T, n_hash_cols]; `state` int32
    [B, max_ngram_size-1] is read and updated in place (None = fresh)."""
    L = load()
    dev = ids.device
    _dev(ids, "ids", torch.int32, None, dev)
    if ids.dim() != 2:
        raise ValueError("ids must be [B, T]")
    B, T = ids.shape
    ht = _tables(tables, g, dev)
    if state is not None:
        _dev(state, "state", torch.int32, (B, g.max_ngram_size - 1), dev)
    if hash_ids is None:
        hash_ids = torch.empty((B, T, g.n_hash_cols), dtype=torch.int32, device=dev)
    _dev(hash_ids, "hash_ids", torch.int32, (B, T, g.n_hash_cols), dev)
    if err is not None:
        _dev(err, "err", torch.int32, (1,), dev)
    _check("engram_hash", L.engram_hash(C.byref(g), C.byref(ht), _ptr(state), ids.data_ptr(), B, T,
                                        hash_ids.data_ptr(), _ptr(err), _stream(dev)))
    return hash_ids


def engram_hash_layers(geoms, tables, ids: torch.Tensor, states=None, hash_ids=None, err=None):
    """Several layers' hashes in one launch: geoms / tables are lists (one
    per layer; only num_embeddings and the tables may differ), ids int32
    [B, T] -> hash_ids int32 [n_layers, B, T, n_hash_cols]; `states` None or a
    list of per-layer int32 [B, max_ngram_size-1] states, updated in place."""
    L = load()
    dev = ids.device
    _dev(ids, "ids", torch.int32, None, dev)
    if ids.dim() != 2:
        raise ValueError("ids must be [B, T]")
    n = len(geoms)
    if len(tables) != n or (states is not None and len(states) != n):
        raise ValueError("one geometry, table set and state per layer")
    B, T = ids.shape
    g0 = geoms[0]
    garr = (Geometry * n)(*geoms)
    tarr = (HashTables * n)(*[_tables(tables[l], geoms[l], dev) for l in range(n)])
    sarr = None
    if states is not None:
        for st in states:
            _dev(st, "state", torch.int32, (B, g0.max_ngram_size - 1), dev)
        sarr = (C.c_void_p * n)(*[st.data_ptr() for st in states])
    if hash_ids is None:
        hash_ids = torch.empty((n, B, T, g0.n_hash_cols), dtype=torch.int32, device=dev)
    _dev(hash_ids, "hash_ids", torch.int32, (n, B, T, g0.n_hash_cols), dev)
    if err is not None:
        _dev(err, "err", torch.int32, (1,), dev)
    _check("engram_hash_layers", L.engram_hash_layers(
        garr, tarr, n, sarr, ids.data_ptr(), B, T, hash_ids.data_ptr(), _ptr(err), _stream(dev)))
    return hash_ids


def engram_gather(g: Geometry, table, scales, hash_ids, rows=None, err=None):
    """table uint8 [num_embeddings, head_dim], scales uint8 [num_embeddings, head_dim/32],
    hash_ids int32 [n_tok, n_hash_cols] -> rows bf16 [n_tok, n_hash_cols*head_dim]."""
    L = load()
    dev = hash_ids.device
    _dev(table, "table", torch.uint8, (g.num_embeddings, g.head_dim), dev)
    _dev(scales, "scales", torch.uint8, (g.num_embeddings, g.head_dim // 32), dev)
    _dev(hash_ids, "hash_ids", torch.int32, None, dev)
    hid = hash_ids.reshape(-1, g.n_hash_cols)
    n_tok = hid.shape[0]
    if rows is None:
        rows = torch.empty((n_tok, g.K), dtype=torch.bfloat16, device=dev)
    _dev(rows, "rows", torch.bfloat16, (n_tok, g.K), dev)
    if err is not None:
        _dev(err, "err", torch.int32, (1,), dev)
    _check("engram_gather", L.engram_gather(C.byref(g), table.data_ptr(), scales.data_ptr(),
                                            hid.data_ptr(), n_tok, rows.data_ptr(), _ptr(err),
                                            _stream(dev)))
    return rows


def engram_wkv(g: Geometry, a, w, kv=None):
    """a bf16 [M, K], w bf16 [N, K] -> kv bf16 [M, N]."""
    L = load()
    dev = a.device
    _dev(a, "a", torch.bfloat16, None, dev)
    if a.dim() != 2 or a.shape[1] != g.K:
        raise ValueError("a must be [M, %d]" % g.K)
    M = a.shape[0]
    _dev(w, "w", torch.bfloat16, (g.N, g.K), dev)
    if kv is None:
        kv = torch.empty((M, g.N), dtype=torch.bfloat16, device=dev)
    _dev(kv, "kv", torch.bfloat16, (M, g.N), dev)
    _check("engram_wkv", L.engram_wkv(C.byref(g), a.data_ptr(), w.data_ptr(), M, kv.data_ptr(),
                                      _stream(dev)))
    return kv


def engram_wkv_gathered_scratch_size(g: Geometry, M: int) -> int:
    return load().engram_wkv_gathered_scratch_size(C.byref(g), int(M))


def engram_wkv_gathered(g: Geometry, table, scales, hash_ids, w, kv=None, scratch=None, err=None):
    """Gather + projection in one: table/scales/hash_ids as in engram_gather,
    w bf16 [N, K] -> kv bf16 [n_tok, N] (head_dim 64 only)."""
    L = load()
    dev = hash_ids.device
    _dev(table, "table", torch.uint8, (g.num_embeddings, g.head_dim), dev)
    _dev(scales, "scales", torch.uint8, (g.num_embeddings, g.head_dim // 32), dev)
    _dev(hash_ids, "hash_ids", torch.int32, None, dev)
    hid = hash_ids.reshape(-1, g.n_hash_cols)
    M = hid.shape[0]
    _dev(w, "w", torch.bfloat16, (g.N, g.K), dev)
    if kv is None:
        kv = torch.empty((M, g.N), dtype=torch.bfloat16, device=dev)
    _dev(kv, "kv", torch.bfloat16, (M, g.N), dev)
    need = engram_wkv_gathered_scratch_size(g, M)
    if scratch is None:
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(scratch, "scratch", torch.uint8, None, dev)
    if err is not None:
        _dev(err, "err", torch.int32, (1,), dev)
    _check("engram_wkv_gathered", L.engram_wkv_gathered(
        C.byref(g), table.data_ptr(), scales.data_ptr(), hid.data_ptr(), M, w.data_ptr(),
        kv.data_ptr(), scratch.data_ptr(), scratch.numel(), _ptr(err), _stream(dev)))
    return kv


def engram_gate_partials_supported(g: Geometry, M: int) -> bool:
    return bool(load().engram_gate_partials_supported(C.byref(g), int(M)))


def engram_wkv_gate_partials(g: Geometry, table, scales, hash_ids, w, x, q, k, v=None, part=None,
                             scratch=None, err=None):
    """Fused gather + projection whose key columns become the gate's partial
    sums: returns (v bf16 [n_tok, dim], part fp32 [n_tok, hc, dim/128, 2])."""
    L = load()
    dev = hash_ids.device
    _dev(table, "table", torch.uint8, (g.num_embeddings, g.head_dim), dev)
    _dev(scales, "scales", torch.uint8, (g.num_embeddings, g.head_dim // 32), dev)
    _dev(hash_ids, "hash_ids", torch.int32, None, dev)
    hid = hash_ids.reshape(-1, g.n_hash_cols)
    M = hid.shape[0]
    _dev(w, "w", torch.bfloat16, (g.N, g.K), dev)
    _dev(x, "x", torch.bfloat16, None, dev)
    if x.numel() != M * g.hc_mult * g.dim:
        raise ValueError("x must hold n_tok*hc_mult*dim values")
    _dev(q, "q", torch.bfloat16, (g.hc_mult, g.dim), dev)
    _dev(k, "k", torch.bfloat16, (g.hc_mult, g.dim), dev)
    if v is None:
        v = torch.empty((M, g.dim), dtype=torch.bfloat16, device=dev)
    _dev(v, "v", torch.bfloat16, (M, g.dim), dev)
    if part is None:
        part = torch.empty((M, g.hc_mult, g.dim // 128, 2), dtype=torch.float32, device=dev)
    _dev(part, "part", torch.float32, (M, g.hc_mult, g.dim // 128, 2), dev)
    need = engram_wkv_gathered_scratch_size(g, M)
    if scratch is None:
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(scratch, "scratch", torch.uint8, None, dev)
    if err is not None:
        _dev(err, "err", torch.int32, (1,), dev)
    _check("engram_wkv_gate_partials", L.engram_wkv_gate_partials(
        C.byref(g), table.data_ptr(), scales.data_ptr(), hid.data_ptr(), M, w.data_ptr(),
        x.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), part.data_ptr(),
        scratch.data_ptr(), scratch.numel(), _ptr(err), _stream(dev)))
    return v, part


def engram_gate_from_partials(g: Geometry, x, v, part, mask=None, out=None, gate=None):
    """x bf16 [n_tok, hc, dim] (any leading shape), v bf16 [n_tok, dim], part from
    engram_wkv_gate_partials -> out (like x); `out` may be x."""
    L = load()
    dev = x.device
    _dev(x, "x", torch.bfloat16, None, dev)
    n_tok = x.numel() // (g.hc_mult * g.dim)
    if x.numel() != n_tok * g.hc_mult * g.dim or x.shape[-1] != g.dim:
        raise ValueError("x must be [..., hc_mult, dim]")
    _dev(v, "v", torch.bfloat16, (n_tok, g.dim), dev)
    _dev(part, "part", torch.float32, (n_tok, g.hc_mult, g.dim // 128, 2), dev)
    m = _mask(mask, n_tok, dev)
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", torch.bfloat16, tuple(x.shape), dev)
    if gate is not None:
        _dev(gate, "gate", torch.float32, None, dev)
        if gate.numel() != n_tok * g.hc_mult:
            raise ValueError("gate must hold n_tok*hc_mult values")
    _check("engram_gate_from_partials", L.engram_gate_from_partials(
        C.byref(g), x.data_ptr(), v.data_ptr(), part.data_ptr(), _ptr(m), n_tok, out.data_ptr(),
        _ptr(gate), _stream(dev)))
    return out


def engram_gate_add(g: Geometry, x, kv, q, k, mask=None, out=None, gate=None):
    """x bf16 [n_tok, hc, dim] (any leading shape), kv bf16 [n_tok, dim*(hc+1)],
    q/k bf16 [hc, dim], mask bool/uint8 [n_tok] or None -> out (same shape as x);
    `out` may be x (in place); `gate` fp32 [n_tok, hc] is filled if given."""
    L = load()
    dev = x.device
    _dev(x, "x", torch.bfloat16, None, dev)
    n_tok = x.numel() // (g.hc_mult * g.dim)
    if x.numel() != n_tok * g.hc_mult * g.dim or x.shape[-1] != g.dim:
        raise ValueError("x must be [..., hc_mult, dim]")
    _dev(kv, "kv", torch.bfloat16, None, dev)
    if kv.numel() != n_tok * g.N:
        raise ValueError("kv must be [n_tok, dim*(hc_mult+1)]")
    _dev(q, "q", torch.bfloat16, (g.hc_mult, g.dim), dev)
    _dev(k, "k", torch.bfloat16, (g.hc_mult, g.dim), dev)
    m = _mask(mask, n_tok, dev)
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", torch.bfloat16, tuple(x.shape), dev)
    if gate is not None:
        _dev(gate, "gate", torch.float32, None, dev)
        if gate.numel() != n_tok * g.hc_mult:
            raise ValueError("gate must hold n_tok*hc_mult values")
    _check("engram_gate_add", L.engram_gate_add(C.byref(g), x.data_ptr(), kv.data_ptr(),
                                                q.data_ptr(), k.data_ptr(), _ptr(m), n_tok,
                                                out.data_ptr(), _ptr(gate), _stream(dev)))
    return out


def _mask(mask, n_tok, dev):
    if mask is None:
        return None
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    _dev(mask, "mask", torch.uint8, None, dev)
    if mask.numel() != n_tok:
        raise ValueError("mask must hold one value per position")
    return mask


def engram_forward(g: Geometry, tables: dict, table, scales, w, q, k, x, ids, mask=None,
                   state=None, out=None, gate=None, workspace=None, err=None):
    """The whole forward: x bf16 [B, T, hc, dim], ids int32 [B, T] -> out (like x)."""
    L = load()
    dev = x.device
    _dev(ids, "ids", torch.int32, None, dev)
    if ids.dim() != 2:
        raise ValueError("ids must be [B, T]")
    B, T = ids.shape
    _dev(x, "x", torch.bfloat16, (B, T, g.hc_mult, g.dim), dev)
    ht = _tables(tables, g, dev)
    _dev(table, "table", torch.uint8, (g.num_embeddings, g.head_dim), dev)
    _dev(scales, "scales", torch.uint8, (g.num_embeddings, g.head_dim // 32), dev)
    _dev(w, "w", torch.bfloat16, (g.N, g.K), dev)
    _dev(q, "q", torch.bfloat16, (g.hc_mult, g.dim), dev)
    _dev(k, "k", torch.bfloat16, (g.hc_mult, g.dim), dev)
    if state is not None:
        _dev(state, "state", torch.int32, (B, g.max_ngram_size - 1), dev)
    m = _mask(mask, B * T, dev)
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", torch.bfloat16, (B, T, g.hc_mult, g.dim), dev)
    if gate is not None:
        _dev(gate, "gate", torch.float32, (B, T, g.hc_mult), dev)
    need = engram_forward_workspace_size(g, B * T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8, None, dev)
    if err is not None:
        _dev(err, "err", torch.int32, (1,), dev)
    _check("engram_forward", L.engram_forward(
        C.byref(g), C.byref(ht), table.data_ptr(), scales.data_ptr(), w.data_ptr(), q.data_ptr(),
        k.data_ptr(), _ptr(state), x.data_ptr(), ids.data_ptr(), _ptr(m), B, T, out.data_ptr(),
        _ptr(gate), workspace.data_ptr(), workspace.numel(), _ptr(err), _stream(dev)))
    return out


def engram_forward_hashed(g: Geometry, table, scales, w, q, k, x, hash_ids, mask=None, out=None,
                          gate=None, workspace=None, err=None):
    """The forward from given hash ids (the block's forward signature): x bf16
    [..., hc, dim], hash_ids int32 [..., n_hash_cols] (same leading shape),
    mask bool/uint8 over the positions or None -> out (like x)."""
    L = load()
    dev = x.device
    _dev(hash_ids, "hash_ids", torch.int32, None, dev)
    n_tok = hash_ids.numel() // g.n_hash_cols
    if hash_ids.numel() != n_tok * g.n_hash_cols or hash_ids.shape[-1] != g.n_hash_cols:
        raise ValueError("hash_ids must be [..., n_hash_cols]")
    _dev(x, "x", torch.bfloat16, None, dev)
    if x.numel() != n_tok * g.hc_mult * g.dim or x.shape[-1] != g.dim:
        raise ValueError("x must be [..., hc_mult, dim] with one position per hash-id row")
    _dev(table, "table", torch.uint8, (g.num_embeddings, g.head_dim), dev)
    _dev(scales, "scales", torch.uint8, (g.num_embeddings, g.head_dim // 32), dev)
    _dev(w, "w", torch.bfloat16, (g.N, g.K), dev)
    _dev(q, "q", torch.bfloat16, (g.hc_mult, g.dim), dev)
    _dev(k, "k", torch.bfloat16, (g.hc_mult, g.dim), dev)
    m = _mask(mask, n_tok, dev)
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", torch.bfloat16, tuple(x.shape), dev)
    if gate is not None:
        _dev(gate, "gate", torch.float32, None, dev)
        if gate.numel() != n_tok * g.hc_mult:
            raise ValueError("gate must hold n_tok*hc_mult values")
    need = engram_forward_workspace_size(g, n_tok)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8, None, dev)
    if err is not None:
        _dev(err, "err", torch.int32, (1,), dev)
    _check("engram_forward_hashed", L.engram_forward_hashed(
        C.byref(g), table.data_ptr(), scales.data_ptr(), w.data_ptr(), q.data_ptr(), k.data_ptr(),
        x.data_ptr(), hash_ids.data_ptr(), _ptr(m), n_tok, out.data_ptr(), _ptr(gate),
        workspace.data_ptr(), workspace.numel(), _ptr(err), _stream(dev)))
    return out


def engram_fixed_scratch_bytes() -> int:
    """Size of the library's fixed per-GPU scratch array (engram_forward_noalloc)."""
    return int(load().engram_fixed_scratch_bytes())


def engram_forward_noalloc(g: Geometry, tables: dict, table, scales, w, q, k, x, ids, out,
                           mask=None, state=None, gate=None, err=None):
    """engram_forward with the library's fixed scratch array as its workspace:
    nothing is allocated by this call (out, and gate/err if wanted, are the
    caller's).  Raises EngramError (ENGRAM_ERR_TOO_LARGE) when the call's
    workspace would not fit the array."""
    L = load()
    dev = x.device
    _dev(ids, "ids", torch.int32, None, dev)
    if ids.dim() != 2:
        raise ValueError("ids must be [B, T]")
    B, T = ids.shape
    _dev(x, "x", torch.bfloat16, (B, T, g.hc_mult, g.dim), dev)
    ht = _tables(tables, g, dev)
    _dev(table, "table", torch.uint8, (g.num_embeddings, g.head_dim), dev)
    _dev(scales, "scales", torch.uint8, (g.num_embeddings, g.head_dim // 32), dev)
    _dev(w, "w", torch.bfloat16, (g.N, g.K), dev)
    _dev(q, "q", torch.bfloat16, (g.hc_mult, g.dim), dev)
    _dev(k, "k", torch.bfloat16, (g.hc_mult, g.dim), dev)
    if state is not None:
        _dev(state, "state", torch.int32, (B, g.max_ngram_size - 1), dev)
    m = _mask(mask, B * T, dev)
    _dev(out, "out", torch.bfloat16, (B, T, g.hc_mult, g.dim), dev)
    if gate is not None:
        _dev(gate, "gate", torch.float32, (B, T, g.hc_mult), dev)
    if err is not None:
        _dev(err, "err", torch.int32, (1,), dev)
    _check("engram_forward_noalloc", L.engram_forward_noalloc(
        C.byref(g), C.byref(ht), table.data_ptr(), scales.data_ptr(), w.data_ptr(), q.data_ptr(),
        k.data_ptr(), _ptr(state), x.data_ptr(), ids.data_ptr(), _ptr(m), B, T, out.data_ptr(),
        _ptr(gate), _ptr(err), _stream(dev)))
    return out


class EngramLayer:
    """One Engram layer's device-resident inputs: geometry, hash tables, the
    fp8 table and scales, the wkv weight and q/k weights, plus a reusable
    workspace.  `forward` is engram_forward."""

    def __init__(self, g: Geometry, tables: dict, table, scales, w, q, k):
        self.g, self.tables = g, tables
        self.table, self.scales, self.w, self.q, self.k = table, scales, w, q, k
        self._ws = None

    def workspace(self, n_tok: int):
        need = max(engram_forward_workspace_size(self.g, n_tok), 1)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.w.device)
        return self._ws

    def forward(self, x, ids, mask=None, state=None, out=None, gate=None, err=None):
        return engram_forward(self.g, self.tables, self.table, self.scales, self.w, self.q, self.k,
                              x, ids, mask=mask, state=state, out=out, gate=gate,
                              workspace=self.workspace(ids.numel()), err=err)
