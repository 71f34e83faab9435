"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before touching the
device (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

import gram_memory_layer_amd as ge

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "engram.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = ge.load()
    names = header_functions()
    assert {"engram_hash", "engram_gather", "engram_wkv", "engram_gate_add",
            "engram_forward", "engram_forward_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_loads_and_refuses_bad_arguments():
    # the bench's MFMA ceiling probe: a library of its own, no Engram symbols
    import ctypes as C
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "bench_probe", "libengram_probe.so")
    lib = C.CDLL(path)
    for n in ("engram_probe_mfma", "engram_probe_mfma_flops", "engram_probe_wall_clock_hz"):
        assert hasattr(lib, n), n
    assert not hasattr(lib, "engram_forward")
    lib.engram_probe_mfma_flops.restype = C.c_double
    lib.engram_probe_mfma_flops.argtypes = [C.c_int, C.c_int]
    # 2 blocks x 8 waves x 10 steps x 8 MFMAs x 2*32*32*16 flop
    assert lib.engram_probe_mfma_flops(2, 10) == 2 * 8 * 10 * 8 * 2 * 32 * 32 * 16
    lib.engram_probe_mfma.restype = C.c_int
    lib.engram_probe_mfma.argtypes = [C.c_void_p] * 3 + [C.c_int] * 3 + [C.c_void_p]
    assert lib.engram_probe_mfma(None, None, None, 1, 1, 0, None) != 0   # nothing launched


def good():
    return ge.Geometry.make(dim=5120, hc_mult=4, max_ngram_size=3, n_heads=12, head_dim=64,
                            num_embeddings=25160950, vocab=129280)


def test_geometry_checks():
    assert ge.engram_check_geometry(good()) == 0
    bad = [dict(dim=12), dict(dim=0), dict(hc_mult=0), dict(hc_mult=9), dict(head_dim=48),
           dict(head_dim=16), dict(max_ngram_size=1), dict(max_ngram_size=17), dict(n_heads=0),
           dict(num_embeddings=0), dict(num_embeddings=1 << 31), dict(n_heads=600)]
    for kw in bad:
        g = good()
        for k, v in kw.items():
            setattr(g, k, v)
        assert ge.engram_check_geometry(g) != 0, kw
    g = good()
    g.norm_eps = float("nan")
    assert ge.engram_check_geometry(g) == 1
    g = good()
    g.reserved = 1
    assert ge.engram_check_geometry(g) == 1


def test_derived_sizes():
    g = good()
    assert (g.n_hash_cols, g.K, g.N) == (24, 1536, 25600)
    ws = ge.engram_forward_workspace_size(g, 4096)
    # hash ids, rows (or the fused scratch), kv, and the live-row maps
    assert ws == 4096 * 24 * 4 + 4096 * 1536 * 2 + 4096 * 25600 * 2 + 4096 * 4 + 4096 * 4 + 256
    assert ge.engram_forward_workspace_size(g, 0) == 0


def test_host_side_rejections_launch_nothing():
    lib = ge.load()
    g = good()
    fake = C.c_void_p(1 << 20)           # never dereferenced: every call below fails validation
    ht = ge.HashTables(fake, fake, fake, fake)
    assert lib.engram_wkv(C.byref(g), None, fake, 16, fake, None) == 1
    assert lib.engram_wkv(C.byref(g), fake, fake, -1, fake, None) == 1
    assert lib.engram_wkv(C.byref(g), C.c_void_p((1 << 20) + 2), fake, 16, fake, None) == 1
    assert lib.engram_gate_add(C.byref(g), fake, None, fake, fake, None, 4, fake, None, None) == 1
    assert lib.engram_gather(C.byref(g), fake, fake, fake, -5, fake, None, None) == 1
    assert lib.engram_hash(C.byref(g), None, None, fake, 1, 4, fake, None, None) == 1
    assert lib.engram_hash(C.byref(g), C.byref(ht), None, fake, -1, 4, fake, None, None) == 1
    # forward: workspace missing / too small / misaligned
    args = [C.byref(g), C.byref(ht), fake, fake, fake, fake, fake, None, fake, fake, None, 1, 8,
            fake, None]
    assert lib.engram_forward(*args, None, 0, None, None) == 3
    assert lib.engram_forward(*args, fake, 100, None, None) == 3
    assert lib.engram_forward(*args, C.c_void_p((1 << 20) + 16), 1 << 30, None, None) == 3
    # empty work is a no-op success
    assert lib.engram_wkv(C.byref(g), fake, fake, 0, fake, None) == 0
    assert lib.engram_hash(C.byref(g), C.byref(ht), None, fake, 0, 5, fake, None, None) == 0
    # unsupported geometry is reported before anything else
    g.head_dim = 40
    assert lib.engram_wkv(C.byref(g), fake, fake, 16, fake, None) == 2
    assert lib.engram_status_string(2) == b"unsupported geometry"


def test_hash_layers_host_checks():
    lib = ge.load()
    fake = C.c_void_p(1 << 20)
    n = 3
    geoms = (ge.Geometry * n)(*[good() for _ in range(n)])
    tabs = (ge.HashTables * n)(*[ge.HashTables(fake, fake, fake, fake) for _ in range(n)])

    def call(n=n, geoms=geoms, tabs=tabs, states=None, B=1, T=8):
        return lib.engram_hash_layers(geoms, tabs, n, states, fake, B, T, fake, None, None)
    assert call(n=0) == 1
    assert call(n=33) == 1
    assert call(B=-1) == 1
    assert call(tabs=None) == 1
    g2 = (ge.Geometry * n)(*[good() for _ in range(n)])
    g2[1].n_heads = 6                                     # shared index arithmetic differs
    assert call(geoms=g2) == 1
    g3 = (ge.Geometry * n)(*[good() for _ in range(n)])
    g3[2].num_embeddings = 1000                           # table sizes may differ
    assert call(geoms=g3, B=0) == 0
    dup = (C.c_void_p * n)(fake, C.c_void_p((1 << 20) + 64), fake)
    assert call(states=dup) == 1                          # states are updated in place
    part = (C.c_void_p * n)(fake, None, C.c_void_p((1 << 20) + 64))
    assert call(states=part) == 1
    b = (ge.HashTables * n)(*[ge.HashTables(fake, fake, fake, fake) for _ in range(n)])
    b[1].prime = None
    assert call(tabs=b) == 1
    assert call(B=0) == 0                                 # empty work: a no-op success


def test_forward_hashed_host_checks():
    lib = ge.load()
    g = good()
    fake = C.c_void_p(1 << 20)

    def call(hid=fake, n=8, ws=fake, nbytes=1 << 40, x=fake):
        return lib.engram_forward_hashed(C.byref(g), fake, fake, fake, fake, fake, x, hid, None,
                                         n, fake, None, ws, nbytes, None, None)
    assert call(n=-1) == 1
    assert call(hid=None) == 1
    assert call(x=C.c_void_p((1 << 20) + 2)) == 1          # x must be 16-byte aligned
    assert call(ws=None) == 3
    assert call(nbytes=100) == 3
    assert call(n=0) == 0


def test_fused_projection_host_checks():
    lib = ge.load()
    g = good()
    fake = C.c_void_p(1 << 20)
    need = ge.engram_wkv_gathered_scratch_size(g, 4096)
    assert need == 24 * 4096 * 72 + 4 * 5120 * 4
    # decode-sized batches keep row offsets (12 bytes a row), larger ones copy rows (72)
    assert ge.engram_wkv_gathered_scratch_size(g, 1) == 24 * 256 * 12 + 4 * 5120 * 4
    assert ge.engram_wkv_gathered_scratch_size(g, 256) == 24 * 256 * 12 + 4 * 5120 * 4
    assert ge.engram_wkv_gathered_scratch_size(g, 257) == 24 * 512 * 72 + 4 * 5120 * 4

    def call(g=g, M=16, scratch=fake, nbytes=1 << 30, table=fake):
        return lib.engram_wkv_gathered(C.byref(g), table, fake, fake, M, fake, fake, scratch,
                                       nbytes, None, None)
    assert call(M=-1) == 1
    assert call(table=None) == 1
    assert call(table=C.c_void_p((1 << 20) + 8)) == 1    # table must be 16-byte aligned
    assert call(scratch=None) == 3
    assert call(nbytes=100) == 3
    assert call(scratch=C.c_void_p((1 << 20) + 64)) == 3  # scratch must be 256-byte aligned
    assert call(M=0) == 0
    h = good()
    h.head_dim = 32                                        # one row is not one k-tile
    assert call(g=h) == 2
    h = good()
    h.num_embeddings = (1 << 26) + 1                       # decode-sized: table offsets 32-bit
    assert call(g=h) == 2
    # larger batches: the copied rows' offsets are 32-bit (24 columns x 64 bytes x rows)
    assert call(M=(1 << 31) // (24 * 64)) == 2
    # small batches: the forward's workspace also holds the fused scratch
    assert ge.engram_forward_workspace_size(g, 1) >= 256 + 24 * 256 * 12


def test_binding_refuses_host_tensors():
    import torch
    g = good()
    with pytest.raises(ValueError):
        ge.engram_wkv(g, torch.zeros(4, 1536, dtype=torch.bfloat16),
                      torch.zeros(25600, 1536, dtype=torch.bfloat16))


def test_forward_noalloc_host_checks():
    # the fixed-scratch forward: every engram_forward argument check, then a
    # size check against the fixed array, all before anything touches a GPU
    lib = ge.load()
    assert lib.engram_fixed_scratch_bytes() == 32 << 20
    assert lib.engram_status_string(5) == b"call needs more than the fixed scratch array holds"
    g = good()
    fake = C.c_void_p(1 << 20)           # never dereferenced: every call below fails validation
    ht = ge.HashTables(fake, fake, fake, fake)

    def call(B, T, ids=fake, x=fake, out=fake):
        return lib.engram_forward_noalloc(C.byref(g), C.byref(ht), fake, fake, fake, fake, fake,
                                          None, x, ids, None, B, T, out, None, None, None)
    assert call(1, 8, ids=None) == 1
    assert call(1, 8, out=None) == 1
    assert call(-1, 8) == 1
    assert call(1, 8, x=C.c_void_p((1 << 20) + 2)) == 1
    assert call(0, 8) == 0  # empty: a no-op success
    big = 1
    while ge.engram_forward_workspace_size(g, big) <= (32 << 20):
        big *= 2
    assert call(1, big) == 5
    g.head_dim = 40
    assert call(1, 8) == 2


def test_build_refuses_kernels_that_use_scratch():
    # the build reads the compiler's resource-usage remarks and refuses any
    # kernel with scratch memory (a spill or a local array placed there)
    from gram_memory_layer_amd import build
    remarks = "\n".join([
        "x.hip:1:1: remark: Function Name: _Z6kernelAv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark: Function Name: _Z6kernelBv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     VGPRs: 512 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]",
    ])
    found = build._scratch_kernels(remarks)
    assert len(found) == 1 and found[0].startswith("_Z6kernelBv")
    assert build._scratch_kernels("") == []
