"""engram_forward_noalloc (the forward with the library's fixed per-GPU
scratch array as its workspace, for callers that cannot allocate) against
engram_forward with a caller workspace: every output, gate, error word and
state bit for bit, on calls in a row that reuse the array with smaller
inputs, on both forward paths it takes (the gathered rows and the general
projection for a mid-sized batch; the fused 64-wide tiles for a decode
step), with and without a mask.  A call too large for the array is refused
before anything is launched."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import Workload, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    import gram_memory_layer_amd as ge
    ge.load()
    return ge


def _pair(ge, wl, B, T, name, with_mask, dev):
    cfg = wl.cfg
    ids = torch.from_numpy(synth.token_ids(cfg, B, T, name="ids_" + name)).to(dev)
    x = synth.activations(cfg, B * T, dev, name="x_" + name).reshape(B, T, cfg.hc_mult, cfg.dim)
    mask = None
    if with_mask:
        mask = torch.from_numpy(synth.token_ids(cfg, B, T, name="m_" + name) % 4 != 0).to(dev)
    state0 = torch.from_numpy(
        synth.token_ids(cfg, B, cfg.max_ngram_size - 1, name="s_" + name) % cfg.n_compressed).to(dev)
    res = []
    for fn in ("ws", "noalloc"):
        state = state0.clone()
        out = torch.empty_like(x)
        gate = torch.empty((B, T, cfg.hc_mult), dtype=torch.float32, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        if fn == "ws":
            ge.engram_forward(wl.g, wl.tables, wl.table, wl.scales, wl.w, wl.q, wl.k, x, ids,
                              mask=mask, state=state, out=out, gate=gate, err=err)
        else:
            ge.engram_forward_noalloc(wl.g, wl.tables, wl.table, wl.scales, wl.w, wl.q, wl.k, x,
                                      ids, out, mask=mask, state=state, gate=gate, err=err)
        res.append((out, gate, err, state))
    torch.cuda.synchronize()
    (o1, g1, e1, s1), (o2, g2, e2, s2) = res
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), name
    assert torch.equal(g1, g2), name
    assert torch.equal(e1, e2) and int(e1.item()) == 0, name
    assert torch.equal(s1, s2), name
    if mask is not None:
        m = ~mask.reshape(-1)
        assert torch.equal(o2.reshape(B * T, -1)[m].view(torch.int16),
                           x.reshape(B * T, -1)[m].view(torch.int16))


def test_forward_noalloc_matches_forward(ge):
    dev = torch.device("cuda:0")
    say("no-alloc forward: building the prefill-shaped tables")
    wl = Workload(ge, "prefill", dev)
    cap = ge.engram_fixed_scratch_bytes()
    # calls in a row on the one array, each smaller than the one before
    for B, T, with_mask in ((2, 300, False), (64, 1, False), (16, 1, True), (1, 5, False)):
        need = ge.engram_forward_workspace_size(wl.g, B * T)
        assert need <= cap
        say("no-alloc forward B=%d T=%d mask=%s (workspace %d of %d bytes)" % (
            B, T, with_mask, need, cap))
        _pair(ge, wl, B, T, "%d_%d_%d" % (B, T, with_mask), with_mask, dev)
    # too large for the array: refused on the host, nothing launched
    B, T = 1, 2048
    assert ge.engram_forward_workspace_size(wl.g, B * T) > cap
    ids = torch.zeros((B, T), dtype=torch.int32, device=dev)
    x = torch.zeros((B, T, wl.cfg.hc_mult, wl.cfg.dim), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ge.EngramError) as ei:
        ge.engram_forward_noalloc(wl.g, wl.tables, wl.table, wl.scales, wl.w, wl.q, wl.k, x, ids,
                                  torch.empty_like(x))
    assert ei.value.status == ge.ERR_TOO_LARGE
