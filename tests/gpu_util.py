"""Shared helpers for the GPU parity tests: build a workload's inputs once
(from the seeded generators) and hand the same bytes to the HIP library and
to the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth


def say(*a):
    """Print and flush, so a GPU run names the case it is in."""
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def geometry(ge, cfg, num_embeddings):
    return ge.Geometry.make(cfg.dim, cfg.hc_mult, cfg.max_ngram_size, cfg.n_heads, cfg.head_dim,
                            num_embeddings, cfg.vocab, cfg.pad_id, cfg.norm_eps)


def device_tables(t: dict, dev) -> dict:
    return {k: torch.from_numpy(np.ascontiguousarray(t[k])).to(dev)
            for k in ("token_map", "mult", "prime", "offset")}


class Workload:
    """Every given input of one configuration, on the device (bulk tensors
    drawn there) and the host tables."""

    def __init__(self, ge, name, dev, with_table: bool = True, with_weights: bool = True):
        """`name`: a configuration name, or a synth.Config itself."""
        self.cfg = cfg = synth.config(name) if isinstance(name, str) else name
        self.t = synth.hash_tables(cfg)
        self.num_emb = self.t["num_embeddings"]
        self.g = geometry(ge, cfg, self.num_emb)
        self.geom = synth.geometry_dict(cfg, self.num_emb)
        self.dev = dev
        self.tables = device_tables(self.t, dev)
        if with_table:
            self.table, self.scales = synth.embedding_table(cfg, self.num_emb, dev)
        if with_weights:
            self.w = synth.wkv_weight(cfg, dev)
            self.q, self.k = synth.qk_weights(cfg, dev)

    def host_rows(self, ids: np.ndarray):
        """The table and scale rows that `ids` reference, copied to the host,
        with the ids renumbered into that compact copy."""
        uniq, inv = np.unique(ids.reshape(-1), return_inverse=True)
        idx = torch.from_numpy(uniq.astype(np.int64)).to(self.dev)
        tab = self.table.index_select(0, idx).cpu().numpy()
        sc = self.scales.index_select(0, idx).cpu().numpy()
        return tab, sc, inv.reshape(ids.shape).astype(np.int32)
