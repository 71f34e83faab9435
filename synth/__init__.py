"""Seeded synthetic inputs for the Engram forward path.

This package only draws random inputs and builds the given tables (token map,
multipliers, primes, offsets, the fp8 table and its scales, weights,
activations, masks).  It holds none of the method's arithmetic: no hashing, no
dequantisation, no projection and no gating happen here.  Both sides of every
parity check (the CPU oracle and the HIP library) receive the bytes produced
here; neither side imports the other.

Five workloads are defined (see ``CONFIGS``): a tiny forward, the
DeepSeek-V4.1-shaped prefill (T=4096, dim=5120, hc=4), a 64-sequence decode
after a 512-token prefill, a gate-and-add bandwidth stress over 65,536 tokens,
and a 32,768-token prefill with Zipf(1.1) ids and masked image spans.

Seeding: each workload has a base seed ``20260 + index``; each tensor draws
from its own named sub-stream, so the same tensor is reproduced whatever else
was drawn.  Host tensors use numpy ``Generator(PCG64)``; bulk device tensors
use a seeded ``torch.Generator`` on that device (host and device draws for the
same name are different numbers, which is fine: every test draws once and feeds
the same bytes to both sides).
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np
import torch

__all__ = [
    "Config", "CONFIGS", "config", "geometry_dict", "n_hash_cols",
    "primes_below", "hash_tables", "token_ids", "token_mask",
    "embedding_table", "wkv_weight", "qk_weights", "activations",
    "gate_stress_kv", "equal_weight_pairs", "np_rng", "torch_gen",
]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    index: int
    B: int
    T: int
    dim: int = 5120
    hc_mult: int = 4
    max_ngram_size: int = 3
    n_heads: int = 12
    head_dim: int = 64
    norm_eps: float = 1e-6
    vocab: int = 129280
    n_compressed: int = 65536
    prime_limit: int = 1 << 20      # primes are the largest ones below this
    pad_id: int = 0
    ids: str = "uniform"            # "uniform" or "zipf1.1"
    scale_codes: tuple = (123, 131)  # e8m0 codes drawn uniformly in this closed range
    mask_frac: float = 0.0          # fraction of positions masked, in spans
    prefill: int = 0                # decode workload: tokens hashed before the steps
    steps: int = 0                  # decode workload: one token per sequence per step

    @property
    def seed(self) -> int:
        return 20260 + self.index

    @property
    def n_tokens(self) -> int:
        return self.B * self.T


CONFIGS = {
    "tiny": Config("tiny", 1, B=1, T=16, dim=256, hc_mult=4, max_ngram_size=3,
                   n_heads=2, head_dim=32, vocab=1000, n_compressed=500,
                   prime_limit=1009, scale_codes=(127, 127)),
    "prefill": Config("prefill", 2, B=1, T=4096),
    "decode": Config("decode", 3, B=64, T=1, prefill=512, steps=128),
    "gate_stress": Config("gate_stress", 4, B=8, T=8192),
    "long_mixed": Config("long_mixed", 5, B=1, T=32768, ids="zipf1.1", mask_frac=0.30),
}


def config(name: str) -> Config:
    return CONFIGS[name]


def n_hash_cols(cfg: Config) -> int:
    # n-gram sizes 2..max_ngram_size, one column per (size, head)
    return (cfg.max_ngram_size - 1) * cfg.n_heads


def geometry_dict(cfg: Config, num_embeddings: int) -> dict:
    return dict(dim=cfg.dim, hc_mult=cfg.hc_mult, max_ngram_size=cfg.max_ngram_size,
                n_heads=cfg.n_heads, head_dim=cfg.head_dim, norm_eps=cfg.norm_eps,
                num_embeddings=int(num_embeddings), vocab=cfg.vocab, pad_id=cfg.pad_id)


# ---------------------------------------------------------------- seeding
def _stream_id(name: str) -> int:
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def np_rng(cfg: Config, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([cfg.seed, _stream_id(name)]))


def torch_gen(cfg: Config, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed * 1_000_003 + _stream_id(name))
    return g


# ---------------------------------------------------------------- given tables
def primes_below(limit: int, count: int) -> list[int]:
    """The `count` largest primes below `limit`, in descending order (trial division)."""
    def is_prime(n: int) -> bool:
        if n < 2:
            return False
        d = 2
        while d * d <= n:
            if n % d == 0:
                return False
            d += 1
        return True

    out, n = [], limit - 1
    while len(out) < count and n >= 2:
        if is_prime(n):
            out.append(n)
        n -= 1
    if len(out) < count:
        raise ValueError("not enough primes below limit")
    return out


def hash_tables(cfg: Config) -> dict:
    """token_map, multipliers, primes and offsets, as a loader would hand them over.

    Columns are ordered size-major: col = (n - 2) * n_heads + head.  Multipliers
    are random odd uint64, one per (size, head, lookback) -> [n_cols, max_ngram];
    size-n columns use lookbacks 0..n-1 and ignore the rest.  Offsets are the
    exclusive prefix sums of the primes, so slot `col` owns rows
    [offset, offset + prime).
    """
    nc = n_hash_cols(cfg)
    rng = np_rng(cfg, "token_map")
    token_map = rng.integers(0, cfg.n_compressed, size=cfg.vocab, dtype=np.int64).astype(np.int32)
    raw = np_rng(cfg, "multipliers").bit_generator.random_raw(nc * cfg.max_ngram_size)
    mult = (np.asarray(raw, dtype=np.uint64) | np.uint64(1)).reshape(nc, cfg.max_ngram_size)
    prime = np.array(primes_below(cfg.prime_limit, nc), dtype=np.uint64)
    offset = np.zeros(nc, dtype=np.uint64)
    offset[1:] = np.cumsum(prime[:-1], dtype=np.uint64)
    num_embeddings = int(prime.sum())
    return dict(token_map=token_map, mult=mult, prime=prime, offset=offset,
                num_embeddings=num_embeddings)


def token_ids(cfg: Config, B: int, T: int, name: str = "ids") -> np.ndarray:
    rng = np_rng(cfg, name)
    if cfg.ids == "uniform":
        return rng.integers(0, cfg.vocab, size=(B, T), dtype=np.int64).astype(np.int32)
    if cfg.ids == "zipf1.1":
        # rank r ~ Zipf(1.1) truncated to [1, vocab]; id = r - 1
        r = np.arange(1, cfg.vocab + 1, dtype=np.float64)
        p = r ** -1.1
        p /= p.sum()
        return rng.choice(cfg.vocab, size=(B, T), p=p).astype(np.int32)
    raise ValueError(cfg.ids)


def token_mask(cfg: Config, B: int, T: int, name: str = "mask") -> np.ndarray:
    """bool [B, T]; False on non-overlapping spans of 256..1024 positions until
    at least `mask_frac` of each row is covered (spans shrink to fit short rows)."""
    mask = np.ones((B, T), dtype=bool)
    if cfg.mask_frac <= 0:
        return mask
    rng = np_rng(cfg, name)
    lo, hi = (256, 1024) if T >= 4096 else (max(1, T // 16), max(1, T // 4))
    for b in range(B):
        covered, tries = 0, 0
        while covered < cfg.mask_frac * T and tries < 100000:
            tries += 1
            L = int(rng.integers(lo, hi + 1))
            s = int(rng.integers(0, T - L + 1))
            if mask[b, max(0, s - 1):s + L + 1].all():
                mask[b, s:s + L] = False
                covered += L
    return mask


# ---------------------------------------------------------------- device tensors
def embedding_table(cfg: Config, rows: int, device, chunk_rows: int = 1 << 20):
    """fp8 e4m3fn table [rows, head_dim] (raw codes, uint8) drawn from N(0,1) and
    cast by torch with round-to-nearest-even, plus e8m0 scale codes
    [rows, head_dim // 32] drawn uniformly from `scale_codes`."""
    hd = cfg.head_dim
    table = torch.empty((rows, hd), dtype=torch.uint8, device=device)
    g = torch_gen(cfg, "table", device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        v = torch.randn((r1 - r0, hd), generator=g, device=device, dtype=torch.float32)
        table[r0:r1] = v.to(torch.float8_e4m3fn).view(torch.uint8)
        del v
    lo, hi = cfg.scale_codes
    gs = torch_gen(cfg, "scales", device)
    scales = torch.randint(lo, hi + 1, (rows, hd // 32), generator=gs, device=device,
                           dtype=torch.int32).to(torch.uint8)
    return table, scales


def wkv_weight(cfg: Config, device) -> torch.Tensor:
    """bf16 [dim*(hc+1), n_hash_cols*head_dim] ~ N(0, std = in^-0.5), layout [out, in]."""
    K = n_hash_cols(cfg) * cfg.head_dim
    N = cfg.dim * (cfg.hc_mult + 1)
    g = torch_gen(cfg, "wkv", device)
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    w.mul_(K ** -0.5)
    return w.to(torch.bfloat16)


def qk_weights(cfg: Config, device):
    """q_weight, k_weight: bf16 [hc, dim] = 1 + U(-0.05, 0.05)."""
    out = []
    for nm in ("q_weight", "k_weight"):
        g = torch_gen(cfg, nm, device)
        u = torch.rand((cfg.hc_mult, cfg.dim), generator=g, device=device, dtype=torch.float32)
        out.append((1.0 + (u * 0.1 - 0.05)).to(torch.bfloat16))
    return out[0], out[1]


def activations(cfg: Config, n_tok: int, device, name: str = "x") -> torch.Tensor:
    """x: bf16 [n_tok, hc, dim] ~ N(0, 1)."""
    g = torch_gen(cfg, name, device)
    x = torch.randn((n_tok, cfg.hc_mult, cfg.dim), generator=g, device=device,
                    dtype=torch.float32)
    return x.to(torch.bfloat16)


def equal_weight_pairs(q: torch.Tensor, k: torch.Tensor) -> list[tuple[int, int]]:
    """Per stream, one feature pair (i, j), i < j, whose q and k are bit-equal,
    so that the two features carry the same gate weight."""
    qb = q.view(torch.int16).cpu().numpy().astype(np.int64) & 0xFFFF
    kb = k.view(torch.int16).cpu().numpy().astype(np.int64) & 0xFFFF
    pairs = []
    for s in range(q.shape[0]):
        seen = {}
        found = None
        for f in range(q.shape[1]):
            key = (int(qb[s, f]), int(kb[s, f]))
            if key in seen:
                found = (seen[key], f)
                break
            seen[key] = f
        if found is None:
            raise ValueError("no equal-weight feature pair in stream %d" % s)
        pairs.append(found)
    return pairs


def gate_stress_kv(cfg: Config, x: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                   name: str = "kv", frac_orth: float = 0.25, frac_mid: float = 0.15):
    """kv bf16 [n_tok, dim*(hc+1)] for the gate-and-add stress workload.

    Per (token, stream) one of three key recipes is drawn:
      * with probability `frac_orth`: a key exactly orthogonal to the stream
        under the gate weight -- zero except key_i = x_j, key_j = -x_i for a
        feature pair (i, j) with equal weights, so the weighted dot is +0;
      * with probability `frac_mid`: key = c*x + 0.1*N(0,1), c ~ U(-0.005, 0.005)
        (gates in the middle of (0, 1));
      * otherwise key = c*x + 0.1*N(0,1), c ~ U(-2, 2).
    The shared value is N(0,1).  Returns (kv, category[n_tok, hc] int8 with
    0 = orthogonal, 1 = mid, 2 = wide).
    """
    n_tok, hc, dim = x.shape
    dev = x.device
    g = torch_gen(cfg, name, dev)
    u = torch.rand((n_tok, hc), generator=g, device=dev)
    cat = torch.full((n_tok, hc), 2, dtype=torch.int8, device=dev)
    cat[u < frac_orth + frac_mid] = 1
    cat[u < frac_orth] = 0
    c_wide = torch.rand((n_tok, hc), generator=g, device=dev) * 4.0 - 2.0
    c_mid = torch.rand((n_tok, hc), generator=g, device=dev) * 0.01 - 0.005
    kv = torch.empty((n_tok, dim * (hc + 1)), dtype=torch.bfloat16, device=dev)
    pairs = equal_weight_pairs(q, k)
    step = 4096
    for t0 in range(0, n_tok, step):
        t1 = min(n_tok, t0 + step)
        xf = x[t0:t1].float()
        noise = torch.randn(xf.shape, generator=g, device=dev)
        cc = torch.where(cat[t0:t1] == 1, c_mid[t0:t1], c_wide[t0:t1])
        key = cc.unsqueeze(-1) * xf + 0.1 * noise
        orth = (cat[t0:t1] == 0)
        for s, (i, j) in enumerate(pairs):
            rows = orth[:, s]
            if rows.any():
                kk = torch.zeros((int(rows.sum()), dim), device=dev)
                xs = xf[rows, s]
                kk[:, i] = xs[:, j]
                kk[:, j] = -xs[:, i]
                key[rows, s] = kk
        kv[t0:t1, :hc * dim] = key.reshape(t1 - t0, hc * dim).to(torch.bfloat16)
        v = torch.randn((t1 - t0, dim), generator=g, device=dev)
        kv[t0:t1, hc * dim:] = v.to(torch.bfloat16)
    return kv, cat
