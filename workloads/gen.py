"""Seeded synthetic inputs shared by the HIP path's harness and by the oracle.

This module generates *inputs only*: token ids and the Q/K/V vectors that a
model would have produced for them. It holds no attention arithmetic and no
radix-tree logic.

Why Q/K/V depend on the whole prefix: the pages state that a token's KV depends
only on the tokens before it (2312.07104_SGLang notes, §3 "KV cache reuse
background" and App. A.1). We model that directly: the vector of kind t (q, k
or v) for head h, dim d at position p of a sequence is a deterministic function
of (seed, t, h, d, tokens[0..p]). Two sequences that share a prefix therefore
share the K/V of that prefix bit for bit, so "reuse cached KV" and "recompute
from scratch" give the same inputs, which is the premise the method relies on.

Construction (all published methods, written here from their definitions):
  * SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): the finaliser z -> mix(z + golden).
  * Rolling prefix hash: h_{-1} = splitmix64(seed), h_p = splitmix64(h_{p-1} ^ tok_p).
  * Per-element bits: x = splitmix64(h_p ^ key[t, h, d]) with
    key[t, h, d] = splitmix64(seed ^ (t << 48) ^ (h << 24) ^ d).
  * Box-Muller (1958) in float64: u1 = (hi24 + 1) / 2^24 in (0, 1],
    u2 = mid24 / 2^24 in [0, 1), z = sqrt(-2 ln u1) * cos(2 pi u2).
  * Rounded once to the working dtype (fp32 or bf16, round-to-nearest-even).

Token ids are uniform in [0, vocab) from numpy's PCG64 generator.

The element generator is written with torch int64 ops (two's-complement wrap)
so that it runs on the CPU for the oracle and on the GPU for the harness.
"""
from __future__ import annotations

import math

import numpy as np
import torch

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

KIND_Q, KIND_K, KIND_V = 0, 1, 2
VOCAB = 32000


def _signed(x: int) -> int:
    x &= MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def splitmix64(x: int) -> int:
    """SplitMix64 output for state value ``x`` (pure Python, exact)."""
    z = (x + GOLDEN) & MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


# ---------------------------------------------------------------- numpy (host)
def _splitmix64_np(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = x + np.uint64(GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
        return z ^ (z >> np.uint64(31))


def prefix_hashes(tokens, seed: int, h0: int | None = None) -> np.ndarray:
    """Rolling prefix hash of one token sequence: uint64[n], h_p covers tokens[0..p].

    ``h0`` continues a chain (the hash of the position before tokens[0]); by
    default the chain starts from splitmix64(seed).
    """
    toks = np.asarray(tokens, dtype=np.int64)
    out = np.empty(len(toks), dtype=np.uint64)
    h = splitmix64(seed & MASK64) if h0 is None else int(h0)
    for i, t in enumerate(toks.tolist()):
        h = splitmix64(h ^ (t & MASK64))
        out[i] = h
    return out


def prefix_hashes_batch(seqs: list, seed: int) -> list:
    """prefix_hashes for many sequences at once (vectorised over sequences, padded)."""
    if not seqs:
        return []
    lens = [len(s) for s in seqs]
    lmax = max(lens)
    toks = np.zeros((len(seqs), max(lmax, 1)), dtype=np.uint64)
    for i, s in enumerate(seqs):
        toks[i, : lens[i]] = np.asarray(s, dtype=np.int64).astype(np.uint64)
    h = np.full(len(seqs), splitmix64(seed & MASK64), dtype=np.uint64)
    res = np.empty((len(seqs), lmax), dtype=np.uint64)
    for p in range(lmax):
        h = _splitmix64_np(h ^ toks[:, p])
        res[:, p] = h
    return [res[i, : lens[i]].copy() for i in range(len(seqs))]


# ----------------------------------------------------------- torch (any device)
_G_S = _signed(GOLDEN)
_M1_S = _signed(MIX1)
_M2_S = _signed(MIX2)


def _srl(x: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 viewed as uint64."""
    return (x >> k) & ((1 << (64 - k)) - 1)


def splitmix64_t(x: torch.Tensor) -> torch.Tensor:
    z = x + _G_S
    z = (z ^ _srl(z, 30)) * _M1_S
    z = (z ^ _srl(z, 27)) * _M2_S
    return z ^ _srl(z, 31)


def _keys(seed: int, kind: int, n_heads: int, head_dim: int, device) -> torch.Tensor:
    h = torch.arange(n_heads, dtype=torch.int64, device=device).view(n_heads, 1)
    d = torch.arange(head_dim, dtype=torch.int64, device=device).view(1, head_dim)
    base = _signed((seed & MASK64) ^ (kind << 48))
    return splitmix64_t(base ^ (h << 24) ^ d)


def normals_from_bits(x: torch.Tensor) -> torch.Tensor:
    """Box-Muller on the high 48 bits of each int64 word, in float64."""
    hi = _srl(x, 40)                       # 24 bits
    mid = _srl(x, 16) & 0xFFFFFF           # next 24 bits
    u1 = (hi + 1).to(torch.float64) * (1.0 / (1 << 24))
    u2 = mid.to(torch.float64) * (1.0 / (1 << 24))
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def qkv_values(hashes, kind: int, n_heads: int, head_dim: int, seed: int,
               dtype=torch.float32, device="cpu", chunk: int = 1 << 22) -> torch.Tensor:
    """Vectors of one kind for positions with the given prefix hashes.

    Returns ``[N, n_heads, head_dim]`` in ``dtype`` on ``device``: N(0,1) values
    computed in float64 and rounded once to ``dtype``.
    """
    if isinstance(hashes, np.ndarray):
        hv = torch.from_numpy(hashes.view(np.int64).copy())
    else:
        hv = hashes
    hv = hv.to(device=device, dtype=torch.int64)
    n = hv.numel()
    out = torch.empty((n, n_heads, head_dim), dtype=dtype, device=device)
    if n == 0:
        return out
    keys = _keys(seed, kind, n_heads, head_dim, device)
    per = max(1, chunk // (n_heads * head_dim))
    for s in range(0, n, per):
        e = min(n, s + per)
        bits = splitmix64_t(hv[s:e].view(-1, 1, 1) ^ keys.unsqueeze(0))
        out[s:e] = normals_from_bits(bits).to(dtype)
    return out


def tokens(rng: np.random.Generator, n: int, vocab: int = VOCAB) -> np.ndarray:
    """Uniform token ids in [0, vocab) as int32."""
    return rng.integers(0, vocab, size=int(n), dtype=np.int64).astype(np.int32)


def projection_inputs(seed: int, t: int, hidden: int, n_out: int):
    """Hidden states x [t, hidden] ~ N(0, 1) and projection weights w [n_out, hidden] ~
    N(0, 1/hidden), both rounded to bf16 (returned as float32 CPU tensors holding bf16
    values), so that projected values are O(1)."""
    g = torch.Generator().manual_seed(int(seed) & 0x7FFFFFFF)
    x = torch.randn((t, hidden), generator=g).to(torch.bfloat16).float()
    w = (torch.randn((n_out, hidden), generator=g) / hidden ** 0.5).to(torch.bfloat16).float()
    return x, w
