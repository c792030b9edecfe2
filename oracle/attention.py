"""fp64 causal attention recomputed from scratch over a whole token sequence.

TEST INFRASTRUCTURE (oracle). Only tests/, the smoke check and the bench's CPU
baseline leg may use this module. It never reads a KV pool: every key and value
is regenerated from the sequence's own tokens.

What it computes. Reusing cached KV is only an optimisation: the pages state
that a token's KV depends on the preceding tokens alone (2312.07104_SGLang
notes, §3 background and App. A.1), so the output for a suffix query that runs
against reused prefix KV equals the output of recomputing the whole sequence.
The oracle is therefore plain causal softmax attention over the full sequence:
for the query at absolute position p and query head h,

    s_j = (q_{p,h} . k_{j,g}) * scale        for j = 0..p,   g = h // (H_q / H_kv)
    o_{p,h} = sum_j softmax(s)_j * v_{j,g}

with scale = 1/sqrt(D). The pages print no attention formula; the scale, the
inclusive causal boundary and the contiguous grouped-query head map are the
plainest readings (decode attends to all earlier tokens and itself, App. A.1).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from workloads import gen


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float | None = None) -> np.ndarray:
    """One query position. q [H_q, D]; K, V [L, H_kv, D] (L >= 1) -> o [H_q, D], all fp64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    h_q, d = q.shape
    h_kv = K.shape[1]
    assert h_q % h_kv == 0 and K.shape[0] >= 1
    g = h_q // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.empty((h_q, d), dtype=np.float64)
    for h in range(h_q):
        kv = h // g
        s = (K[:, kv, :] @ q[h]) * scale
        w = np.exp(s - s.max())
        w /= w.sum()
        o[h] = w @ V[:, kv, :]
    return o


def attend_causal(Q: np.ndarray, K: np.ndarray, V: np.ndarray, positions, scale=None) -> np.ndarray:
    """Q [P, H_q, D] for the given absolute positions; K, V [L, H_kv, D]; row i sees keys 0..positions[i]."""
    return np.stack([attend(Q[i], K[: int(p) + 1], V[: int(p) + 1], scale)
                     for i, p in enumerate(positions)])


def sequence_qkv(tokens, positions, h_q: int, h_kv: int, d: int, seed: int, dtype: str,
                 kv_upto: int | None = None):
    """Regenerate, from the tokens alone, Q at ``positions`` and K/V at 0..kv_upto (fp64).

    Values are rounded to the working dtype first (fp32 or bf16), exactly as the
    inputs the GPU path consumes, then widened to fp64.
    """
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    positions = [int(p) for p in positions]
    last = max(positions) if kv_upto is None else int(kv_upto)
    hashes = gen.prefix_hashes(np.asarray(tokens[: last + 1]), seed)
    Q = gen.qkv_values(hashes[positions], gen.KIND_Q, h_q, d, seed, tdt).double().numpy()
    K = gen.qkv_values(hashes, gen.KIND_K, h_kv, d, seed, tdt).double().numpy()
    V = gen.qkv_values(hashes, gen.KIND_V, h_kv, d, seed, tdt).double().numpy()
    return Q, K, V


def outputs_from_scratch(tokens, positions, h_q, h_kv, d, seed, dtype) -> np.ndarray:
    """Attention outputs [len(positions), H_q, D] (fp64) for a sequence, recomputed from scratch."""
    Q, K, V = sequence_qkv(tokens, positions, h_q, h_kv, d, seed, dtype)
    return attend_causal(Q, K, V, positions)
