"""Plain QKV projection of new tokens.

TEST INFRASTRUCTURE (oracle). Only tests/, the smoke check and the bench's CPU
baseline leg may use this module. It shares no code with the HIP path.

What is computed: before attention, each new token's hidden state is projected to its
query, key and value (hustzhy SGLang post, §2.3 (2): the unmatched suffix is computed;
2312.07104_SGLang notes, App. A.1: prefill computes the new tokens' KV, which the cache
keeps). The pages give no formula; the plainest reading is one linear map per token:
y = x W^T with W of shape [(h_q + 2 h_kv) d, hidden], whose output features are Q
(first h_q d), then K (next h_kv d), then V (last h_kv d), each [heads, d] in head-major
order. In fp64; the kernel rounds its fp32 sums to bf16 once.
"""
from __future__ import annotations

import numpy as np


def qkv_project(x, w, h_q: int, h_kv: int, d: int):
    """(q [T, h_q, d], k [T, h_kv, d], v [T, h_kv, d]) of tokens x [T, hidden], weights
    w [(h_q + 2 h_kv) d, hidden], in fp64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if w.shape != ((h_q + 2 * h_kv) * d, x.shape[1]):
        raise ValueError("w must be [(h_q + 2 h_kv) d, hidden]")
    y = x @ w.T
    t = x.shape[0]
    nq, nkv = h_q * d, h_kv * d
    return (y[:, :nq].reshape(t, h_q, d), y[:, nq: nq + nkv].reshape(t, h_kv, d),
            y[:, nq + nkv:].reshape(t, h_kv, d))


def qkv_project_rows(x, w, rows, h_q: int, h_kv: int, d: int):
    """The same for a subset of token rows only (for sampled checks at full size)."""
    x = np.asarray(x)[np.asarray(rows)]
    return qkv_project(x, w, h_q, h_kv, d)
