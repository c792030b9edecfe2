"""Pins for the oracle's fp64 attention and for the shared input generator.

Attention is pinned by textbook special cases (one key gives its value exactly;
a zero query averages the visible values), by a library routine (torch's
scaled_dot_product_attention in fp64 on the CPU, with an explicit causal mask
and grouped KV heads), and by the premise the method rests on: KV reused from
another request that shares the prefix equals KV recomputed from scratch
(2312.07104_SGLang notes, §3 background, App. A.1).

The generator is pinned by SplitMix64's published first outputs for state 0,
by a pure-Python SplitMix64, and by the normal distribution's moments.
"""
import math

import numpy as np
import pytest
import torch
from scipy import stats

from oracle.attention import attend, attend_causal, outputs_from_scratch, sequence_qkv
from workloads import configs, gen


# ------------------------------------------------------------------ attention
def test_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 16))
    K = rng.standard_normal((1, 2, 16))
    V = rng.standard_normal((1, 2, 16))
    o = attend(q, K, V)
    assert np.array_equal(o, V[0, [0, 0, 1, 1]])


def test_zero_query_is_mean_of_visible_values():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((9, 1, 8))
    V = rng.standard_normal((9, 1, 8))
    o = attend_causal(np.zeros((3, 2, 8)), K, V, positions=[0, 4, 8])
    for i, p in enumerate([0, 4, 8]):
        np.testing.assert_allclose(o[i, 0], V[: p + 1, 0].mean(0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[i, 1], V[: p + 1, 0].mean(0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("h_q,h_kv", [(4, 4), (8, 2), (6, 1)])
def test_matches_torch_sdpa_fp64(h_q, h_kv):
    rng = np.random.default_rng(h_q * 10 + h_kv)
    L, D = 13, 8
    pos = list(range(5, L))
    Q = rng.standard_normal((len(pos), h_q, D))
    K = rng.standard_normal((L, h_kv, D))
    V = rng.standard_normal((L, h_kv, D))
    ours = attend_causal(Q, K, V, pos)
    g = h_q // h_kv
    q = torch.from_numpy(Q).permute(1, 0, 2)                               # [H, P, D]
    k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, dim=0)   # [H, L, D]
    v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, dim=0)
    mask = torch.tensor([[j <= p for j in range(L)] for p in pos])
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    np.testing.assert_allclose(ours, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_scale_is_inverse_sqrt_head_dim():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 16))
    K = rng.standard_normal((5, 1, 16))
    V = rng.standard_normal((5, 1, 16))
    assert np.array_equal(attend(q, K, V), attend(q, K, V, scale=1 / math.sqrt(16)))
    assert not np.allclose(attend(q, K, V), attend(q, K, V, scale=1.0))


def test_reused_prefix_kv_equals_recompute():
    """Request 1 of the tiny trace computes its suffix against request 0's cached prefix KV."""
    job = configs.make(0)
    r0, r1 = job.requests[0], job.requests[1]
    m = 200
    pos = list(range(m, r1.n))
    scratch = outputs_from_scratch(r1.prompt, pos, job.h_q, job.h_kv, job.d, job.seed, job.dtype)
    # "pool": prefix rows produced while serving request 0, suffix rows from request 1
    _, K0, V0 = sequence_qkv(r0.prompt, [m - 1], job.h_q, job.h_kv, job.d, job.seed, job.dtype)
    Q1, K1, V1 = sequence_qkv(r1.prompt, pos, job.h_q, job.h_kv, job.d, job.seed, job.dtype)
    K = np.concatenate([K0[:m], K1[m:]])
    V = np.concatenate([V0[:m], V1[m:]])
    reused = attend_causal(Q1, K, V, pos)
    assert np.array_equal(reused, scratch)
    # and the prefix really is shared while the suffix is not
    assert np.array_equal(K0[:m], K1[:m]) and not np.array_equal(K0[m:m + 20], K1[m:m + 20])


# ------------------------------------------------------------------ generator
def test_splitmix64_published_first_outputs():
    # SplitMix64 seeded with 0 (Steele et al. 2014; reference C code by S. Vigna)
    outs = [gen.splitmix64((k * gen.GOLDEN) & gen.MASK64) for k in range(3)]
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_torch_splitmix_matches_python():
    rng = np.random.default_rng(3)
    xs = [int(x) for x in rng.integers(0, 2**63, 2000, dtype=np.uint64)] + [0, 2**64 - 1, 2**63]
    t = torch.tensor([gen._signed(x) for x in xs], dtype=torch.int64)
    got = [(int(v) & gen.MASK64) for v in gen.splitmix64_t(t)]
    assert got == [gen.splitmix64(x) for x in xs]
    npv = gen._splitmix64_np(np.array(xs, dtype=np.uint64))
    assert [int(v) for v in npv] == [gen.splitmix64(x) for x in xs]


def test_prefix_hash_batch_equals_single():
    rng = np.random.default_rng(4)
    seqs = [rng.integers(0, 32000, n) for n in (5, 9, 9, 1, 0)]
    b = gen.prefix_hashes_batch(seqs, 11)
    for s, h in zip(seqs, b):
        assert np.array_equal(h, gen.prefix_hashes(s, 11))


def test_values_depend_only_on_prefix():
    a = np.array([5, 6, 7, 8, 9, 10], dtype=np.int32)
    b = np.array([5, 6, 7, 1, 9, 10], dtype=np.int32)
    ha, hb = gen.prefix_hashes(a, 3), gen.prefix_hashes(b, 3)
    ka = gen.qkv_values(ha, gen.KIND_K, 2, 8, 3)
    kb = gen.qkv_values(hb, gen.KIND_K, 2, 8, 3)
    assert torch.equal(ka[:3], kb[:3])
    assert not torch.equal(ka[3:], kb[3:]) and not torch.equal(ka[5], kb[5])
    # kinds and seeds give different streams
    assert not torch.equal(ka, gen.qkv_values(ha, gen.KIND_V, 2, 8, 3))
    assert not torch.equal(ka, gen.qkv_values(ha, gen.KIND_K, 2, 8, 4))


def test_values_are_standard_normal():
    h = gen.prefix_hashes(np.arange(4000) % 977, 99)
    x = gen.qkv_values(h, gen.KIND_Q, 4, 64, 99, dtype=torch.float64).flatten().numpy()
    assert abs(x.mean()) < 0.005 and abs(x.var() - 1) < 0.01
    assert stats.kstest(x[:200000], "norm").pvalue > 1e-4


def test_rounding_to_bf16_is_nearest_even():
    h = gen.prefix_hashes(np.arange(64), 1)
    x64 = gen.qkv_values(h, gen.KIND_V, 2, 32, 1, dtype=torch.float64)
    xb = gen.qkv_values(h, gen.KIND_V, 2, 32, 1, dtype=torch.bfloat16)
    assert torch.equal(xb, x64.to(torch.bfloat16))
    # round-to-nearest: no representable bf16 value is closer than the chosen one
    err = (xb.double() - x64).abs()
    ulp = torch.ldexp(torch.ones_like(x64), torch.frexp(x64)[1] - 8)
    assert bool((err <= ulp / 2 + 1e-300).all())
