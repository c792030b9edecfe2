"""Pins of the oracle's helper functions against definitions they do not share code with.

* lca_depth (the sharing hint handed to the kernels): the token depth of the deepest
  common ancestor of two radix nodes. In a radix tree sibling edges start with different
  tokens, so that depth equals the length of the longest common token prefix of the two
  nodes' root paths; the paths are rebuilt here from the model's dump alone
  (2312.07104_SGLang notes, §3, "RadixAttention core idea": edges are token sequences;
  hustzhy SGLang post, §2.3 (1), the three requests branch below their common prefix).
* Admission (reading S2): a batch is the longest prefix of the ordered queue whose
  prompt tokens fit the pool, whose new tokens fit the token budget and whose size fits
  the request limit, and never empty. With a pool that never evicts, the cached prefix
  of a request is the longest common prefix with any prompt already run, computed here
  by brute force, and the orders (arrival, longest cached prefix first with ties in
  arrival order, lexicographic) are rebuilt from their definitions (notes App. A.2 and
  §3 "cache-aware scheduling").
* Random order (reading S4): Fisher-Yates with j = draw mod (i + 1), checked against a
  permutation worked out by hand, against the published SplitMix64 outputs for state 0
  (Steele, Lea, Flood 2014), and for uniformity: every permutation of 3 and of 4 items
  appears with its expected frequency (a Sattolo-style j = draw mod i would only give
  cyclic permutations).
"""
import itertools
import math

import numpy as np
import pytest

from oracle import scheduler as O
from oracle.radix_model import RadixCacheModel


# ------------------------------------------------------------------ lca_depth
def _root_paths(model):
    paths = {0: ()}
    for nid, par, _ln, _ref, _tick, toks, _slots in model.dump():   # preorder: parents first
        paths[nid] = paths[par] + tuple(toks)
    return paths


def _lcp(a, b):
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


@pytest.mark.parametrize("seed", range(6))
def test_lca_depth_is_common_prefix_of_root_paths(seed):
    rng = np.random.default_rng(seed)
    model = RadixCacheModel(4000)
    for _ in range(60):
        toks = [int(t) for t in rng.integers(0, 3, int(rng.integers(1, 14)))]
        if rng.random() < 0.3:
            model.match(toks)                                   # splits at the match end
        else:
            m, slots, _node = model.match(toks)
            new = model.alloc(len(toks) - m)
            model.insert(toks, list(slots) + new)
    paths = _root_paths(model)
    nodes = sorted(paths)
    assert len(nodes) > 20
    for a in nodes:
        for b in nodes:
            assert model.lca_depth(a, b) == _lcp(paths[a], paths[b]), (a, b)
    for a in nodes:
        assert model.lca_depth(a, a) == len(paths[a])
        assert model.lca_depth(0, a) == 0


def test_lca_depth_three_requests_example():
    """The three printed requests share a 37-byte prefix and branch into AI?, ML?, DL?
    (hustzhy SGLang post, §2.3 (1)): any two leaves meet at depth 37, a leaf with itself
    at its own length."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "three_requests.json")) as f:
        gold = json.load(f)
    reqs = [list(r.encode("utf-8")) for r in gold["requests"]]
    model = RadixCacheModel(1000)
    leaves = []
    for toks in reqs:
        m, slots, _ = model.match(toks)
        _, node, _ = model.insert(toks, list(slots) + model.alloc(len(toks) - m))
        leaves.append(node)
    for i, a in enumerate(leaves):
        for j, b in enumerate(leaves):
            assert model.lca_depth(a, b) == (len(reqs[i]) if i == j else gold["shared_prefix_bytes"])


# ------------------------------------------------------------------ admission (S2)
def _workloads():
    rng = np.random.default_rng(5)
    out = []
    for w in range(6):
        vocab = 3 + w
        out.append([[int(t) for t in rng.integers(0, vocab, int(rng.integers(1, 20)))] for _ in range(25)])
    return out


def _brute_cached(done, p):
    """Cached prefix of p when every prompt in `done` is cached (nothing evicted)."""
    return max([_lcp(p, q) for q in done] + [0])


def _order(policy, prompts, waiting, m):
    idx = list(range(len(waiting)))
    if policy == "fcfs":
        return idx
    if policy == "lpm":
        out = []
        for v in sorted({m[r] for r in waiting}, reverse=True):   # longest first, arrival within
            out += [j for j in idx if m[waiting[j]] == v]
        return out
    if policy == "dfs":
        out = []
        for j in idx:                                            # insertion into a sorted list
            k = 0
            while k < len(out) and not prompts[waiting[j]] < prompts[waiting[out[k]]]:
                k += 1
            out.insert(k, j)
        return out
    raise ValueError(policy)


@pytest.mark.parametrize("policy", ["fcfs", "lpm", "dfs"])
@pytest.mark.parametrize("limits", [dict(max_batch=1), dict(max_batch=4), dict(max_batch_tokens=30),
                                    dict(max_batch_tokens=12, max_batch=3)])
def test_admission_takes_the_longest_fitting_prefix_of_the_order(policy, limits):
    budget = limits.get("max_batch_tokens", 1 << 30)
    size = limits.get("max_batch", 1 << 30)
    for prompts in _workloads():
        pool = sum(len(p) for p in prompts) + 1                  # nothing is ever evicted
        batches, computed, _ = O.run_prefill(prompts, pool, policy, **limits)
        waiting = list(range(len(prompts)))
        done, total_new = [], 0
        for batch in batches:
            m = {r: _brute_cached(done, prompts[r]) for r in waiting}
            new = {r: len(prompts[r]) - min(m[r], len(prompts[r]) - 1) for r in waiting}
            order = [waiting[j] for j in _order(policy, prompts, waiting, m)]
            # the longest prefix of the order that fits (one request always goes in)
            want, tok, nn = [], 0, 0
            for r in order:
                if want and (tok + len(prompts[r]) > pool or nn + new[r] > budget or len(want) >= size):
                    break
                want.append(r)
                tok += len(prompts[r])
                nn += new[r]
            assert batch == want
            assert len(batch) == 1 or (nn <= budget and len(batch) <= size and tok <= pool)
            total_new += nn
            done += [prompts[r] for r in batch]
            waiting = [r for r in waiting if r not in batch]
        assert not waiting and computed == total_new


@pytest.mark.parametrize("policy", ["fcfs", "lpm", "dfs", "random"])
def test_admission_respects_a_tight_pool(policy):
    """With evictions the cached prefixes depend on the eviction order, so only what
    lengths alone fix is checked: every request runs once, batches fit the pool unless
    they hold one request, and batches fit the size limit."""
    for prompts in _workloads():
        pool = max(len(p) for p in prompts) + 7
        batches, _, _ = O.run_prefill(prompts, pool, policy, max_batch=5, seed=3)
        assert sorted(r for b in batches for r in b) == list(range(len(prompts)))
        for b in batches:
            assert 1 <= len(b) <= 5
            assert len(b) == 1 or sum(len(prompts[r]) for r in b) <= pool


# ------------------------------------------------------------------ random order (S4)
def test_fisher_yates_hand_worked():
    # n = 4, draws 5, 7, 2:
    #   i = 3: j = 5 mod 4 = 1, swap 3 and 1 -> [0, 3, 2, 1]
    #   i = 2: j = 7 mod 3 = 1, swap 2 and 1 -> [0, 2, 3, 1]
    #   i = 1: j = 2 mod 2 = 0, swap 1 and 0 -> [2, 0, 3, 1]
    assert O.fisher_yates(4, [5, 7, 2]) == [2, 0, 3, 1]
    # n = 5, draws 0, 0, 0, 0: every step swaps with position 0
    #   [4, 1, 2, 3, 0] -> [3, 1, 2, 4, 0] -> [2, 1, 3, 4, 0] -> [1, 2, 3, 4, 0]
    assert O.fisher_yates(5, [0, 0, 0, 0]) == [1, 2, 3, 4, 0]
    # j = i at every step leaves everything in place
    assert O.fisher_yates(5, [4, 3, 2, 1]) == [0, 1, 2, 3, 4]
    assert O.fisher_yates(1, []) == [0] and O.fisher_yates(0, []) == []


def test_random_order_draws_are_the_splitmix64_stream():
    # published first outputs of SplitMix64 from state 0
    assert O.splitmix_draws(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    for seed in (0, 1, 123, 2 ** 63 + 5):
        for n in range(7):
            got = O.order(None, [[0]] * n, list(range(n)), "random", seed)
            assert got == O.fisher_yates(n, O.splitmix_draws(seed, max(n - 1, 0)))


@pytest.mark.parametrize("n", [3, 4])
def test_random_order_is_uniform(n):
    trials = 6000 * math.factorial(n) // 6
    counts = {p: 0 for p in itertools.permutations(range(n))}
    for s in range(trials):
        counts[tuple(O.order(None, [[0]] * n, list(range(n)), "random", 1000 + s))] += 1
    expect = trials / len(counts)
    # every permutation appears; each count within 5 standard deviations of its mean
    sd = math.sqrt(expect * (1 - 1 / len(counts)))
    for p, c in counts.items():
        assert abs(c - expect) < 5 * sd, (p, c, expect)
