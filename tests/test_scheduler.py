"""Cache-aware scheduling: Theorem 3.1 pins, and the native scheduler against the oracle.

* Theorem 3.1 (2312.07104_SGLang notes, §3 and App. A.3): with a cache of exactly the
  longest request and one request at a time, a depth-first order of the requests'
  radix tree computes every edge once, so computed tokens = the node count of a naive
  per-token trie of all prompts (exact integers). Longest-shared-prefix-first reaches
  the same optimum (the pages call the two equivalent); FCFS and random orders of a
  shuffled two-level workload do not (the pages' ablation, §6).
* The native ordering (rax_schedule_order) and the batch runs on the C++ tree agree
  bit for bit with the oracle scheduler on the oracle's model: batches, computed
  tokens, and the match / evict / alloc / insert event log.
"""
import numpy as np
import pytest

from oracle import scheduler as O
from oracle.counts import hit_rate_computed
from oracle.trie import NaiveTrie

pytestmark = pytest.mark.filterwarnings("ignore")


def _lib():
    from prefix_shared_kv_extend_amd import _lib
    return _lib


def two_level(seed, n_blocks=4, n_q=6, sys_len=40, blk_len=25, vocab=50):
    """System prompt -> blocks -> questions (notes §3 Figure 3's shapes), shuffled arrival."""
    rng = np.random.default_rng(seed)
    sysp = list(rng.integers(0, vocab, sys_len))
    prompts = []
    for _ in range(n_blocks):
        blk = list(rng.integers(0, vocab, blk_len))
        for _ in range(n_q):
            prompts.append(sysp + blk + list(rng.integers(0, vocab, int(rng.integers(3, 12)))))
    return [prompts[i] for i in rng.permutation(len(prompts))]


def branches(seed, n=20, prefix=60, vocab=50):
    """One shared prefix, ragged branches of 0..30 tokens (self-consistency shape)."""
    rng = np.random.default_rng(seed)
    pre = list(rng.integers(0, vocab, prefix))
    return [pre + list(rng.integers(0, vocab, int(rng.integers(0, 31)))) for _ in range(n)]


def random_prompts(seed, n=30, vocab=6):
    """Small vocabulary: many accidental shared prefixes and full-prompt hits."""
    rng = np.random.default_rng(seed)
    return [list(rng.integers(0, vocab, int(rng.integers(1, 25)))) for _ in range(n)]


def trie_edges(prompts):
    t = NaiveTrie()
    for p in prompts:
        t.insert(p)
    return t.num_nodes()


@pytest.mark.parametrize("make", [lambda: two_level(1), lambda: two_level(2, n_blocks=6, n_q=3),
                                  lambda: branches(3)])
def test_theorem_3_1_dfs_and_lpm_optimal_at_tight_cache(make):
    from prefix_shared_kv_extend_amd import scheduler as S
    prompts = make()
    opt = trie_edges(prompts)
    cap = max(len(p) for p in prompts)                 # cache = the longest request
    total = sum(len(p) for p in prompts)
    for policy in ("dfs", "lpm"):
        r = S.run_prefill(prompts, cap, policy, max_batch=1)
        assert r.computed == opt, (policy, r.computed, opt)
        assert r.hit_rate == pytest.approx(hit_rate_computed(opt, [len(p) for p in prompts]))
    assert opt < total


def test_fcfs_and_random_lose_on_shuffled_two_level():
    from prefix_shared_kv_extend_amd import scheduler as S
    prompts = two_level(1)
    opt = trie_edges(prompts)
    cap = max(len(p) for p in prompts)
    for policy in ("fcfs", "random"):
        assert S.run_prefill(prompts, cap, policy, max_batch=1, seed=11).computed > opt


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("policy", ["fcfs", "lpm", "dfs", "random"])
def test_native_scheduler_matches_oracle(seed, policy):
    from prefix_shared_kv_extend_amd import scheduler as S
    for prompts, cap, kw in ((two_level(seed), None, dict(max_batch=1)),
                             (two_level(seed + 10), 4, dict(max_batch_tokens=150)),
                             (random_prompts(seed), 2, dict(max_batch=3)),
                             (branches(seed), 3, dict(max_batch_tokens=70))):
        slots = max(len(p) for p in prompts) * (cap or 1)
        r = S.run_prefill(prompts, slots, policy, seed=seed, record_log=True, **kw)
        b, c, log = O.run_prefill(prompts, slots, policy, seed=seed, **kw)
        assert r.batches == b and r.computed == c and r.log == log
        assert sorted(x for bb in b for x in bb) == list(range(len(prompts)))


def test_schedule_order_is_read_only_and_matches_definitions():
    L = _lib()
    t = L.Tree(64)
    cached = [5, 1, 2, 3, 4, 0, 0]
    slots = t.alloc_slots(len(cached))
    t.insert(cached, slots)
    before = (t.dump(), t.stats()["clock"])
    prompts = [[5, 1, 9], [7], [5, 1, 2, 3, 4, 0, 0, 8], [5, 1, 2], [7], [0, 1]]
    ip = np.cumsum([0] + [len(p) for p in prompts])
    toks = np.concatenate([np.asarray(p, dtype=np.int32) for p in prompts])
    m = t.prefix_len_batch(toks, ip)
    assert m.tolist() == [2, 0, 7, 3, 0, 0]
    o_lpm, m2 = t.schedule_order(L.SCHED_LPM, toks, ip)
    assert m2.tolist() == m.tolist() and o_lpm.tolist() == [2, 3, 0, 1, 4, 5]
    o_dfs, _ = t.schedule_order(L.SCHED_DFS, toks, ip)
    assert o_dfs.tolist() == sorted(range(6), key=lambda i: prompts[i])
    o_fcfs, _ = t.schedule_order(L.SCHED_FCFS, toks, ip)
    assert o_fcfs.tolist() == list(range(6))
    o_rnd, _ = t.schedule_order(L.SCHED_RANDOM, toks, ip, seed=123)
    assert o_rnd.tolist() == O.order(None, prompts, list(range(6)), "random", 123)
    assert (t.dump(), t.stats()["clock"]) == before            # no split, no tick
    with pytest.raises(L.RaxError):
        t.schedule_order(7, toks, ip)
