"""Host-memory KV tier: the C++ tree against the oracle model, and pins of the oracle.

The pages name the tier (hustzhy SGLang post, §6.1, HiCache: the hottest KV in GPU
memory, the next level in host memory) but not its mechanics; the rules are the
oracle model's readings H1-H5. Pins that do not rest on the model itself:
  * data: every cached token's KV, followed through the recorded moves in order and
    through the caller's own writes, is the KV computed for that token's prefix
    (checked on both the oracle and the C++ tree; a wrong move order, source or
    destination breaks it);
  * nothing is lost with a tier that can hold every token: device + host tokens
    equal the node count of a naive per-token trie of all inserted sequences;
  * a tight device pool plus a large tier reaches, at batch size one, the hit rate of
    an unbounded cache, computed by brute force over earlier prompts;
  * a tier of size zero is the plain cache (same events as the model without a tier).
No kernel is launched here; the device copies are covered by the GPU parity tests.
"""
import os
import random

import numpy as np
import pytest

from oracle import scheduler as O
from oracle.radix_model import CacheError, RadixCacheModel
from oracle.trie import NaiveTrie


@pytest.fixture(scope="module")
def L():
    from prefix_shared_kv_extend_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("librax.so not built (run __graft_entry__.build())")
    return _lib


class Contents:
    """What each device and host slot holds: the prefix (a token tuple) whose KV it is."""

    def __init__(self):
        self.dev, self.host = {}, {}

    def run(self, moves):
        for kind, src, dst in moves:
            if kind == 0:
                self.host[dst] = self.dev.get(src)
            else:
                self.dev[dst] = self.host.get(src)

    def write(self, tokens, slots):
        for i, s in enumerate(slots):
            self.dev[int(s)] = tuple(tokens[: i + 1])

    def check(self, dump):
        path = {0: ()}
        for nid, par, ln, _, _, toks, slots in dump:     # preorder: parents first
            pre = path[par]
            for i, s in enumerate(slots):
                want = pre + tuple(toks[: i + 1])
                got = self.host.get(-1 - s) if s < 0 else self.dev.get(s)
                assert got == want, (nid, i, s)
            path[nid] = pre + tuple(toks)


def _moves_native(tree):
    k, s, d = tree.take_moves()
    return list(zip(k.tolist(), s.tolist(), d.tolist()))


@pytest.mark.parametrize("seed", range(8))
def test_random_ops_with_host_tier_match_oracle(L, seed):
    rnd = random.Random(100 + seed)
    S = rnd.choice([30, 64, 150])
    H = rnd.choice([0, 7, 40, 400])
    vocab = rnd.choice([2, 3, 6])
    model = RadixCacheModel(S, H)
    tree = L.Tree(S)
    tree.set_host_tier(H)
    cm, cn = Contents(), Contents()
    nodes, held = [0], []
    for it in range(400):
        r = rnd.random()
        if r < 0.2:
            toks = [rnd.randrange(vocab) for _ in range(rnd.randint(0, 14))]
            m1, s1, n1 = model.match(toks)
            m2, s2, n2 = tree.match_prefix(toks)
            assert (m1, list(s1), n1) == (m2, s2.tolist(), n2)
            nodes.append(n1)
        elif r < 0.4:
            n = rnd.randint(0, 12)
            try:
                short = n - model.num_free()
                f1 = model.evict(short) if short > 0 else []
                a = model.alloc(n)
            except CacheError:
                a = None
            try:
                b, f2 = tree.alloc_slots_evict(n)
            except L.RaxError as e:
                assert a is None and e.status == L.ENOMEM
                b = None
            if a is not None:
                assert a == b.tolist() and f1 == f2.tolist()
                if a:
                    held.append(a)
        elif r < 0.6 and held:
            slots = held.pop(rnd.randrange(len(held)))
            toks = [rnd.randrange(vocab) for _ in range(len(slots))]
            cm.write(toks, slots)
            cn.write(toks, slots)
            e1, n1, t1 = model.insert(toks, slots)
            e2, n2, t2 = tree.insert(toks, slots)
            assert (e1, n1, list(t1)) == (e2, n2, t2.tolist())
            nodes.append(n1)
        elif r < 0.72:
            node, d = rnd.choice(nodes), rnd.choice([1, -1])
            try:
                model.lock_ref(node, d)
                ea = None
            except CacheError as e:
                ea = e.code
            try:
                tree.lock_ref(node, d)
                eb = None
            except L.RaxError as e:
                eb = {-3: "ESTATE"}.get(e.status, "?")
            assert ea == eb
        elif r < 0.82:
            k = rnd.randint(0, 20)
            assert model.evict(k) == tree.evict_lru(k).tolist()
        else:
            reqs = [[rnd.randrange(vocab) for _ in range(rnd.randint(1, 16))] for _ in range(rnd.randint(1, 3))]
            p1, f1 = [], []
            for q in reqs:
                d, f = model.promote(q)
                p1.append(d)
                f1 += f
            ip = np.cumsum([0] + [len(q) for q in reqs])
            p2, f2 = tree.promote_batch(np.concatenate([np.asarray(q, np.int32) for q in reqs]), ip)
            assert p1 == p2.tolist() and f1 == f2.tolist()
        mm, mn = model.take_moves(), _moves_native(tree)
        assert mm == mn
        cm.run(mm)
        cn.run(mn)
        d1, d2 = model.dump(), tree.dump()
        assert d1 == d2
        cm.check(d1)
        cn.check(d2)
        st, ms = tree.stats(), model.stats()
        assert (st["cached_tokens"], st["locked_tokens"], st["num_nodes"], st["free_slots"],
                st["host_tokens"], st["host_free_slots"]) == \
            (ms["cached"], ms["locked"], ms["nodes"], ms["free"], ms["host"], ms["host_free"])
        assert st["pending_moves"] == 0


def test_large_tier_loses_nothing(L):
    """Every inserted token stays cached on one of the two levels."""
    rnd = random.Random(7)
    seqs = [[rnd.randrange(4) for _ in range(rnd.randint(1, 20))] for _ in range(60)]
    trie = NaiveTrie()
    for q in seqs:
        trie.insert(q)
    S = 25
    for impl in ("model", "native"):
        if impl == "model":
            t = RadixCacheModel(S, 10_000)
            alloc = lambda n: (t.evict(n - t.num_free()) if n > t.num_free() else None, t.alloc(n))[1]
            ins = t.insert
            totals = lambda: (t.stats()["cached"], t.stats()["host"])
        else:
            t = L.Tree(S)
            t.set_host_tier(10_000)
            alloc = lambda n: t.alloc_slots_evict(n)[0].tolist()
            ins = t.insert
            totals = lambda: (t.stats()["cached_tokens"], t.stats()["host_tokens"])
        for q in seqs:
            ins(q, alloc(len(q)))
        dev, host = totals()
        assert dev + host == trie.num_nodes() and dev <= S and host > 0


def _brute_computed(prompts):
    """Unbounded cache, one request at a time: each prompt reuses its longest common prefix with
    any earlier prompt (cut to n - 1 so the last token is computed)."""
    total = 0
    for i, p in enumerate(prompts):
        best = 0
        for q in prompts[:i]:
            k = 0
            while k < min(len(p), len(q)) and p[k] == q[k]:
                k += 1
            best = max(best, k)
        total += len(p) - min(best, len(p) - 1)
    return total


def _workload(seed):
    rng = np.random.default_rng(seed)
    sysp = list(rng.integers(0, 30, 30))
    blocks = [list(rng.integers(0, 30, 20)) for _ in range(5)]
    prompts = [sysp + blocks[int(rng.integers(0, 5))] + list(rng.integers(0, 30, int(rng.integers(2, 10))))
               for _ in range(40)]
    return prompts


@pytest.mark.parametrize("seed", range(3))
def test_tier_recovers_unbounded_hit_rate(L, seed):
    from prefix_shared_kv_extend_amd import scheduler as S
    prompts = _workload(seed)
    cap = max(len(p) for p in prompts)                   # device pool = the longest prompt
    best = _brute_computed(prompts)
    total = sum(len(p) for p in prompts)
    plain = S.run_prefill(prompts, cap, "fcfs", max_batch=1).computed
    tiered = S.run_prefill(prompts, cap, "fcfs", max_batch=1, host_slots=total).computed
    assert tiered == best < plain
    b, c, _ = O.run_prefill(prompts, cap, "fcfs", max_batch=1, host_slots=total)
    assert c == best


@pytest.mark.parametrize("policy", ["fcfs", "lpm"])
@pytest.mark.parametrize("host", [0, 30, 100, 10_000])
def test_native_scheduler_with_tier_matches_oracle(L, policy, host):
    from prefix_shared_kv_extend_amd import scheduler as S
    for seed, (cap, kw) in enumerate(((1, dict(max_batch=1)), (2, dict(max_batch=3)),
                                      (3, dict(max_batch_tokens=90)))):
        prompts = _workload(10 + seed)
        slots = max(len(p) for p in prompts) * cap
        r = S.run_prefill(prompts, slots, policy, seed=seed, record_log=True, host_slots=host, **kw)
        b, c, log = O.run_prefill(prompts, slots, policy, seed=seed, host_slots=host, **kw)
        assert r.batches == b and r.computed == c and r.log == log


def test_tier_of_size_zero_is_the_plain_cache(L):
    prompts = _workload(5)
    slots = max(len(p) for p in prompts) * 2
    a = O.run_prefill(prompts, slots, "lpm", max_batch=2)
    b = O.run_prefill(prompts, slots, "lpm", max_batch=2, host_slots=0)
    assert a == b


def test_host_tier_errors(L):
    t = L.Tree(8)
    with pytest.raises(L.RaxError) as e:
        t.set_host_tier(-1)
    assert e.value.status == L.EINVAL
    t.set_host_tier(4)
    s = t.alloc_slots(3)
    t.insert([1, 2, 3], s)
    assert t.evict_lru(3).tolist() == s.tolist()
    assert t.stats()["host_tokens"] == 3 and t.stats()["pending_moves"] == 3
    with pytest.raises(L.RaxError) as e:
        t.set_host_tier(8)                               # host nodes exist
    assert e.value.status == L.ESTATE
    import ctypes
    lib = L.lib()
    assert lib.rax_run_moves(t._h, None, None, 1, 128, 1, None) == L.EINVAL
    assert lib.rax_run_moves(t._h, ctypes.c_void_p(4096), ctypes.c_void_p(4096), 1, 128, 1, None) == L.ESTATE
    k, src, dst = t.take_moves()
    assert k.tolist() == [0, 0, 0] and src.tolist() == s.tolist() and dst.tolist() == [0, 1, 2]
    d, fr = t.promote_batch(np.array([1, 2, 3, 4], np.int32), [0, 4])
    assert d.tolist() == [3] and len(fr) == 0 and t.stats()["host_tokens"] == 0
    k, src, dst = t.take_moves()
    assert k.tolist() == [1, 1, 1] and src.tolist() == [0, 1, 2] and dst.tolist() == s.tolist()
    assert lib.rax_set_host_tier(t._h, 4, ctypes.c_void_p(12345), None) == L.EINVAL


@pytest.mark.parametrize("host_slots", [0, 300, 20000])
def test_trace_lifecycle_with_tier_matches_oracle(L, host_slots):
    """The runtime's tree-side sequence (driver.tree_replay) equals the oracle's replay."""
    from oracle.runner import run_trace
    from workloads import configs
    job = configs.multi_turn(n_sessions=12, max_depth=3, median=40, lo=4, hi=150, system=30, h_q=8, h_kv=2,
                             max_running=6, max_extend_tokens=400)
    from prefix_shared_kv_extend_amd.driver import tree_replay
    ref = run_trace(job, host_slots=host_slots)
    log, rows, tree, computed = tree_replay(job, host_slots)
    assert log == ref["log"] and rows == ref["rows"] and tree.dump() == ref["dump"]
    assert computed == ref["computed"]
    if host_slots:
        st = tree.stats()
        assert st["demoted_tokens"] > 0 and st["promoted_tokens"] > 0
        assert ref["computed"] < run_trace(job)["computed"]   # the tier saves prefill work
