"""Pins for the oracle's cache model (naive trie + segment model + trace replay).

Each test fixes a result from outside the model itself: numbers the pages print
(tests/golden/*.json, each with its citation), Theorem 3.1's closed form
counted by an independent naive trie, and invariants of LRU leaf-first
eviction checked on a random workload.
"""
import json
import os
import random

import numpy as np
import pytest

from oracle import counts
from oracle.radix_model import CacheError, RadixCacheModel
from oracle.runner import run_trace
from oracle.trie import NaiveTrie
from workloads import configs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def serve(model, prompt, output):
    """Whole request lifecycle at once: match, lock, allocate (evicting), insert, unlock."""
    m, ps, node = model.match(prompt)
    if m == len(prompt):
        m -= 1
        ps = ps[:m]
    model.lock_ref(node, +1)
    need = len(prompt) - m + len(output)
    freed = []
    if need > model.num_free():
        freed = model.evict(need - model.num_free())
    new = model.alloc(need)
    _, leaf, _ = model.insert(list(prompt) + list(output), list(ps) + list(new))
    model.lock_ref(node, -1)
    return m, node, leaf, freed


# ----------------------------------------------------------------- page pins
def test_worked_example_2150_not_6150():
    g = _gold("worked_example.json")
    job = configs.fewshot(n_req=g["n_requests"], prefix=g["shared_prefix_tokens"],
                          suffix=g["query_tokens"], n_decode=0)
    res = run_trace(job)
    n = [job.requests[r].n for r in range(3)]
    m = [res["prefix_len"][r] for r in range(3)]
    assert m == [0, 2000, 2000]
    assert [n[i] - m[i] for i in range(3)] == [g["first_request_computed_tokens"]] + \
        [g["later_request_computed_tokens"]] * 2
    assert counts.no_cache_tokens(n) == g["no_cache_computed_tokens"]
    assert res["computed"] == counts.computed_tokens(m, n) == g["radix_computed_tokens"]
    assert round(100 * (1 - res["computed"] / counts.no_cache_tokens(n))) == g["saving_percent_as_printed"]
    assert counts.hit_rate_cached(m, n) == pytest.approx(counts.hit_rate_computed(res["computed"], n), abs=1e-15)


def test_three_request_split():
    g = _gold("three_requests.json")
    model = RadixCacheModel(1024)
    reqs = [list(s.encode("utf-8")) for s in g["requests"]]
    ms = [serve(model, r, [])[0] for r in reqs]
    # the first request is cold; each later one matches exactly the shared prefix
    assert ms == [0, g["shared_prefix_bytes"], g["shared_prefix_bytes"]]
    dump = model.dump()
    top = [d for d in dump if d[1] == 0]
    assert len(top) == 1 and bytes(top[0][5]).decode() == g["shared_prefix"]
    leaves = [bytes(d[5]).decode() for d in dump if d[1] == top[0][0]]
    assert leaves == g["leaves"]                      # children ordered by first token
    assert len(dump) == 4
    # all slots distinct and none leaked
    st = model.stats()
    assert st["cached"] + st["free"] == 1024 and st["cached"] == 37 + 9


def test_fig3_nine_steps():
    _gold("fig3_events.json")
    rng = np.random.Generator(np.random.PCG64(7))
    L = dict(SYS=12, U1a=4, A1a=4, U1b=20, A1b=20, U2a=10, A2a=10, U2b=10, A2b=10,
             FS=16, Q1=4, Q2=4, Q3=4, Q4=4, U1c=2, A1c=2, ANS0=3, ANS1=3, ANS2=3)
    s = {k: [int(x) for x in rng.integers(0, 32000, v)] for k, v in L.items()}
    model = RadixCacheModel(96)
    node_of = lambda toks: next(d for d in model.dump() if list(d[5]) == list(toks))
    slots_of = lambda nid: list(next(d for d in model.dump() if d[0] == nid)[6])

    # (1) empty
    assert model.dump() == []
    # (2) first turn -> one edge from the root
    m, _, a, fr = serve(model, s["SYS"] + s["U1a"], s["A1a"])
    assert m == 0 and fr == [] and [d[1] for d in model.dump()] == [0]
    # (3) same chat, new turn: reuse the whole edge, append a node
    m, node, c, fr = serve(model, s["SYS"] + s["U1a"] + s["A1a"] + s["U1b"], s["A1b"])
    assert m == 20 and node == a and fr == []
    assert node_of(s["U1b"] + s["A1b"])[1] == a
    # (4) second session: the node holding the system prompt splits
    m, node, d, fr = serve(model, s["SYS"] + s["U2a"], s["A2a"])
    assert m == 12 and fr == []
    sysn = node_of(s["SYS"])
    assert sysn[0] == node and sysn[1] == 0
    assert node_of(s["U1a"] + s["A1a"])[0] == a and node_of(s["U1a"] + s["A1a"])[1] == node
    assert node_of(s["U2a"] + s["A2a"])[1] == node
    # (5) session 2 continues; memory is short; exactly node c (session 1, turn 2) goes
    c_slots = slots_of(c)
    m, node, h, fr = serve(model, s["SYS"] + s["U2a"] + s["A2a"] + s["U2b"], s["A2b"])
    assert fr == c_slots and node == d
    assert node_of(s["U2b"] + s["A2b"])[1] == d
    # (6) unrelated few-shot query: a new child of the root
    m, node, e, fr = serve(model, s["FS"] + s["Q1"], [])
    assert m == 0 and fr == [] and node_of(s["FS"] + s["Q1"])[1] == 0
    # (7) more queries over the same examples: e splits at the examples
    qn = {}
    for q in ("Q2", "Q3", "Q4"):
        m, node, qn[q], fr = serve(model, s["FS"] + s[q], [])
        assert m == 16 and fr == []
    fs = node_of(s["FS"])
    assert fs[1] == 0 and node_of(s["Q1"])[0] == e and node_of(s["Q1"])[1] == fs[0]
    assert all(node_of(s[q])[1] == fs[0] for q in ("Q2", "Q3", "Q4"))
    # (8) session 1 returns: session 2's nodes (g = its turn 1, h = its turn 2) are evicted, leaf first
    g_slots, h_slots = slots_of(d), slots_of(h)
    m, node, _, fr = serve(model, s["SYS"] + s["U1a"] + s["A1a"] + s["U1b"] + s["A1b"] + s["U1c"], s["A1c"])
    assert m == 20 and fr == h_slots + g_slots
    # (9) more answers to question j = Q2: the other query leaves i, k, l are evicted
    i_, k_, l_ = slots_of(e), slots_of(qn["Q3"]), slots_of(qn["Q4"])
    freed = []
    for k in range(3):
        m, node, _, fr = serve(model, s["FS"] + s["Q2"], s[f"ANS{k}"])
        assert m == 19 and node == qn["Q2"]
        freed += fr
    assert freed == i_ + k_ + l_
    st = model.stats()
    assert st["cached"] + st["free"] == 96


# ------------------------------------------------------- Theorem 3.1 pins
@pytest.mark.parametrize("index,expect_c,expect_prompt", [
    (0, 260, 660),            # 200 shared + 3 x 20
    (1, 5200, 131200),        # 2000 shared + 64 x 50
    (2, 13312, 217088),       # 1024 + 8 x 512 + 128 x 64
])
def test_dfs_order_computes_each_edge_once(index, expect_c, expect_prompt):
    job = configs.make(index)
    res = run_trace(job)
    trie = NaiveTrie()
    for r in job.requests:
        trie.insert(r.prompt)
    assert res["computed"] == trie.num_nodes() == expect_c
    assert res["prompt_total"] == expect_prompt
    m = list(res["prefix_len"].values())
    n = [job.requests[r].n for r in res["prefix_len"]]
    assert counts.hit_rate_cached(m, n) == pytest.approx(counts.hit_rate_computed(res["computed"], n), abs=1e-12)
    assert not any(ev[0] == "evict" for ev in res["log"])


def test_self_consistency_matches_naive_trie_per_batch():
    """No eviction here, so every match equals a naive trie of the prompts of earlier batches
    (requests in one batch all match before any of them is inserted), cut to n - 1 when the
    whole prompt is cached."""
    job = configs.make(3)
    res = run_trace(job)
    trie = NaiveTrie()
    expect_c = 0
    for st in job.steps:
        for rid in st.extend:
            r = job.requests[rid]
            m = min(trie.match(r.prompt), r.n - 1)
            assert res["prefix_len"][rid] == m
            expect_c += r.n - m
        for rid in st.extend:
            trie.insert(job.requests[rid].prompt)
    assert res["computed"] == expect_c
    assert not any(ev[0] == "evict" for ev in res["log"])


# ------------------------------------------------ eviction invariants (random)
def _check_conservation(model, private):
    tree = [s for d in model.dump() for s in d[6]]
    pool = tree + [s for v in private.values() for s in v] + list(model.free_set)
    assert sorted(pool) == list(range(model.num_slots))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_workload_invariants(seed):
    rnd = random.Random(seed)
    vocab = 4
    model = RadixCacheModel(300)
    trie_paths = {}
    running = {}          # rid -> (node, private slots, prompt+generated)
    private = {}
    n_evict = 0
    for step in range(400):
        op = rnd.random()
        if op < 0.5 and len(running) < 6:
            prompt = [rnd.randrange(vocab) for _ in range(rnd.randint(1, 30))]
            m, ps, node = model.match(prompt)
            model.lock_ref(node, +1)
            need = len(prompt) - m
            if need > model.num_free():
                snap = {d[0]: d for d in model.dump()}
                asked = need - model.num_free()
                freed = model.evict(asked)
                _check_eviction(model, snap, freed, asked)
                n_evict += 1
            try:
                new = model.alloc(need)
            except CacheError:
                model.lock_ref(node, -1)
                continue
            rid = step
            running[rid] = (node, list(ps) + new, prompt)
            private[rid] = new
        elif running:
            rid = rnd.choice(sorted(running))
            node, row, toks = running.pop(rid)
            private.pop(rid)
            model.insert(toks, row)
            model.lock_ref(node, -1)
        _check_conservation(model, private)
        # match lengths of random queries equal a naive trie built from the cached paths
        paths = _paths(model)
        trie = NaiveTrie()
        for p in paths:
            trie.insert(p)
        q = [rnd.randrange(vocab) for _ in range(12)]
        v, sl = model._walk(q)
        assert len(sl) == trie.match(q)
    assert n_evict > 5
    # drain: everything unlocked -> evicting everything empties the tree
    for rid, (node, row, toks) in list(running.items()):
        model.insert(toks, row)
        model.lock_ref(node, -1)
    model.evict(10 ** 9)
    assert model.dump() == [] and model.num_free() == 300


def _paths(model):
    dump = model.dump()
    by_id = {d[0]: d for d in dump}
    out = []
    for d in dump:
        toks = []
        x = d
        while True:
            toks = list(x[5]) + toks
            if x[1] == 0:
                break
            x = by_id[x[1]]
        out.append(toks)
    return out


def _check_eviction(model, snap, freed, asked):
    after = {d[0] for d in model.dump()}
    removed = [nid for nid in snap if nid not in after]
    # freed slots are exactly the removed nodes' slots, node by node
    order = []
    pos = 0
    slot_owner = {s: nid for nid, d in snap.items() for s in d[6]}
    while pos < len(freed):
        nid = slot_owner[freed[pos]]
        order.append(nid)
        assert list(freed[pos: pos + snap[nid][2]]) == list(snap[nid][6])
        pos += snap[nid][2]
    assert sorted(order) == sorted(removed)
    for nid in removed:
        assert snap[nid][3] == 0                          # never a referenced node
        kids = [x for x in snap.values() if x[1] == nid]
        assert all(k[0] in removed and order.index(k[0]) < order.index(nid) for k in kids)  # leaves first
    ticks = [snap[nid][4] for nid in order]
    assert ticks == sorted(ticks)                         # least recently used first
    # survivors that are evictable leaves are at least as recent as anything evicted
    dump = model.dump()
    parents = {d[1] for d in dump}
    for d in dump:
        if d[3] == 0 and d[0] not in parents and ticks:
            assert d[4] >= ticks[-1]
    # freed >= asked unless nothing evictable remains; never more than one extra leaf
    if len(freed) < asked:
        assert not any(d[3] == 0 and d[0] not in parents for d in dump)
    elif order:
        assert len(freed) - snap[order[-1]][2] < asked


# ---------------------------------------------------------- error behaviour
def test_allocator_and_errors():
    model = RadixCacheModel(8)
    assert model.alloc(3) == [0, 1, 2]
    model.free_slots([1])
    assert model.alloc(2) == [1, 3]
    with pytest.raises(CacheError) as e:
        model.alloc(5)
    assert e.value.code == "ENOMEM" and model.num_free() == 4   # nothing taken
    with pytest.raises(CacheError):
        model.free_slots([5])                                     # already free
    _, _, node = model.match([1, 2])
    assert node == 0
    _, leaf, _ = model.insert([1, 2], [0, 1])
    with pytest.raises(CacheError) as e:
        model.lock_ref(leaf, -1)
    assert e.value.code == "ESTATE"
    model.lock_ref(leaf, +1)
    assert model.evict(10) == []                                  # everything referenced
    model.lock_ref(leaf, -1)
    assert model.evict(1) == [0, 1]                               # whole leaf, may overshoot


def test_insert_duplicate_slots_are_returned():
    model = RadixCacheModel(16)
    a = model.alloc(4)
    model.insert([5, 6, 7, 8], a)
    b = model.alloc(4)                                            # a second copy of the same tokens
    existing, node, tslots = model.insert([5, 6, 7, 8], b)
    assert existing == 4 and tslots == a
    assert sorted(model.free_set) == sorted(set(range(16)) - set(a))
