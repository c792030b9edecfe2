"""CPU tests of librax's host side: exported symbols, and the C++ radix tree checked
bit for bit against the oracle's segment model (random operation sequences and the
five traces' host lifecycles). No kernel is launched here.
"""
import os
import random
import re

import numpy as np
import pytest

from oracle.radix_model import CacheError, RadixCacheModel
from oracle.runner import run_trace
from workloads import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from prefix_shared_kv_extend_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("librax.so not built (run __graft_entry__.build())")
    return _lib


def declared_symbols():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(rax_[a-z0-9_]+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported(L):
    names = declared_symbols()
    assert {"rax_match_prefix", "rax_insert", "rax_evict_lru", "rax_kv_scatter", "rax_extend_attention",
            "rax_decode_attention"} <= names
    lib = L.lib()
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, missing
    assert set(L.EXPORTS) <= names            # the binding declares nothing that the header lacks
    assert lib.rax_abi_version() == 4


def test_error_codes(L):
    t = L.Tree(8)
    with pytest.raises(L.RaxError) as e:
        t.alloc_slots(9)
    assert e.value.status == L.ENOMEM and t.free_count() == 8
    s = t.alloc_slots(2)
    with pytest.raises(L.RaxError) as e:
        t.free_slots([s[0], s[0]])
    assert e.value.status == L.EINVAL
    with pytest.raises(L.RaxError) as e:
        t.free_slots([7])                            # already free
    assert e.value.status == L.EINVAL
    _, node, _ = t.insert([4, 5], s)
    with pytest.raises(L.RaxError) as e:
        t.lock_ref(node, -1)
    assert e.value.status == L.ESTATE
    with pytest.raises(L.RaxError) as e:
        t.lock_ref(12345, +1)
    assert e.value.status == L.ESTATE
    with pytest.raises(L.RaxError) as e:
        t.insert([1], [6])                           # slot 6 is free: not the caller's
    assert e.value.status == L.EINVAL
    t.lock_ref(node, +1)
    assert len(t.evict_lru(5)) == 0                  # all referenced
    t.lock_ref(node, -1)
    assert t.evict_lru(1).tolist() == s.tolist()
    import ctypes
    lib = L.lib()
    assert lib.rax_tree_create(0, ctypes.byref(ctypes.c_void_p())) == L.EINVAL
    assert lib.rax_kv_scatter(None, None, None, 5, None, None, 1, 1, 128, 1, None) == L.EINVAL
    assert lib.rax_decode_attention(None, None, None, 1, None, 1, 1, None, None, None, 1, 1,
                                    6, 4, 128, 1.0, 1, None, 0, None, 0, None) == L.EINVAL   # h_q % h_kv
    assert lib.rax_extend_attention(None, None, None, None, None, 1, None, 1, 1, None, None, None, None,
                                    1, 1, 0, 4, 4, 96, 1.0, 1, None, 0, None, 0, None) == L.EINVAL  # d = 96
    assert lib.rax_extend_attention(None, None, None, None, None, 1, None, 1, 1, None, None, None, None,
                                    1, 1, -1, 4, 4, 128, 1.0, 1, None, 0, None, 0, None) == L.EINVAL  # length
    # extend workspace: none for many row blocks or unknown lengths, split partials for few
    assert L.attention_workspace_bytes(False, 3150, 32, 32, 128, 2050) == 0
    assert L.attention_workspace_bytes(False, 500, 32, 8, 128, 0) == 0
    assert L.attention_workspace_bytes(False, 500, 32, 8, 128, 2500) > 0


def _both(op, model, tree, *args):
    """Apply the same op to the oracle model and the C++ tree; return both results."""
    try:
        a = getattr(model, op[0])(*args)
        ea = None
    except CacheError as e:
        a, ea = None, e.code
    try:
        b = op[1](tree, *args)
        eb = None
    except Exception as e:                           # RaxError
        b, eb = None, {-1: "EINVAL", -2: "ENOMEM", -3: "ESTATE"}.get(getattr(e, "status", 0), "?")
    return a, ea, b, eb


@pytest.mark.parametrize("seed", range(6))
def test_random_ops_match_oracle(L, seed):
    rnd = random.Random(seed)
    S = rnd.choice([40, 97, 300])
    vocab = rnd.choice([2, 3, 8])
    model = RadixCacheModel(S)
    tree = L.Tree(S)
    nodes = [0]
    held = []                                        # caller-held slots not yet inserted
    for it in range(500):
        r = rnd.random()
        if r < 0.25:
            toks = [rnd.randrange(vocab) for _ in range(rnd.randint(0, 14))]
            m1, s1, n1 = model.match(toks)
            m2, s2, n2 = tree.match_prefix(toks)
            assert (m1, list(s1), n1) == (m2, s2.tolist(), n2)
            nodes.append(n1)
        elif r < 0.45:
            n = rnd.randint(0, 12)
            a, ea, b, eb = _both(("alloc", lambda t, k: t.alloc_slots(k).tolist()), model, tree, n)
            assert ea == eb and a == b
            if a:
                held.append(a)
        elif r < 0.65 and held:
            slots = held.pop(rnd.randrange(len(held)))
            toks = [rnd.randrange(vocab) for _ in range(len(slots))]
            e1, n1, t1 = model.insert(toks, slots)
            e2, n2, t2 = tree.insert(toks, slots)
            assert (e1, n1, list(t1)) == (e2, n2, t2.tolist())
            nodes.append(n1)
        elif r < 0.8:
            node, d = rnd.choice(nodes), rnd.choice([1, -1])
            a, ea, b, eb = _both(("lock_ref", lambda t, x, y: t.lock_ref(x, y)), model, tree, node, d)
            assert ea == eb
        elif r < 0.9:
            k = rnd.randint(0, 20)
            assert model.evict(k) == tree.evict_lru(k).tolist()
        elif r < 0.95 and len(nodes) > 1:
            a, b = rnd.choice(nodes), rnd.choice(nodes)
            x, ex, y, ey = _both(("lca_depth", lambda t, p, q: t.lca_depth(p, q)), model, tree, a, b)
            if ex is None and a in model.segs and b in model.segs:
                assert x == y
        else:
            n = rnd.randint(0, 12)
            try:
                a = model.alloc(n)
                model.free_slots(a)
            except CacheError:
                a = None
            if a is not None:
                b, fr = tree.alloc_slots_evict(n)
                tree.free_slots(b)
        assert model.dump() == tree.dump()
        assert model.num_free() == tree.free_count()
        st = tree.stats()
        ms = model.stats()
        assert (st["cached_tokens"], st["locked_tokens"], st["num_nodes"], st["free_slots"]) == \
            (ms["cached"], ms["locked"], ms["nodes"], ms["free"])


def host_lifecycle(L, job, from_node=False):
    """The trace lifecycle on the C++ tree alone (no kernels); same log format as the oracle.
    from_node: inserts walk from each request's locked node (rax_insert_batch_from), with
    the positions known to hold the tree's slots (the match length, then the prompt)."""
    tree = L.Tree(job.num_slots)
    log, rows, held, trusted = [], {}, {}, {}

    def insert(rid, tokens, slots):
        if not from_node:
            return tree.insert(tokens, slots)
        ts, ex, nodes = tree.insert_batch_from([held[rid]], [trusted[rid]], tokens, slots, [0, len(tokens)])
        return int(ex[0]), int(nodes[0]), ts
    for si, st in enumerate(job.steps):
        pend = []
        for rid in st.extend:
            r = job.requests[rid]
            m, ps, node = tree.match_prefix(r.prompt)
            if m == r.n:
                m -= 1
                ps = ps[:m]
            log.append(("match", rid, m, node))
            tree.lock_ref(node, +1)
            held[rid] = node
            trusted[rid] = m
            pend.append((rid, m, ps.tolist()))
        if st.extend:
            new, freed = tree.alloc_slots_evict(sum(job.requests[rid].n - m for rid, m, _ in pend))
            if len(freed):
                log.append(("evict", si, tuple(freed.tolist())))
            log.append(("alloc", si, tuple(new.tolist())))
            off = 0
            for rid, m, ps in pend:
                k = job.requests[rid].n - m
                rows[rid] = ps + new[off: off + k].tolist()
                off += k
        for rid in st.extend:
            r = job.requests[rid]
            ex, node, ts = insert(rid, r.prompt, np.array(rows[rid][: r.n], dtype=np.int32))
            log.append(("insert", rid, ex, node))
            rows[rid][: r.n] = ts.tolist()
            tree.lock_ref(node, +1)
            tree.lock_ref(held[rid], -1)
            held[rid] = node
            trusted[rid] = r.n
        if st.decode:
            new, freed = tree.alloc_slots_evict(len(st.decode))
            if len(freed):
                log.append(("evict", si, tuple(freed.tolist())))
            log.append(("alloc", si, tuple(new.tolist())))
            for i, rid in enumerate(st.decode):
                rows[rid].append(int(new[i]))
        for rid in st.finish:
            r = job.requests[rid]
            k = len(rows[rid]) - r.n
            ex, node, ts = insert(rid, np.concatenate([r.prompt, r.output[:k]]).astype(np.int32),
                                  np.array(rows[rid], dtype=np.int32))
            log.append(("insert", rid, ex, node))
            rows[rid] = ts.tolist()
            tree.lock_ref(held.pop(rid), -1)
    return log, rows, tree


@pytest.mark.parametrize("from_node", [False, True])
@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])
def test_trace_host_lifecycle_matches_oracle(L, index, from_node):
    job = configs.make(index)
    ref = run_trace(job)
    log, rows, tree = host_lifecycle(L, job, from_node)
    assert len(log) == len(ref["log"])
    for a, b in zip(log, ref["log"]):
        assert a == b
    assert rows == ref["rows"]
    assert tree.dump() == ref["dump"]
    if index == 4:
        assert any(e[0] == "evict" for e in log)     # the 60% pool really forces eviction


def test_decode_step_workspace_check_changes_nothing(L):
    """rax_decode_step checks the workspace before doing anything: too small -> EINVAL with
    ws_needed set, and the tree, the host lengths and the slots stay as they were."""
    import ctypes
    t = L.Tree(64)
    seq = np.array([5, 9], dtype=np.int32)
    a = L.DecodeStepArgs()
    out = np.zeros(2, np.int32)
    fr = np.zeros(64, np.int32)
    a.batch, a.seq_len, a.out_slots, a.out_freed, a.cap = 2, L._p32(seq), L._p32(out), L._p32(fr), 64
    a.h_q, a.h_kv, a.d, a.dt, a.o_dt, a.sm_scale = 8, 2, 128, L.BF16, L.BF16, 0.1
    a.rtt_stride, a.rtt_rows = 16, 2
    for name in ("req_pool_idx", "seq_len_dev", "req_to_token", "q", "k_new", "v_new", "k_pool", "v_pool", "o"):
        setattr(a, name, 4096)                      # never dereferenced: the call stops first
    a.workspace, a.ws_bytes = 4096, 16
    free0 = t.free_count()
    st = L.lib().rax_decode_step(t._h, ctypes.byref(a))
    need = L.lib().rax_attention_workspace_bytes(1, 2, 8, 2, 128, 10)
    assert st == L.EINVAL and a.ws_needed == need > 16
    assert seq.tolist() == [5, 9] and t.free_count() == free0 and a.num_freed == 0


def test_insert_from_node_errors(L):
    """rax_insert_batch_from refuses a start node that is unknown, a host node, deeper than
    the request or whose label differs from the request's tokens (RAX_ESTATE), and a bad
    slot past the walk's start (RAX_EINVAL); the tree is unchanged by a refused request."""
    tree = L.Tree(64)
    a = np.arange(10, 20, dtype=np.int32)
    sa, _ = tree.alloc_slots_evict(10)
    ex, node, _ = tree.insert(a, sa)
    tree.lock_ref(node, +1)
    before = tree.dump()
    b = np.concatenate([a, np.arange(50, 55, dtype=np.int32)])
    sb = np.concatenate([sa, tree.alloc_slots_evict(5)[0]])
    ip = [0, len(b)]
    for start, trusted in ((10 ** 9, 10), (node, -1)):
        with pytest.raises(RuntimeError, match="ESTATE|-3"):
            tree.insert_batch_from([start], [trusted], b, sb, ip)
    with pytest.raises(RuntimeError, match="ESTATE|-3"):   # deeper than the request
        tree.insert_batch_from([node], [5], b[:5], sb[:5], [0, 5])
    c = b.copy()
    c[9] = 99                                               # the start's label differs
    with pytest.raises(RuntimeError, match="ESTATE|-3"):
        tree.insert_batch_from([node], [10], c, sb, ip)
    bad = sb.copy()
    bad[12] = 1000                                          # out of range past the start
    with pytest.raises(RuntimeError, match="EINVAL|-1"):
        tree.insert_batch_from([node], [10], b, bad, ip)
    assert tree.dump() == before
    ts, ex, nodes = tree.insert_batch_from([node], [10], b, sb, ip)
    assert int(ex[0]) == 10 and np.array_equal(ts, sb)
    # a start deeper than the trusted length walks from its ancestor instead
    tree2 = L.Tree(64)
    s2, _ = tree2.alloc_slots_evict(10)
    _, n2, _ = tree2.insert(a, s2)
    own = np.concatenate([s2[:9], tree2.alloc_slots_evict(1)[0]])   # position 9 not the tree's
    ts2, ex2, _ = tree2.insert_batch_from([n2], [9], a, own, [0, 10])
    assert int(ex2[0]) == 10 and np.array_equal(ts2, s2)


def _decode_step_ws_needed(L, seq, hints):
    """ws_needed that rax_decode_step reports for a bf16 MHA 32 x 128 batch (the call stops
    at the workspace check, so no device pointer is dereferenced)."""
    import ctypes
    n = len(seq)
    t = L.Tree(1 << 16)
    seq = np.array(seq, dtype=np.int32)
    a = L.DecodeStepArgs()
    out = np.zeros(n, np.int32)
    fr = np.zeros(64, np.int32)
    a.batch, a.seq_len, a.out_slots, a.out_freed, a.cap = n, L._p32(seq), L._p32(out), L._p32(fr), 64
    a.h_q, a.h_kv, a.d, a.dt, a.o_dt, a.sm_scale = 32, 32, 128, L.BF16, L.BF16, 0.1
    a.rtt_stride, a.rtt_rows = 4096, n
    for name in ("req_pool_idx", "seq_len_dev", "shared_len", "req_to_token", "q", "k_new", "v_new", "k_pool",
                 "v_pool", "o"):
        setattr(a, name, 4096)
    h = np.array(hints, dtype=np.int32) if hints is not None else None
    a.shared_len_host = L._p32(h) if h is not None else None
    a.workspace, a.ws_bytes = 4096, 16
    assert L.lib().rax_decode_step(t._h, ctypes.byref(a)) == L.EINVAL
    assert seq.tolist() == [1600] * n and a.num_freed == 0    # nothing done
    return a.ws_needed


def test_decode_step_host_hints_keep_the_workspace_check(L):
    """A host copy of the hints (which sizes the shared-prefix splits for deeper runs) is
    read before anything is done: the workspace check still comes first and changes
    nothing, and the workspace it asks for covers the hinted layout. Two-level batch (128
    requests: a 1024-token prefix, groups of 16 sharing 512 more) and a few-shot batch
    (one common prefix). (Which kernel form runs is seen in the GPU kernel traces.)"""
    seq = [1600] * 128
    plain = _decode_step_ws_needed(L, seq, None)
    assert plain == L.lib().rax_attention_workspace_bytes(1, 128, 32, 32, 128, 1601)
    two_level = [0 if i == 0 else (1536 if i % 16 else 1024) for i in range(128)]
    few_shot = [0] + [1500] * 127
    for hints in (two_level, few_shot):
        assert _decode_step_ws_needed(L, seq, hints) >= plain
