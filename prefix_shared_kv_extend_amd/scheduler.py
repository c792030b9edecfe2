"""Cache-aware scheduling of prefill batches over the radix tree (host side).

What the pages fix (2312.07104_SGLang notes, §3 "cache-aware scheduling" and App. A.2;
papers.lqhl.me review, "Cache-aware scheduling"): the hit rate is cached prompt tokens
over all prompt tokens; the scheduler takes every waiting request, matches it against
the tree, orders the queue by matched prefix length (longest first) and forms a batch
while memory suffices, evicting when short; then the batch runs and the cache is
updated. Longest-shared-prefix-first approximates a depth-first order of the requests'
radix tree, which Theorem 3.1 (notes App. A.3) shows optimal offline when the cache
holds at least the longest request: every edge is computed exactly once. FCFS and
random orders are the pages' ablation baselines.

The ordering is native (rax_schedule_order: read-only prefix lengths, no split, no
clock tick); this module runs the batches on the tree exactly as the runtime's extend
path does (match and lock, one allocation with eviction, insert, unlock), without
device work, so hit rates of whole request streams can be measured on the host.
"""
from __future__ import annotations

import time
from dataclasses import dataclass, field

import numpy as np

from . import _lib as L

POLICIES = {"fcfs": L.SCHED_FCFS, "lpm": L.SCHED_LPM, "dfs": L.SCHED_DFS, "random": L.SCHED_RANDOM}


@dataclass
class PrefillResult:
    batches: list                      # request ids of each batch, in admission order
    computed: int                      # prompt tokens computed (not served from the cache)
    prompt_total: int
    log: list = field(default_factory=list)   # ("match" | "evict" | "alloc" | "insert", ...) events
    sched_seconds: float = 0.0         # time spent ordering the queue

    @property
    def hit_rate(self) -> float:
        return 1.0 - self.computed / self.prompt_total if self.prompt_total else 0.0


def _flat(prompts, ids):
    lens = [len(prompts[i]) for i in ids]
    ip = np.zeros(len(ids) + 1, dtype=np.int64)
    ip[1:] = np.cumsum(lens)
    toks = np.concatenate([np.asarray(prompts[i], dtype=np.int32) for i in ids]) if ids else np.zeros(0, np.int32)
    return toks, ip


def run_prefill(prompts, num_slots: int, policy: str = "lpm", max_batch_tokens: int = 1 << 30,
                max_batch: int = 1 << 30, seed: int = 0, record_log: bool = False,
                host_slots: int = 0) -> PrefillResult:
    """Admit and run every prompt (all waiting from the start, in list order = arrival).

    Each scheduling step orders the waiting queue under `policy` and admits requests in
    that order while the batch's prompt tokens fit the pool (so its locked prefixes and
    new tokens always fit), its new tokens fit `max_batch_tokens` and it has at most
    `max_batch` requests; the first request of a step is always admitted. A prompt fully
    in the cache still computes its last token (the match is cut to n - 1). The random
    policy draws with seed + step index. With host_slots > 0 the tree has a host tier of that
    many token rows: eviction demotes, and each batch first promotes its requests'
    host-resident prefixes (ordering looks at the device-resident prefix only)."""
    if policy not in POLICIES:
        raise ValueError(f"policy must be one of {sorted(POLICIES)}")
    if any(len(p) > num_slots for p in prompts):
        raise ValueError("a prompt is longer than the pool")
    tree = L.Tree(num_slots)
    if host_slots:
        tree.set_host_tier(host_slots)
    waiting = list(range(len(prompts)))
    res = PrefillResult([], 0, sum(len(p) for p in prompts))
    log = res.log if record_log else None
    step = 0
    while waiting:
        toks, ip = _flat(prompts, waiting)
        t0 = time.perf_counter()
        order, m = tree.schedule_order(POLICIES[policy], toks, ip, seed + step)
        res.sched_seconds += time.perf_counter() - t0
        batch, tot, new = [], 0, 0
        for j in order:
            rid = waiting[j]
            n = len(prompts[rid])
            need = n - min(int(m[j]), n - 1)
            if batch and (tot + n > num_slots or new + need > max_batch_tokens or len(batch) >= max_batch):
                break
            batch.append(rid)
            tot += n
            new += need
        res.batches.append(batch)
        _run_batch(tree, prompts, batch, res, log, step, host_slots > 0)
        chosen = set(batch)
        waiting = [r for r in waiting if r not in chosen]
        step += 1
    return res


def _run_batch(tree, prompts, batch, res, log, step, tier):
    toks, ip = _flat(prompts, batch)
    if tier:
        done, freed = tree.promote_batch(toks, ip)
        if log is not None:
            log.append(("promote", step, tuple(done.tolist()), tuple(freed.tolist())))
    pslots, m, nodes = tree.match_prefix_batch(toks, ip, cut_full=True, lock=True)
    if log is not None:
        for i, rid in enumerate(batch):
            log.append(("match", rid, int(m[i]), int(nodes[i])))
    need = int(sum(len(prompts[rid]) - int(m[i]) for i, rid in enumerate(batch)))
    new, freed = tree.alloc_slots_evict(need)
    if log is not None:
        if len(freed):
            log.append(("evict", step, tuple(freed.tolist())))
        log.append(("alloc", step, tuple(new.tolist())))
    slots, off = [], 0
    for i, rid in enumerate(batch):
        n, mi = len(prompts[rid]), int(m[i])
        slots.append(np.concatenate([pslots[ip[i]: ip[i] + mi], new[off: off + n - mi]]))
        off += n - mi
        res.computed += n - mi
    _, existing, ins_nodes = tree.insert_batch(toks, np.concatenate(slots), ip)
    if log is not None:
        for i, rid in enumerate(batch):
            log.append(("insert", rid, int(existing[i]), int(ins_nodes[i])))
    tree.lock_ref_batch(nodes, -1)     # prefill-only requests finish with their batch
    if tier:
        tree.take_moves()              # no device data here: the moves are only counted
