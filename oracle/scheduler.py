"""Plain model of cache-aware prefill scheduling.

TEST INFRASTRUCTURE (oracle). Only tests/, the smoke check and the bench's CPU
baseline leg may use this module. It shares no code with the native scheduler.

What the pages fix (cited by page title and section):
  * Cache hit rate = cached prompt tokens / prompt tokens
    (2312.07104_SGLang notes, §3 "cache-aware scheduling"; App. A.3 formula
    1 - C / sum of prefill tokens).
  * The scheduler takes all waiting requests, matches each against the radix tree,
    orders them by matched length, longest first, and forms a batch while memory
    suffices, evicting when short; the batch runs, the cache is updated
    (notes App. A.2, steps 1-5; papers.lqhl.me review, "Cache-aware scheduling").
  * Longest-shared-prefix-first is equivalent to a depth-first order of the
    requests' radix tree; with a cache of at least the longest request, DFS order
    computes every edge exactly once (Theorem 3.1, notes App. A.3).
  * FCFS and random orders are the ablation baselines (notes §6 ablation).

Readings where the pages are silent (the native scheduler follows the same rules):
  S1  Ties keep arrival order. The DFS order is the lexicographic order of the
      token sequences (a depth-first walk of the requests' own trie, children in
      ascending token order).
  S2  Admission walks the ordered queue and stops at the first request that does
      not fit: the batch's prompt tokens must fit the pool, its new tokens the
      token budget, its size the request limit; a step always admits one request.
  S3  A batch runs like an extend batch (match and lock every request, one
      allocation with eviction, insert every prompt) and then unlocks: these
      requests only prefill.
  S5  With a host tier, each batch first promotes its requests' host-resident
      prefixes (model rule H3), in batch order; ordering and admission look at the
      device-resident prefix only.
  S4  The random order is a Fisher-Yates shuffle whose k-th draw is SplitMix64
      output k of a stream started at seed + step (Steele, Lea, Flood 2014),
      j = draw mod (i + 1) for i = n-1 down to 1.
"""
from __future__ import annotations

from workloads.gen import GOLDEN, MASK64, splitmix64

from .radix_model import RadixCacheModel


def cached_prefix_len(model: RadixCacheModel, tokens) -> int:
    """Longest cached prefix, read only: a walk of the per-token trie (no split, no tick)."""
    _, slots = model._walk(tokens)
    return len(slots)


def order(model, prompts, waiting, policy: str, seed: int) -> list:
    """Positions (into `waiting`) in admission order under `policy` (S1, S4)."""
    idx = list(range(len(waiting)))
    if policy == "fcfs":
        return idx
    if policy == "lpm":
        m = [cached_prefix_len(model, prompts[r]) for r in waiting]
        return sorted(idx, key=lambda j: -m[j])                      # stable: ties by arrival
    if policy == "dfs":
        return sorted(idx, key=lambda j: list(prompts[waiting[j]]))  # lexicographic, stable
    if policy == "random":
        return fisher_yates(len(idx), splitmix_draws(seed, max(len(idx) - 1, 0)))
    raise ValueError(policy)


def splitmix_draws(seed: int, count: int) -> list:
    """The first `count` outputs of a SplitMix64 stream whose state starts at `seed` (S4)."""
    state = seed & MASK64
    out = []
    for _ in range(count):
        out.append(splitmix64(state))
        state = (state + GOLDEN) & MASK64
    return out


def fisher_yates(n: int, draws) -> list:
    """Fisher-Yates shuffle of [0, n): for i = n-1 down to 1 the next draw picks
    j = draw mod (i + 1) and positions i and j swap (S4)."""
    idx = list(range(n))
    it = iter(draws)
    for i in range(n - 1, 0, -1):
        j = next(it) % (i + 1)
        idx[i], idx[j] = idx[j], idx[i]
    return idx


def run_prefill(prompts, num_slots: int, policy: str = "lpm", max_batch_tokens: int = 1 << 30,
                max_batch: int = 1 << 30, seed: int = 0, host_slots: int = 0):
    """Schedule and run every prompt (all waiting, list order = arrival). Returns
    (batches, computed tokens, event log)."""
    model = RadixCacheModel(num_slots, host_slots)
    waiting = list(range(len(prompts)))
    batches, log, computed, step = [], [], 0, 0
    while waiting:
        m_peek = {r: cached_prefix_len(model, prompts[r]) for r in waiting}
        batch, tot, new = [], 0, 0
        for j in order(model, prompts, waiting, policy, seed + step):
            r = waiting[j]
            n = len(prompts[r])
            need = n - min(m_peek[r], n - 1)
            if batch and (tot + n > num_slots or new + need > max_batch_tokens or len(batch) >= max_batch):
                break
            batch.append(r)
            tot += n
            new += need
        batches.append(batch)
        if host_slots:                                # S5
            done, freed = [], []
            for r in batch:
                d, f = model.promote(prompts[r])
                done.append(d)
                freed += f
            log.append(("promote", step, tuple(done), tuple(freed)))
        # S3: the batch as an extend batch
        held, pending = {}, []
        for r in batch:
            m, pslots, node = model.match(prompts[r])
            n = len(prompts[r])
            if m == n:
                m -= 1
                pslots = pslots[:m]
            log.append(("match", r, m, node))
            model.lock_ref(node, +1)
            held[r] = node
            pending.append((r, m, pslots))
        need = sum(len(prompts[r]) - m for r, m, _ in pending)
        short = need - model.num_free()
        if short > 0:
            log.append(("evict", step, tuple(model.evict(short))))
        new_slots = model.alloc(need)
        log.append(("alloc", step, tuple(new_slots)))
        off, rows = 0, {}
        for r, m, pslots in pending:
            n = len(prompts[r])
            rows[r] = list(pslots) + list(new_slots[off: off + n - m])
            off += n - m
            computed += n - m
        for r in batch:
            existing, node, _ = model.insert(prompts[r], rows[r])
            log.append(("insert", r, existing, node))
        for r in batch:
            model.lock_ref(held[r], -1)
        model.take_moves()
        chosen = set(batch)
        waiting = [r for r in waiting if r not in chosen]
        step += 1
    return batches, computed, log
