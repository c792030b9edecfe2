"""Replay a request trace through the plain cache model.

TEST INFRASTRUCTURE (oracle). Only tests/, the smoke check and the bench's CPU
baseline leg may use this module.

The request loop follows the pages: traverse (match) -> reuse -> compute the
unmatched suffix only -> insert (hustzhy SGLang post, §2.3 (2); bowenzhou
SGLang review, "Work loop"); a batch is formed after matching, evicting when
memory is short, and the tree is updated after the batch runs (2312.07104_SGLang
notes, App. A.2). The per-step order (extend, then decode, then finish) and the
full-match cut are the trace's documented lifecycle.

Outputs the event log both sides must agree on bit for bit:
  ("promote", step, promoted, freed) with a host tier: per extend request, tokens
                                     promoted (model rule H3), and the device slots freed
  ("match", rid, m, node)            m after the full-match cut
  ("evict", step, freed slots)       only when an allocation had to evict
  ("alloc", step, slots)             one batch allocation per extend / decode call
  ("insert", rid, existing, node)    after extend (prompt) and at finish (prompt+output)
plus each request's final slot row, the final tree dump and the counts.
"""
from __future__ import annotations

from .radix_model import RadixCacheModel


def _alloc(model, log, si, n):
    short = n - model.num_free()
    if short > 0:
        freed = model.evict(short)
        log.append(("evict", si, tuple(freed)))
    slots = model.alloc(n)
    log.append(("alloc", si, tuple(slots)))
    return slots


def run_trace(job, steps=None, host_slots: int = 0):
    """Run ``job.steps`` (or a prefix of them) through a fresh model (with a host tier of
    host_slots rows if > 0: promotion before each extend batch's match). Returns a dict."""
    model = RadixCacheModel(job.num_slots, host_slots)
    log = []
    rows = {}
    held = {}
    prefix_len = {}
    extend_step = {}
    computed = 0
    prompt_total = 0
    matched_total = 0
    steps = job.steps if steps is None else steps
    for si, st in enumerate(steps):
        pending = []
        if host_slots and st.extend:
            done, freed = [], []
            for rid in st.extend:
                d, f = model.promote(job.requests[rid].prompt)
                done.append(d)
                freed += f
            log.append(("promote", si, tuple(done), tuple(freed)))
        for rid in st.extend:
            r = job.requests[rid]
            m, pslots, node = model.match(r.prompt)
            if m == r.n:
                m -= 1
                pslots = pslots[:m]
            log.append(("match", rid, m, node))
            model.lock_ref(node, +1)
            held[rid] = node
            pending.append((rid, m, pslots))
        if st.extend:
            new = _alloc(model, log, si, sum(job.requests[rid].n - m for rid, m, _ in pending))
            off = 0
            for rid, m, pslots in pending:
                r = job.requests[rid]
                rows[rid] = list(pslots) + list(new[off: off + r.n - m])
                off += r.n - m
                prefix_len[rid] = m
                extend_step[rid] = si
                computed += r.n - m
                prompt_total += r.n
                matched_total += m
        for rid in st.extend:
            r = job.requests[rid]
            existing, node, tslots = model.insert(r.prompt, rows[rid][: r.n])
            log.append(("insert", rid, existing, node))
            rows[rid][: r.n] = tslots
            model.lock_ref(node, +1)
            model.lock_ref(held[rid], -1)
            held[rid] = node
        if st.decode:
            new = _alloc(model, log, si, len(st.decode))
            for i, rid in enumerate(st.decode):
                rows[rid].append(new[i])
        for rid in st.finish:
            r = job.requests[rid]
            k = len(rows[rid]) - r.n
            full = list(r.prompt) + list(r.output[:k])
            existing, node, tslots = model.insert(full, rows[rid])
            log.append(("insert", rid, existing, node))
            rows[rid] = tslots
            model.lock_ref(held[rid], -1)
            del held[rid]
    return dict(model=model, log=log, rows=rows, prefix_len=prefix_len, extend_step=extend_step,
                computed=computed, prompt_total=prompt_total, matched_total=matched_total,
                dump=model.dump(), stats=model.stats())
