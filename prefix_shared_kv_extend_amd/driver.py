"""Run a synthetic request trace (workloads.configs.Job) through RadixRuntime.

The driver plays the role of the model around the attention layer: for every
token whose attention runs, it produces that token's Q/K/V with the seeded
generator (workloads.gen) directly on the GPU, then calls the runtime. It
records the host event log (matches, evictions, allocations, inserts) and hands
each attention output to an optional callback.
"""
from __future__ import annotations

import numpy as np
import torch

from workloads import gen

from .runtime import RadixRuntime


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


class JobRunner:
    def __init__(self, job, device: str = "cuda", out_dtype: torch.dtype = torch.float32,
                 max_reqs: int | None = None, record_log: bool = True, host_slots: int = 0):
        self.job = job
        self.device = torch.device(device)
        self.dtype = torch_dtype(job.dtype)
        self.out_dtype = out_dtype
        self.full = [job.full_tokens(r.rid) for r in job.requests]
        self.hashes = gen.prefix_hashes_batch(self.full, job.seed)
        max_ctx = max(len(f) for f in self.full)
        if max_reqs is None:
            max_reqs = max(len(st.extend) for st in job.steps) + max(len(st.decode) for st in job.steps)
            max_reqs = min(max_reqs, len(job.requests))
        self.log = [] if record_log else None
        self.rt = RadixRuntime(job.num_slots, job.h_q, job.h_kv, job.d, self.dtype, max_reqs, max_ctx,
                               device=device, log=self.log, host_slots=host_slots)
        self.final_rows = {}

    # ------------------------------------------------------------------ inputs
    def qkv(self, pairs):
        """Q, K, V for (rid, position) pairs, in order, generated on the device."""
        h = np.array([self.hashes[r][p] for r, p in pairs], dtype=np.uint64)
        hv = torch.from_numpy(h.view(np.int64)).to(self.device)
        j = self.job
        q = gen.qkv_values(hv, gen.KIND_Q, j.h_q, j.d, j.seed, self.dtype, self.device)
        k = gen.qkv_values(hv, gen.KIND_K, j.h_kv, j.d, j.seed, self.dtype, self.device)
        v = gen.qkv_values(hv, gen.KIND_V, j.h_kv, j.d, j.seed, self.dtype, self.device)
        return q, k, v

    # --------------------------------------------------------------------- run
    def run(self, on_extend=None, on_decode=None, steps=None, progress: int = 0):
        """Execute the trace. Callbacks get (step, batch, positions, o) after each attention call.
        With progress > 0, print a line every `progress` steps."""
        job, rt = self.job, self.rt
        steps = range(len(job.steps)) if steps is None else steps
        for si in steps:
            if progress and si % progress == 0:
                print(f"  step {si}/{len(job.steps)}", flush=True)
            st = job.steps[si]
            rt.step = si
            if st.extend:
                eb = rt.begin_extend([(rid, job.requests[rid].prompt) for rid in st.extend])
                pairs = [(rid, p) for rid, m in zip(eb.rids, eb.prefix_len.tolist())
                         for p in range(m, job.requests[rid].n)]
                q, k, v = self.qkv(pairs)
                o = torch.empty((eb.total_q, job.h_q, job.d), dtype=self.out_dtype, device=self.device)
                rt.run_extend(eb, q, k, v, o)
                if on_extend is not None:
                    on_extend(si, eb, pairs, o)
                rt.end_extend(eb, {rid: job.requests[rid].prompt for rid in eb.rids})
            if st.decode:
                db = rt.begin_decode(st.decode)
                pairs = [(rid, int(n) - 1) for rid, n in zip(db.rids, db.seq_len.tolist())]
                q, k, v = self.qkv(pairs)
                o = torch.empty((len(db.rids), job.h_q, job.d), dtype=self.out_dtype, device=self.device)
                rt.run_decode(db, q, k, v, o)
                if on_decode is not None:
                    on_decode(si, db, pairs, o)
            if st.finish:
                rows = rt.finish_batch([(rid, self.full[rid][: rt.seq_len(rid)]) for rid in st.finish])
                if self.log is not None:
                    for rid, row in zip(st.finish, rows):
                        self.final_rows[rid] = row.tolist()
        return self


def tree_replay(job, host_slots: int = 0):
    """The runtime's tree-side sequence for a whole trace, without device work: per step,
    promote (with a host tier), match and lock the extend batch, one allocation with
    eviction, insert and move the locks; one decode allocation per step; insert and unlock
    at finish. Moves are taken and dropped. Returns (event log, final slot rows, tree,
    computed prompt tokens), the log in the runtime's format."""
    from . import _lib as L
    tree = L.Tree(job.num_slots)
    if host_slots:
        tree.set_host_tier(host_slots)
    log, rows, held, computed = [], {}, {}, 0
    for si, st in enumerate(job.steps):
        if st.extend:
            prompts = [job.requests[rid].prompt for rid in st.extend]
            ip = np.zeros(len(prompts) + 1, dtype=np.int64)
            ip[1:] = np.cumsum([len(p) for p in prompts])
            toks = np.concatenate(prompts)
            if host_slots:
                done, pfreed = tree.promote_batch(toks, ip)
                log.append(("promote", si, tuple(done.tolist()), tuple(pfreed.tolist())))
            pslots, m, nodes = tree.match_prefix_batch(toks, ip, cut_full=True, lock=True)
            for i, rid in enumerate(st.extend):
                log.append(("match", rid, int(m[i]), int(nodes[i])))
            n = np.diff(ip)
            new, freed = tree.alloc_slots_evict(int((n - m).sum()))
            if len(freed):
                log.append(("evict", si, tuple(freed.tolist())))
            log.append(("alloc", si, tuple(new.tolist())))
            off, flat = 0, []
            for i, rid in enumerate(st.extend):
                mi, qi = int(m[i]), int(n[i] - m[i])
                rows[rid] = pslots[ip[i]: ip[i] + mi].tolist() + new[off: off + qi].tolist()
                flat.append(np.asarray(rows[rid], dtype=np.int32))
                off += qi
                computed += qi
            tslots, existing, inodes = tree.insert_batch(toks, np.concatenate(flat), ip)
            for i, rid in enumerate(st.extend):
                log.append(("insert", rid, int(existing[i]), int(inodes[i])))
                rows[rid] = tslots[ip[i]: ip[i + 1]].tolist()
            tree.lock_ref_batch(inodes, +1)
            tree.lock_ref_batch(nodes, -1)
            for i, rid in enumerate(st.extend):
                held[rid] = int(inodes[i])
        if st.decode:
            new, freed = tree.alloc_slots_evict(len(st.decode))
            if len(freed):
                log.append(("evict", si, tuple(freed.tolist())))
            log.append(("alloc", si, tuple(new.tolist())))
            for i, rid in enumerate(st.decode):
                rows[rid].append(int(new[i]))
        if st.finish:
            full = [np.concatenate([job.requests[rid].prompt,
                                    job.requests[rid].output[: len(rows[rid]) - job.requests[rid].n]])
                    for rid in st.finish]
            ip = np.zeros(len(full) + 1, dtype=np.int64)
            ip[1:] = np.cumsum([len(f) for f in full])
            tslots, existing, inodes = tree.insert_batch(
                np.concatenate(full), np.concatenate([np.asarray(rows[r], np.int32) for r in st.finish]), ip)
            for i, rid in enumerate(st.finish):
                log.append(("insert", rid, int(existing[i]), int(inodes[i])))
                rows[rid] = tslots[ip[i]: ip[i + 1]].tolist()
            tree.lock_ref_batch([held.pop(rid) for rid in st.finish], -1)
        if host_slots:
            tree.take_moves()
    return log, rows, tree, computed
