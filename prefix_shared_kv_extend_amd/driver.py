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
