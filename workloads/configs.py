"""Synthetic request traces for the five shared-prefix workloads.

A trace is data only: the requests (prompt tokens, tokens to be generated) and
a step schedule saying which requests are prefilled ("extend"), which decode
one token, and which finish in each step. It carries no cache state: matched
lengths, slots and evictions are what each side computes from it. The shapes
stand in for the sharing patterns of the pages' benchmarks (few-shot MMLU /
HellaSwag, self-consistency and multi-turn chat; 2312.07104_SGLang notes,
App. A.1 Fig. 9) without using any benchmark item.

Lifecycle that both the harness and the oracle apply to a trace, per step:
  1. extend: in the listed order, match each prompt and lock the matched node;
     then allocate the slots of all unmatched suffixes at once (evicting LRU
     leaves first if the pool is short) and hand them out in request order;
     run attention for the suffix queries; then, in order, insert each prompt,
     lock the new node and unlock the old one.
  2. decode: allocate one slot per listed request at once (evicting if short),
     in request order, for the token generated k-th (output[k], at position
     len(prompt) + k); then attention.
  3. finish: in order, insert prompt + output and unlock the held node.
A match that covers the whole prompt is cut to len(prompt) - 1 so that the
last prompt token is recomputed (the request needs one query to run).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .gen import tokens

SEED_BASE = 0x5EED0000


@dataclass
class Request:
    rid: int
    prompt: np.ndarray            # int32 token ids
    output: np.ndarray            # int32 token ids produced by decode steps
    session: int = -1
    turn: int = -1

    @property
    def n(self) -> int:
        return int(len(self.prompt))


@dataclass
class Step:
    extend: list = field(default_factory=list)
    decode: list = field(default_factory=list)
    finish: list = field(default_factory=list)


@dataclass
class Job:
    name: str
    index: int
    dtype: str                     # "f32" or "bf16"
    h_q: int
    h_kv: int
    d: int
    num_slots: int
    seed: int
    requests: list
    steps: list
    notes: dict = field(default_factory=dict)

    def full_tokens(self, rid: int) -> np.ndarray:
        r = self.requests[rid]
        return np.concatenate([r.prompt, r.output]).astype(np.int32)

    @property
    def gqa(self) -> int:
        return self.h_q // self.h_kv


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _cat(*parts) -> np.ndarray:
    return np.concatenate([np.asarray(p, dtype=np.int32) for p in parts]).astype(np.int32)


def _phase_job(name, index, dtype, h_q, h_kv, d, num_slots, seed, groups, decode_rids, n_decode, reqs):
    """Steps: each group is extended (and finished when it generates nothing), then n_decode
    decode steps over decode_rids, which finish after the last one."""
    steps = []
    for g in groups:
        fin = [rid for rid in g if len(reqs[rid].output) == 0]
        steps.append(Step(extend=list(g), finish=fin))
    for s in range(n_decode):
        steps.append(Step(decode=list(decode_rids), finish=list(decode_rids) if s == n_decode - 1 else []))
    return Job(name, index, dtype, h_q, h_kv, d, num_slots, seed, reqs, steps)


def tiny(n_req=3, prefix=200, suffix=20, n_decode=8, h=4, d=64, num_slots=4096, index=0):
    """Plumbing case: fp32, n_req requests share a prefix; request 0 runs cold first."""
    seed = SEED_BASE + index
    rng = _rng(seed)
    pre = tokens(rng, prefix)
    reqs = []
    for i in range(n_req):
        reqs.append(Request(i, _cat(pre, tokens(rng, suffix)), tokens(rng, n_decode)))
    return _phase_job("tiny", index, "f32", h, h, d, num_slots, seed,
                      [[0], list(range(1, n_req))], list(range(n_req)), n_decode, reqs)


def fewshot(n_req=64, prefix=2000, suffix=50, n_decode=32, h=32, d=128, num_slots=1 << 20,
            dtype="bf16", index=1):
    """Few-shot: n_req requests share a `prefix`-token block of examples, each adds `suffix`."""
    seed = SEED_BASE + index
    rng = _rng(seed)
    pre = tokens(rng, prefix)
    reqs = [Request(i, _cat(pre, tokens(rng, suffix)), tokens(rng, n_decode)) for i in range(n_req)]
    return _phase_job("fewshot", index, dtype, h, h, d, num_slots, seed,
                      [[0], list(range(1, n_req))], list(range(n_req)), n_decode, reqs)


def two_level(system=1024, n_blocks=8, block=512, n_q=16, q=64, n_decode=16, h=32, d=128,
              num_slots=1 << 18, dtype="bf16", index=2):
    """System prefix -> n_blocks exemplar blocks -> n_q questions each (leaves in DFS order)."""
    seed = SEED_BASE + index
    rng = _rng(seed)
    sys_t = tokens(rng, system)
    blocks = [tokens(rng, block) for _ in range(n_blocks)]
    reqs = []
    for b in range(n_blocks):                       # warm-up: system + block b, nothing generated
        reqs.append(Request(len(reqs), _cat(sys_t, blocks[b]), np.zeros(0, np.int32)))
    leaves = []
    for b in range(n_blocks):
        for _ in range(n_q):
            leaves.append(len(reqs))
            reqs.append(Request(len(reqs), _cat(sys_t, blocks[b], tokens(rng, q)), tokens(rng, n_decode)))
    return _phase_job("two_level", index, dtype, h, h, d, num_slots, seed,
                      [[0], list(range(1, n_blocks)), leaves], leaves, n_decode, reqs)


def self_consistency(prefix=4096, n_branch=256, max_branch=1024, n_decode=64, h_q=64, h_kv=8, d=128,
                     num_slots=1 << 18, dtype="bf16", index=3):
    """Self-consistency fork: branches of length U{0..max_branch} off one cold prefix, then decode."""
    seed = SEED_BASE + index
    rng = _rng(seed)
    pre = tokens(rng, prefix)
    lens = rng.integers(0, max_branch + 1, size=n_branch)
    reqs = [Request(0, pre.copy(), np.zeros(0, np.int32))]
    for i in range(n_branch):
        reqs.append(Request(len(reqs), _cat(pre, tokens(rng, int(lens[i]))), tokens(rng, n_decode)))
    br = list(range(1, n_branch + 1))
    job = _phase_job("self_consistency", index, dtype, h_q, h_kv, d, num_slots, seed,
                     [[0], br], br, n_decode, reqs)
    job.notes["branch_lens"] = lens.tolist()
    return job


def _lognormal_len(rng, median, sigma, lo, hi, size):
    x = np.exp(np.log(median) + sigma * rng.standard_normal(size))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def multi_turn(n_sessions=512, max_depth=8, median=200, sigma=1.0, lo=16, hi=2048, system=200,
               h_q=32, h_kv=8, d=128, pool_frac=0.6, max_running=256, max_extend_tokens=16384,
               dtype="bf16", index=4):
    """Multi-turn chat under memory pressure.

    Sessions of U{1..max_depth} turns; user and assistant segments lognormal(median, sigma)
    clipped to [lo, hi]; one shared system prompt. Turn k's prompt is the whole history plus
    the new user segment; its output is the assistant segment. The pool holds pool_frac of
    all distinct tokens. The step schedule is built from lengths alone (FCFS admission while
    the running requests' full footprints fit in the pool and at most max_running run), so it
    never depends on cache state and every step is feasible with leaf-first eviction.
    """
    seed = SEED_BASE + index
    rng = _rng(seed)
    sys_t = tokens(rng, system)
    depth = rng.integers(1, max_depth + 1, size=n_sessions)
    reqs = []
    sess_turns = []
    total_unique = system
    for s in range(n_sessions):
        ul = _lognormal_len(rng, median, sigma, lo, hi, int(depth[s]))
        al = _lognormal_len(rng, median, sigma, lo, hi, int(depth[s]))
        hist = sys_t
        turns = []
        for k in range(int(depth[s])):
            user = tokens(rng, ul[k])
            asst = tokens(rng, al[k])
            prompt = _cat(hist, user)
            turns.append(len(reqs))
            reqs.append(Request(len(reqs), prompt, asst, session=s, turn=k))
            hist = _cat(prompt, asst)
            total_unique += int(ul[k] + al[k])
        sess_turns.append(turns)
    num_slots = int(pool_frac * total_unique)

    steps = []
    ready = [t[0] for t in sess_turns]             # FCFS queue of rids
    running = []                                   # [rid, remaining decode tokens]
    footprint = 0
    next_ready = []
    while ready or running or next_ready:
        ready.extend(next_ready)
        next_ready = []
        st = Step()
        ext_tokens = 0
        while ready and len(running) + len(st.extend) < max_running:
            r = reqs[ready[0]]
            need = r.n + len(r.output)
            if footprint + need > num_slots:
                break
            if st.extend and ext_tokens + r.n > max_extend_tokens:
                break
            st.extend.append(ready.pop(0))
            footprint += need
            ext_tokens += r.n
        for item in running:
            st.decode.append(item[0])
            item[1] -= 1
        done = [it for it in running if it[1] == 0]
        running = [it for it in running if it[1] > 0]
        for rid in st.extend:
            running.append([rid, len(reqs[rid].output)])
        for it in done:
            rid = it[0]
            st.finish.append(rid)
            r = reqs[rid]
            footprint -= r.n + len(r.output)
            turns = sess_turns[r.session]
            if r.turn + 1 < len(turns):
                next_ready.append(turns[r.turn + 1])
        if not (st.extend or st.decode or st.finish):
            raise RuntimeError("multi_turn schedule stalled")
        steps.append(st)
    job = Job("multi_turn", index, dtype, h_q, h_kv, d, num_slots, seed, reqs, steps)
    job.notes.update(total_unique=total_unique, pool_frac=pool_frac, n_sessions=n_sessions)
    return job


CONFIGS = {
    0: tiny,
    1: fewshot,
    2: two_level,
    3: self_consistency,
    4: multi_turn,
}


def make(index: int, **kw) -> Job:
    return CONFIGS[index](**kw)
