"""Benchmark of the RadixAttention hot path on one MI355X.

Headline workload (the multi-turn chat configuration, the largest one): one attention
layer at Mixtral-8x7B attention shape (32 query heads, 8 KV heads, head_dim 128), bf16
inputs, fp32 accumulation, bf16 outputs. 512 sessions of 1..8 turns whose user and
assistant segments are lognormal (median 200 tokens) behind one 200-token system prompt;
each turn's prompt is the session history plus the new user segment. The pool holds 60%
of the distinct tokens (878,695 slots), so leaf-first LRU eviction runs throughout. The
trace is 6040 mixed steps: a ragged extend batch (1474 calls, 737,768 suffix queries)
and a decode batch of up to 256 requests (6038 calls, 732,323 decode queries).

One timed step = the whole job from an empty cache, through the C ABI: every trace step's
extend (match, lock, allocate with eviction, fill req_to_token, KV write-back, extend
attention, insert), decode (allocate with eviction, append, write-back, decode
attention) and finish (insert prompt + output, unlock); then the whole tree is evicted so
the next step starts empty. Q/K/V of every call are generated before timing and stay
resident in HBM (about 18 GB).

Passes over the same job (--passes):
  wall     K timed jobs, each between two synchronisations: value (attention tokens per
           second of wall clock, host tree work included), median/p10/p90 of the job time,
           host time to issue a job;
  cold     one job with a 512 MiB scratch write (untimed) before every attention call, so
           L2 and the 256 MB MALL hold nothing of it, and a HIP event pair around the call
           on the stream it runs on: per-call kernel times, the per-kind rates and the
           roofline of the dominant kernel (the headline figures);
  natural  one job with the event pairs and no scratch writes (calls as they run);
  host     one job synchronised after every trace step: the host time of each runtime
           call with no launch waiting for the GPU (the host work alone, by phase).
Beside the headline, each of the other shared-prefix configurations (few-shot, two-level
tree, self-consistency fork) runs its whole trace and times every attention call over
--reps cold repetitions (scratch write before each) and --reps warm ones (back to back):
medians, p10 and p90. The JSON line also carries the CPU oracle's rate on a bounded sample
of the headline workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
COPY_READ_BYTES = 2 * (1 << 15) * 64 * 128 * 2 + (1 << 15) * 4   # --copy-calib: K, V and slot list read
COPY_WRITE_BYTES = 2 * (1 << 15) * 64 * 128 * 2                    # K and V written
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "prefix_shared_kv_extend_amd", "csrc", "kernels", "attention.hip")
METRIC = "attn tokens/s (extend, decode) + % MFMA/HBM peak on radix-cached KV"
HEADLINE = 4                  # workloads.configs index of the headline job (multi-turn)
SIDE = {"fewshot": 1, "two_level": 2, "self_consistency": 3}
DESCR = {
    1: "fewshot: 64 requests x (2000 shared + 50 own) tokens, then 32 decode steps; 32 heads MHA x 128, bf16",
    2: "two_level: 1024-token system prefix -> 8 x 512-token exemplar blocks -> 16 x 64-token questions "
       "(128 leaves), leaf extend then 16 decode steps; 32 heads MHA x 128, bf16",
    3: "self_consistency: 4096-token prefix, 256 branches of U{0..1024} tokens, 64 decode steps; "
       "GQA 64/8 x 128, bf16",
    4: "multi_turn: 512 sessions, 1-8 turns, lognormal(200, 1.0) segments in [16, 2048], 200-token system "
       "prompt, pool = 60% of distinct tokens (878,695 slots, LRU eviction), 6040 mixed extend + decode "
       "steps (<= 256 running); GQA 32/8 x 128, bf16",
}
# kernels that start a launch of each attention entry point (substrings of their names); the
# kernels after one (own parts, merges) belong to it, up to the next launch's first kernel
ENTRY_FIRST = {"decode": "shared_kernel", "extend": "extend_kernel"}
ENTRY_REST = ("own_", "merge_kernel")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed jobs of the wall pass")
    ap.add_argument("--warmup", type=int, default=1, help="untimed jobs before the wall pass")
    ap.add_argument("--reps", type=int, default=20, help="cold and warm repetitions per call (side sections)")
    ap.add_argument("--passes", default="wall,cold,natural,host", help="comma list of wall, cold, natural, host")
    ap.add_argument("--flush-mib", type=int, default=512, help="scratch written before each cold call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the sections beside the headline (other configurations, scheduler, host tier, "
                         "projection)")
    ap.add_argument("--only", default=None, choices=sorted(SIDE),
                    help="run only this configuration's per-call section (cold and warm reps) and print it")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--traffic", default=TRAFFIC_JSON, help="counter summary with HBM bytes per launch")
    ap.add_argument("--write-traffic", default=None, metavar="DIR",
                    help="condense rocprofv3 counter runs in DIR into profiles/traffic.json and exit")
    ap.add_argument("--summarize-trace", default=None, metavar="CSV",
                    help="print a markdown summary of a rocprofv3 kernel trace (per kernel; GPU idle between "
                         "kernels over the window of the hot path's kernels) and exit")
    ap.add_argument("--summarize-counters", default=None, nargs="+", metavar="DIR",
                    help="print a markdown summary of rocprofv3 counter runs (one directory per pass) and exit")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain copy kernel of known size (for counter scaling) and exit")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers
def pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q)) if len(xs) else None


def stats(xs):
    return {"median": pct(xs, 50), "p10": pct(xs, 10), "p90": pct(xs, 90), "n": len(xs)}


class Flusher:
    """An untimed write of a scratch buffer larger than L2 (8 x 4 MB) and the 256 MB MALL, so
    that the next call finds nothing of its inputs in either."""

    def __init__(self, dev, mib):
        import torch
        self.buf = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n & 0xFF)


def extend_flops(job, pairs):
    """QK^T and PV over keys 0..p of every suffix query (causal): 4 D h_q (p + 1) each."""
    p = np.fromiter((q for _, q in pairs), dtype=np.float64, count=len(pairs))
    return float(4.0 * job.d * job.h_q * (p + 1).sum())


def decode_bytes(job, n_req, n_keys, distinct):
    """Distinct K/V rows read (each slot once), Q in and O out, 4 B per req_to_token entry."""
    return distinct * 2 * job.h_kv * job.d * 2 + 2 * n_req * job.h_q * job.d * 2 + n_keys * 4


def distinct_slots(rt, db):
    """Number of distinct slot ids in the batch's req_to_token rows (device sort, no sync):
    the K/V rows the decode call must read at least once."""
    import torch
    dev = rt.rtt.device
    width = int(db.max_seq_len)
    lens = torch.from_numpy(db.seq_len.astype(np.int32)).to(dev, non_blocking=True)
    keys = rt.rtt[db.dev["req_pool_idx"].long(), :width]
    inside = torch.arange(width, device=dev)[None, :] < lens[:, None]
    k = torch.where(inside, keys, torch.full_like(keys, -1)).flatten().sort().values
    return ((k[1:] != k[:-1]) & (k[1:] >= 0)).sum() + (k[0] >= 0).to(torch.int64)


# ------------------------------------------------------------------ the headline job
def call_plan(job):
    """Every attention call of one job from an empty cache, in order: (step, kind, pairs of
    (request, position)). Match lengths come from the tree alone (the runtime's sequence of
    tree calls, driver.tree_replay), so nothing runs on the GPU."""
    from prefix_shared_kv_extend_amd.driver import tree_replay
    log, _, tree, _ = tree_replay(job)
    tree.close()
    matches = iter([e for e in log if e[0] == "match"])
    length, calls = {}, []
    for si, st in enumerate(job.steps):
        if st.extend:
            pairs = []
            for rid in st.extend:
                ev = next(matches)
                assert ev[1] == rid
                n = job.requests[rid].n
                pairs += [(rid, p) for p in range(ev[2], n)]
                length[rid] = n
            calls.append((si, "extend", pairs))
        if st.decode:
            pairs = []
            for rid in st.decode:
                pairs.append((rid, length[rid]))
                length[rid] += 1
            calls.append((si, "decode", pairs))
    return calls


class Inputs:
    """Q/K/V of every attention call of the job, generated on the device before timing."""

    def __init__(self, runner, calls):
        import torch
        job = runner.job
        self.calls = calls
        self.qkv = [runner.qkv(pairs) for _, _, pairs in calls]
        most = max(len(p) for _, _, p in calls)
        self.o = torch.empty((most, job.h_q, job.d), dtype=torch.bfloat16, device=runner.device)
        self.flops = [extend_flops(job, p) if kind == "extend" else 0.0 for _, kind, p in calls]
        torch.cuda.synchronize()


PHASES = ("begin_extend", "run_extend", "end_extend", "begin_decode", "run_decode", "finish")


def run_job(runner, inp, pre=None, timed=False, after_decode=None, phases=None):
    """One job pass through the runtime. pre: called right before each attention call is
    issued; timed: a HIP event pair around every attention call (rt.timers); phases: a dict
    that accumulates the host time of each runtime call, with the device synchronised after
    every trace step (so no launch waits for the GPU and the times are host work alone)."""
    import torch
    rt, job = runner.rt, runner.job
    rt.timers = {} if timed else None
    rt.pre_attention = pre
    clock = time.perf_counter

    def tick(name, t0):
        t1 = clock()
        if phases is not None:
            phases[name] = phases.get(name, 0.0) + (t1 - t0)
        return t1

    i = 0
    for si, st in enumerate(job.steps):
        rt.step = si
        t = clock()
        if st.extend:
            eb = rt.begin_extend([(rid, job.requests[rid].prompt) for rid in st.extend])
            t = tick("begin_extend", t)
            q, k, v = inp.qkv[i]
            rt.run_extend(eb, q, k, v, inp.o[: q.shape[0]])
            t = tick("run_extend", t)
            rt.end_extend(eb)
            t = tick("end_extend", t)
            i += 1
        if st.decode:
            db = rt.begin_decode(st.decode)
            t = tick("begin_decode", t)
            q, k, v = inp.qkv[i]
            rt.run_decode(db, q, k, v, inp.o[: q.shape[0]])
            t = tick("run_decode", t)
            if after_decode is not None:
                after_decode(i, db)
            i += 1
        if st.finish:
            rt.finish_batch([(rid, runner.full[rid][: rt.seq_len(rid)]) for rid in st.finish])
            t = tick("finish", t)
        if phases is not None:
            torch.cuda.synchronize()
    rt.tree.evict_lru(rt.num_slots)             # the cache yields everything: next job starts empty
    timers, rt.timers, rt.pre_attention = rt.timers, None, None
    return timers


def per_kind(job, inp, timers, dec_bytes):
    """Per-call times (us) and work of one timed pass, by kind."""
    out = {}
    for kind in ("extend", "decode"):
        idx = [i for i, c in enumerate(inp.calls) if c[1] == kind]
        us = [a.elapsed_time(b) * 1e3 for a, b in timers.get(kind, [])]
        assert len(us) == len(idx), (kind, len(us), len(idx))
        work = [inp.flops[i] for i in idx] if kind == "extend" else [dec_bytes[i] for i in idx]
        out[kind] = (us, work)
    return out


def summarize_kind(kind, us, work, n_tok):
    tot_us, tot_w = sum(us), sum(work)
    if kind == "extend":
        rate = tot_w / (tot_us * 1e-6) / 1e12
        per_call = [w / (u * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS for u, w in zip(us, work)]
        return {"us_per_step": tot_us, "calls": len(us), "tok_s_kernel": n_tok / (tot_us * 1e-6),
                "tflops": rate, "frac_mfma_peak": rate / MFMA_BF16_PEAK_TFLOPS,
                "per_call_frac": stats(per_call)}
    rate = tot_w / (tot_us * 1e-6) / 1e9
    per_call = [w / (u * 1e-6) / 1e9 / HBM_PEAK_GBS for u, w in zip(us, work)]
    return {"us_per_step": tot_us, "calls": len(us), "tok_s_kernel": n_tok / (tot_us * 1e-6),
            "gbs_unique": rate, "frac_hbm_peak": rate / HBM_PEAK_GBS, "mb_per_call": tot_w / len(us) / 1e6,
            "per_call_frac": stats(per_call)}


def headline(args, dev):
    import torch
    from prefix_shared_kv_extend_amd.driver import JobRunner
    from workloads import configs
    job = configs.make(HEADLINE)
    calls = call_plan(job)
    runner = JobRunner(job, device="cuda:0", out_dtype=torch.bfloat16, record_log=False)
    inp = Inputs(runner, calls)
    n_ext = sum(len(p) for _, k, p in calls if k == "extend")
    n_dec = sum(len(p) for _, k, p in calls if k == "decode")
    passes = set(args.passes.split(","))
    unknown = passes - {"wall", "cold", "natural", "host"}
    if unknown:
        raise SystemExit(f"bench.py: unknown passes {sorted(unknown)}")
    out = {"config": {"workload": DESCR[HEADLINE], "extend_tokens_per_step": n_ext,
                      "decode_tokens_per_step": n_dec, "prompt_tokens_per_step": sum(r.n for r in job.requests),
                      "extend_calls_per_step": sum(1 for c in calls if c[1] == "extend"),
                      "decode_calls_per_step": sum(1 for c in calls if c[1] == "decode"),
                      "trace_steps": len(job.steps), "pool_slots": job.num_slots}}
    out["hit_rate"] = 1.0 - n_ext / out["config"]["prompt_tokens_per_step"]

    if "wall" in passes:
        for _ in range(args.warmup):
            run_job(runner, inp)
        torch.cuda.synchronize()
        walls, issue = [], []
        for _ in range(args.steps):
            t0 = time.perf_counter()
            run_job(runner, inp)
            t1 = time.perf_counter()          # the host never waits inside a job
            torch.cuda.synchronize()
            t2 = time.perf_counter()
            walls.append(t2 - t0)
            issue.append(t1 - t0)
        out["wall"] = {"value": (n_ext + n_dec) * len(walls) / sum(walls), "ms_per_step": sum(walls) * 1e3 / len(walls),
                       "ms_stats": stats([w * 1e3 for w in walls]), "host_issue_ms": sum(issue) * 1e3 / len(issue)}

    # distinct K/V rows of every decode call, counted on the device after the call (outside
    # its event pair) in the first timed pass
    counts, dec_bytes = {}, {}

    def count(i, db):
        counts[i] = distinct_slots(runner.rt, db)

    def finish_counts():
        for i, c in enumerate(calls):
            if c[1] == "decode" and i not in dec_bytes:
                pairs = c[2]
                dec_bytes[i] = decode_bytes(job, len(pairs), sum(p + 1 for _, p in pairs), int(counts[i]))

    for name in ("cold", "natural"):
        if name not in passes:
            continue
        flush = Flusher(dev, args.flush_mib) if name == "cold" else None
        timers = run_job(runner, inp, pre=flush, timed=True, after_decode=None if dec_bytes else count)
        torch.cuda.synchronize()
        finish_counts()
        res = per_kind(job, inp, timers, dec_bytes)
        out[name] = {k: summarize_kind(k, *res[k], n_ext if k == "extend" else n_dec) for k in res}
        del flush
    if "host" in passes:
        # host work alone: every trace step synchronised, so no launch waits for the GPU
        ph = {}
        run_job(runner, inp, phases=ph)
        torch.cuda.synchronize()
        out["host"] = {"ms_per_step": sum(ph.values()) * 1e3, "phases_ms": {k: ph.get(k, 0.0) * 1e3 for k in PHASES}}
    from prefix_shared_kv_extend_amd import _lib
    assert _lib.device_errors() == 0
    out["_job"] = job
    out["_inp"] = None
    return out


def roofline_of(cold, traffic_path):
    ext, dec = cold["extend"], cold["decode"]
    if ext["us_per_step"] >= dec["us_per_step"]:
        roof = {"kernel": "extend attention (extend_kernel, bf16, D=128)", "bound": "mfma",
                "achieved": ext["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ext["frac_mfma_peak"], "launches_per_step": ext["calls"],
                "avg_launch_us": ext["us_per_step"] / ext["calls"]}
        entry = "extend"
    else:
        roof = {"kernel": "decode attention (shared_kernel + own part + merge_kernel)", "bound": "hbm",
                "achieved": dec["gbs_unique"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec["frac_hbm_peak"],
                "launches_per_step": dec["calls"], "avg_launch_us": dec["us_per_step"] / dec["calls"],
                "algorithmic_bytes_per_launch": dec["mb_per_call"] * 1e6}
        entry = "decode"
    roof["traffic"] = load_traffic(entry, traffic_path)
    roof["timing"] = "cold: 512 MiB scratch write before every call, HIP events on the call's stream"
    return roof


# ------------------------------------------------------------------ side configurations
def side_config(index, reps, flush):
    """Run configuration `index` through the runtime and time each attention call: after
    the call runs in the job, 2 untimed repetitions, `reps` cold ones (a scratch write before
    each, HIP events around the call) and `reps` warm ones (back to back). Decode calls are
    replayed through rax_decode_attention_hinted in the layout the decode step chose; extend
    calls through rax_extend_attention with the call's own inputs."""
    import torch
    from prefix_shared_kv_extend_amd import _lib as L
    from prefix_shared_kv_extend_amd.driver import JobRunner
    from workloads import configs
    job = configs.make(index)
    runner = JobRunner(job, out_dtype=torch.bfloat16, record_log=False)
    rt = runner.rt
    rec = {"extend": [], "decode": []}

    def measure(fn):
        fn()
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2 * reps)]
        for a, b in ev[:reps]:
            flush()
            a.record()
            fn()
            b.record()
        for a, b in ev[reps:]:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in ev]
        return us[:reps], us[reps:]

    def on_extend(si, eb, pairs, o):
        q, k, v = runner.qkv(pairs)
        ws = rt._workspace(L.attention_workspace_bytes(False, eb.total_q, job.h_q, job.h_kv, job.d, eb.max_kv_len))
        fn = lambda: L.extend_attention(q, k, v, rt.k_pool, rt.v_pool, rt.rtt, eb.dev["req_pool_idx"],
                                        eb.dev["prefix_len"], eb.dev["qo_indptr"], o, shared_len=eb.dev["shared_len"],
                                        workspace=ws, max_kv_len=eb.max_kv_len)
        cold, warm = measure(fn)
        rec["extend"].append({"queries": len(pairs), "requests": len(eb.rids), "work": extend_flops(job, pairs),
                              "cold": cold, "warm": warm})

    def on_decode(si, db, pairs, o):
        q = torch.randn((len(db.rids), job.h_q, job.d), device=o.device).to(torch.bfloat16)

        def call(w):
            return L.decode_attention_hinted(q, rt.k_pool, rt.v_pool, rt.rtt, db.dev["req_pool_idx"], db.dev["seq_len"],
                                             db.max_seq_len, o, db.seq_len, db.shared_len_host, workspace=w,
                                             shared_len=db.dev["shared_len"])
        ws = rt._workspace(call(None))
        cold, warm = measure(lambda: call(ws))
        n_keys = int(db.seq_len.astype(np.int64).sum())
        rec["decode"].append({"requests": len(db.rids), "work": decode_bytes(job, len(db.rids), n_keys,
                                                                            int(distinct_slots(rt, db))),
                              "cold": cold, "warm": warm})

    runner.run(on_extend=on_extend, on_decode=on_decode)
    assert L.device_errors() == 0

    def agg(kind, items):
        if not items:
            return None
        res = {"calls": len(items)}
        for temp in ("cold", "warm"):
            med = [pct(it[temp], 50) for it in items]
            p10 = [pct(it[temp], 10) for it in items]
            p90 = [pct(it[temp], 90) for it in items]
            w = sum(it["work"] for it in items)
            if kind == "extend":
                rate = lambda us: w / (sum(us) * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS
                key = "frac_mfma_peak"
            else:
                rate = lambda us: w / (sum(us) * 1e-6) / 1e9 / HBM_PEAK_GBS
                key = "frac_hbm_peak"
            res[temp] = {"us_per_call_median": sum(med) / len(med), key: rate(med),
                         key + "_p10_time": rate(p90), key + "_p90_time": rate(p10)}
        if kind == "extend":
            res["per_call"] = [{"queries": it["queries"], "requests": it["requests"], "gflop": it["work"] / 1e9,
                                "cold_us": stats(it["cold"]), "warm_us": stats(it["warm"]),
                                "cold_frac_mfma_peak": it["work"] / (pct(it["cold"], 50) * 1e-6) / 1e12
                                / MFMA_BF16_PEAK_TFLOPS} for it in items]
        else:
            res["mb_per_call"] = sum(it["work"] for it in items) / len(items) / 1e6
            res["requests"] = items[0]["requests"]
        return res

    return {"workload": DESCR[index], "reps": reps, "extend": agg("extend", rec["extend"]),
            "decode": agg("decode", rec["decode"])}


# ------------------------------------------------------------------ other sections
def scheduler_ablation():
    """Cache-aware scheduling on the host (no device work): the two-level workload's 136
    prompts (1024-token system prompt, 8 blocks of 512, 16 questions of 64 per block) in a
    seeded random arrival order, all waiting at once. Computed prompt tokens and hit rate per
    policy, against Theorem 3.1's optimum (each edge of the requests' radix tree once):
      tight: a pool of exactly the longest prompt, one request per batch (the theorem's case);
      batched: a pool of 16384 slots, at most 4096 new tokens per batch."""
    from prefix_shared_kv_extend_amd import _lib
    from prefix_shared_kv_extend_amd import scheduler as S
    from workloads import configs
    job = configs.make(2)
    rng = np.random.default_rng(7)
    prompts = [job.requests[i].prompt for i in rng.permutation(len(job.requests))]
    total = sum(len(pr) for pr in prompts)
    # the optimum: every distinct token prefix computed once = the tokens a tree large
    # enough for all prompts caches after inserting each of them
    every = _lib.Tree(total)
    for pr in prompts:
        m, slots, _ = every.match_prefix(pr)
        every.insert(pr, np.concatenate([slots[:m], every.alloc_slots(len(pr) - m)]))
    opt = every.stats()["cached_tokens"]
    every.close()
    out = {"workload": "two_level: 136 prompts (8 x 1536, 128 x 1600), shuffled arrival",
           "prompt_tokens": total, "optimal_computed": opt, "optimal_hit_rate": 1 - opt / total}
    for regime, kw in (("tight", dict(num_slots=max(len(pr) for pr in prompts), max_batch=1)),
                       ("batched", dict(num_slots=16384, max_batch_tokens=4096))):
        res = {}
        for pol in ("lpm", "dfs", "fcfs", "random"):
            r = S.run_prefill(prompts, policy=pol, seed=1, **kw)
            res[pol] = {"computed": r.computed, "hit_rate": r.hit_rate, "batches": len(r.batches),
                        "order_us_per_step": r.sched_seconds / len(r.batches) * 1e6}
        out[regime] = res
    return out


def host_tier_measure(dev):
    """Host-memory KV tier. Hit rate: the multi-turn trace (512 sessions, GQA 32/8) with the
    device pool cut to 30% of its distinct tokens, replayed on the tree alone (the runtime's
    sequence of tree calls) without a tier and with tiers of 25% and 50% of the distinct
    tokens. Bandwidth: 65536 tokens of 32 x 128 bf16 K and V (1 GiB each way) demoted to the
    pinned tier and promoted back by the move kernels, HIP events on the current stream."""
    import torch
    from prefix_shared_kv_extend_amd import _lib
    from prefix_shared_kv_extend_amd.driver import tree_replay
    from workloads import configs
    job = configs.multi_turn(pool_frac=0.3)
    uniq = job.notes["total_unique"]
    prompt = sum(r.n for r in job.requests)
    out = {"workload": f"multi_turn: 512 sessions, pool {job.num_slots} slots = 30% of {uniq} distinct tokens",
           "prompt_tokens": prompt}
    for name, frac in (("no_tier", 0.0), ("tier_25pct", 0.25), ("tier_50pct", 0.5)):
        hs = int(frac * uniq)
        _, _, tree, computed = tree_replay(job, hs)
        st = tree.stats()
        out[name] = {"host_slots": hs, "computed": computed, "hit_rate": 1 - computed / prompt,
                     "demoted": st["demoted_tokens"], "promoted": st["promoted_tokens"]}
    n, h, d = 65536, 32, 128
    g = torch.Generator(device=dev).manual_seed(5)
    kp = torch.randn((n, h, d), generator=g, device=dev).to(torch.bfloat16)
    vp = torch.randn((n, h, d), generator=g, device=dev).to(torch.bfloat16)
    kh = torch.empty((n, h, d), dtype=torch.bfloat16, pin_memory=True)
    vh = torch.empty_like(kh, pin_memory=True)
    t = _lib.Tree(n)
    t.set_host_tier(n, kh, vh)
    seq = 1024
    toks = np.arange(n, dtype=np.int32)
    for i in range(n // seq):
        t.insert(toks[i * seq: (i + 1) * seq], t.alloc_slots(seq))
    ip = np.arange(0, n + 1, seq, dtype=np.int64)
    times = {"demote": [], "promote": []}
    for rep_i in range(3):
        for kind in ("demote", "promote"):
            if kind == "demote":
                t.evict_lru(n)
            else:
                t.promote_batch(toks, ip)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            t.run_moves(kp, vp)
            b.record()
            torch.cuda.synchronize()
            if rep_i:
                times[kind].append(a.elapsed_time(b) * 1e-3)
    nbytes = n * 2 * h * d * 2
    for kind, v in times.items():
        out[f"{kind}_gbs"] = nbytes / (sum(v) / len(v)) / 1e9
    out["moved_bytes"] = nbytes
    assert _lib.device_errors() == 0
    return out


def projection_measure(dev):
    """QKV projection fused with the KV write-back, on the cached few-shot extend batch:
    3150 new tokens, hidden 4096, 32 heads x 128 (MHA), so W is [12288, 4096]. Fused: one
    kernel writes Q, the contiguous K/V and the pool rows. Unfused: the same GEMM without
    pool writes, then rax_kv_scatter from the contiguous K/V. Beside them, the projection
    alone and the library GEMM (torch.matmul) of the same shape. HIP events around 10 calls
    of each; the four are timed in turn, 7 rounds, and each reports its median (the clock
    drifts as the GPU warms, so a fixed order would favour the first)."""
    import torch
    from prefix_shared_kv_extend_amd import _lib
    from workloads.gen import projection_inputs
    t, hidden, h, d = 3150, 4096, 32, 128
    x, w = projection_inputs(5, t, hidden, 3 * h * d)
    x, w = x.to(torch.bfloat16).to(dev), w.to(torch.bfloat16).to(dev)
    loc = (torch.randperm(1 << 16, generator=torch.Generator().manual_seed(1))[:t]).to(torch.int32).to(dev)
    kp = torch.zeros((1 << 16, h, d), dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    q, k, v = _lib.qkv_project(x, w, h, h)

    def fused():
        _lib.qkv_project(x, w, h, h, out_loc=loc, k_pool=kp, v_pool=vp, q_out=q, k_ext=k, v_ext=v)

    def projection():
        _lib.qkv_project(x, w, h, h, q_out=q, k_ext=k, v_ext=v)

    def unfused():
        projection()
        _lib.kv_scatter(k, v, loc, kp, vp)

    def library():
        torch.matmul(x, w.t())

    out = {"workload": "cached few-shot extend batch: 3150 tokens, hidden 4096, 32 heads x 128 (W 12288 x 4096)"}
    flops = 2.0 * t * hidden * 3 * h * d
    fns = (("fused", fused), ("gemm_then_scatter", unfused), ("projection_only", projection),
           ("library_gemm_same_shape", library))
    times = {name: [] for name, _ in fns}
    for _ in range(3):
        for _, fn in fns:
            fn()
    for _ in range(7):
        for name, fn in fns:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(10):
                fn()
            b.record()
            torch.cuda.synchronize()
            times[name].append(a.elapsed_time(b) * 1e3 / 10)
    for name, _ in fns:
        us = statistics.median(times[name])
        out[name] = {"us": us, "tflops": flops / (us * 1e-6) / 1e12,
                     "frac_mfma_peak": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    out["saved_us"] = out["gemm_then_scatter"]["us"] - out["fused"]["us"]
    assert _lib.device_errors() == 0
    return out


def cpu_baseline(job, seconds):
    """The oracle (fp64 recompute from scratch) on a bounded sample of the headline job:
    random requests, each with all of its attention queries (its extend suffix and every
    decode position) recomputed from scratch over its full sequence."""
    import torch
    from oracle.attention import outputs_from_scratch
    threads = len(os.sched_getaffinity(0))
    torch.set_num_threads(threads)
    first = {}
    for _, kind, pairs in call_plan(job):
        if kind == "extend":
            for rid, p in pairs:
                first.setdefault(rid, p)
    rng = np.random.default_rng(0)
    done, reqs, keys = 0, 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        rid = int(rng.integers(0, len(job.requests)))
        r = job.requests[rid]
        pos = list(range(first[rid], r.n + len(r.output)))
        outputs_from_scratch(job.full_tokens(rid), pos, job.h_q, job.h_kv, job.d, job.seed, job.dtype)
        done += len(pos)
        keys += sum(p + 1 for p in pos)
        reqs += 1
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "attn tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reqs} random multi-turn requests, each with all of its queries ({done} in total: the extend "
                      f"suffix and every decode position, {keys / done:.0f} keys per query on average) recomputed "
                      f"from scratch over its full sequence in fp64 ({dt:.1f} s)"}


# ------------------------------------------------------------------ counter and trace summaries
def _sha256(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _counter_rows(csv_path, counter):
    """(dispatch id, kernel name, value) of one counter, in dispatch order."""
    import csv
    out = []
    with open(csv_path) as f:
        for x in csv.DictReader(f):
            if x["Counter_Name"] == counter:
                did = int(x.get("Dispatch_Id") or x.get("Correlation_Id") or len(out))
                out.append((did, x["Kernel_Name"], float(x["Counter_Value"])))
    out.sort()
    return out


def _per_launch(rows):
    """Sum a counter over each attention launch: a launch is its entry point's first kernel
    and the own-part and merge kernels that follow it. Returns {entry: [sums]} and, per
    entry, {kernel: total}."""
    sums, per_kernel, cur = {}, {}, None
    for _, k, v in rows:
        entry = next((e for e, first in ENTRY_FIRST.items() if first in k), None)
        if entry is not None:
            cur = entry
            sums.setdefault(cur, []).append(0.0)
        elif cur is None or not any(r in k for r in ENTRY_REST):
            cur = None  # another kernel: the launch ended
            continue
        sums[cur][-1] += v
        per_kernel.setdefault(cur, {})
        per_kernel[cur][k] = per_kernel[cur].get(k, 0.0) + v
    return sums, per_kernel


def write_traffic(run_dir):
    """Condense rocprofv3 FETCH_SIZE / WRITE_SIZE runs (of this script with --passes cold, and
    of --copy-calib) into profiles/traffic.json: HBM bytes per launch of each attention entry
    point = its kernels' counters summed per launch (dispatch order), averaged over launches,
    each counter scaled by what it reads for the plain copy of known size."""
    fetch = _counter_rows(os.path.join(run_dir, "pmc_FETCH_SIZE", "bench_counter_collection.csv"), "FETCH_SIZE")
    write = _counter_rows(os.path.join(run_dir, "pmc_WRITE_SIZE", "bench_counter_collection.csv"), "WRITE_SIZE")
    cf = _counter_rows(os.path.join(run_dir, "copy_FETCH_SIZE", "run_counter_collection.csv"), "FETCH_SIZE")
    cw = _counter_rows(os.path.join(run_dir, "copy_WRITE_SIZE", "run_counter_collection.csv"), "WRITE_SIZE")
    copy_f = np.mean([v for _, k, v in cf if "kv_scatter_kernel" in k])
    copy_w = np.mean([v for _, k, v in cw if "kv_scatter_kernel" in k])
    f_scale = COPY_READ_BYTES / (copy_f * 1024.0)
    w_scale = COPY_WRITE_BYTES / (copy_w * 1024.0)
    fs, fk = _per_launch(fetch)
    ws, wk = _per_launch(write)
    out = {"source_sha256": _sha256(KERNEL_SOURCE), "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w, "entries": {}}
    for entry in ENTRY_FIRST:
        if not fs.get(entry) or not ws.get(entry):
            continue
        n = len(fs[entry])
        per = {k: {"fetch_kib_per_launch": fk[entry].get(k, 0.0) / n, "write_kib_per_launch": wk[entry].get(k, 0.0) / n}
               for k in set(fk[entry]) | set(wk[entry].keys())}
        out["entries"][entry] = {
            "launches": n, "kernels": per,
            "bytes_per_launch": (sum(fs[entry]) * f_scale + sum(ws[entry]) * w_scale) * 1024 / n}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def load_traffic(entry, path):
    """HBM bytes per launch of `entry` from the committed counter summary, or None when there
    is none or the kernel source changed since the counters were taken."""
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != _sha256(KERNEL_SOURCE):
        return None
    return t.get("entries", {}).get(entry, {}).get("bytes_per_launch")


def summarize_counters(run_dirs):
    """Markdown summary of rocprofv3 counter runs (one directory per pass): per kernel of the
    hot path, dispatches and the mean per dispatch of every counter, plus the MFMA
    utilisation (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x 1024 SIMDs) and the
    fraction of wave cycles spent waiting (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES) where the pass
    holds those counters. MOPS_BF16 counts 512 flops per unit."""
    import csv
    import glob
    acc = {}
    for d in run_dirs:
        for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
            with open(f) as fh:
                for x in csv.DictReader(fh):
                    k = x["Kernel_Name"]
                    if not any(h in k for h in HOT):
                        continue
                    per = acc.setdefault(k, {})
                    per.setdefault(x["Counter_Name"], []).append(float(x["Counter_Value"]))
    for k, per in sorted(acc.items()):
        n = max(len(v) for v in per.values())
        print(f"\n`{k[:120]}` ({n} dispatches)\n")
        print("| counter | mean per dispatch |\n|---|---|")
        mean = {c: sum(v) / len(v) for c, v in per.items()}
        for c in sorted(mean):
            print(f"| {c} | {mean[c]:.6g} |")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "GRBM_GUI_ACTIVE" in mean:
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs; the busy cycles over all 1024 SIMDs
            print(f"| MFMA utilisation (busy / (GUI_ACTIVE / 8 XCDs x 1024 SIMDs)) | "
                  f"{mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (mean['GRBM_GUI_ACTIVE'] / 8 * 1024):.3f} |")
        if "SQ_WAIT_INST_ANY" in mean and "SQ_WAVE_CYCLES" in mean:
            print(f"| waves waiting (WAIT_INST_ANY / WAVE_CYCLES) | {mean['SQ_WAIT_INST_ANY'] / mean['SQ_WAVE_CYCLES']:.3f} |")
        if "SQ_INSTS_VALU" in mean and "SQ_INSTS_MFMA" in mean and mean["SQ_INSTS_MFMA"]:
            print(f"| VALU instructions per MFMA | {mean['SQ_INSTS_VALU'] / mean['SQ_INSTS_MFMA']:.2f} |")
        if "SQ_INSTS_SALU" in mean and "SQ_INSTS_MFMA" in mean and mean["SQ_INSTS_MFMA"]:
            print(f"| SALU instructions per MFMA | {mean['SQ_INSTS_SALU'] / mean['SQ_INSTS_MFMA']:.2f} |")


HOT = ("shared_kernel", "own_", "merge_kernel", "attn_kernel", "extend_kernel", "kv_scatter_kernel",
       "rtt_write_kernel", "decode_append_kernel", "kv_move_kernel")


def summarize_trace(csv_path):
    """Markdown summary of a rocprofv3 kernel trace: per kernel name, dispatches, mean and
    total duration; and GPU idle over the window from the first to the last dispatch of the
    hot path's kernels: the time no kernel runs (the union of dispatch intervals subtracted
    from the window), in total and per trace step."""
    import csv
    rows = []
    with open(csv_path) as f:
        for x in csv.DictReader(f):
            rows.append((int(x["Start_Timestamp"]), int(x["End_Timestamp"]), x["Kernel_Name"]))
    rows.sort()
    per = {}
    for s, e, k in rows:
        p = per.setdefault(k, [0, 0])
        p[0] += 1
        p[1] += e - s
    # the library's kernels one by one; the rest (the seeded input generator, scratch fills,
    # copies) in one line
    print("| kernel | dispatches | mean us | total ms |\n|---|---|---|---|")
    other_n, other_t = 0, 0
    for k, (n, tot) in sorted(per.items(), key=lambda kv: -kv[1][1]):
        if "raxk" in k:  # also the mangled names the demangler leaves (bf16 template arguments)
            print(f"| `{k[:110]}` | {n} | {tot / n / 1e3:.2f} | {tot / 1e6:.3f} |")
        else:
            other_n, other_t = other_n + n, other_t + tot
    if other_n:
        print(f"| other kernels (input generator, scratch fills, copies) | {other_n} | {other_t / other_n / 1e3:.2f} | "
              f"{other_t / 1e6:.3f} |")
    hot = [r for r in rows if any(h in r[2] for h in HOT)]
    if not hot:
        return
    w0, w1 = hot[0][0], max(e for _, e, _ in hot)
    busy, cur_s, cur_e = 0, None, None
    for s, e, _ in rows:
        if e <= w0 or s >= w1:
            continue
        s, e = max(s, w0), min(e, w1)
        if cur_e is None or s > cur_e:
            if cur_e is not None:
                busy += cur_e - cur_s
            cur_s, cur_e = s, e
        else:
            cur_e = max(cur_e, e)
    if cur_e is not None:
        busy += cur_e - cur_s
    win = w1 - w0
    print(f"\nWindow of the hot path's kernels: {win / 1e6:.3f} ms; kernels busy {busy / 1e6:.3f} ms; "
          f"GPU idle {(win - busy) / 1e6:.3f} ms ({(win - busy) / win:.1%}).")
    # idle gaps (no kernel running) by the kernel that ends them, and by tenth of the window
    by_next, by_tenth, last_end = {}, [0] * 10, None
    for s, e, k in rows:
        if e <= w0 or s >= w1:
            continue
        if last_end is not None and s > last_end:
            gap = s - last_end
            name = k.split("(")[0].split("<")[0].replace("void ", "")[-40:]
            by_next[name] = by_next.get(name, 0) + gap
            by_tenth[min(9, int((last_end - w0) * 10 // win))] += gap
        last_end = e if last_end is None else max(last_end, e)
    if by_next:
        print("\n| idle gap ended by | ms |\n|---|---|")
        for name, g in sorted(by_next.items(), key=lambda kv: -kv[1])[:8]:
            print(f"| `{name}` | {g / 1e6:.3f} |")
        print("\nIdle ms by tenth of the window: " + ", ".join(f"{g / 1e6:.1f}" for g in by_tenth))
    # idle inside runs of 5 consecutive decode launches (no extend between them), from the
    # first one's start to the fifth one's end: the median and the worst over the job
    starts = [i for i, (_, _, k) in enumerate(rows) if ENTRY_FIRST["decode"] in k]
    runs = []
    for j in range(len(starts) - 5):
        a_i, b_i = starts[j], starts[j + 5]
        if any(ENTRY_FIRST["extend"] in rows[x][2] for x in range(a_i, b_i)):
            continue
        seg = rows[a_i:b_i]
        t0, t1 = seg[0][0], max(e for _, e, _ in seg)
        busy5, cs, ce = 0, None, None
        for s_, e_, _ in seg:
            if ce is None or s_ > ce:
                if ce is not None:
                    busy5 += ce - cs
                cs, ce = s_, e_
            else:
                ce = max(ce, e_)
        busy5 += ce - cs
        runs.append((t1 - t0 - busy5, t1 - t0))
    if runs:
        idle5 = sorted(r[0] for r in runs)
        print(f"\nRuns of 5 consecutive decode launches with no extend between them: {len(runs)}; GPU idle "
              f"inside a run: median {idle5[len(idle5) // 2] / 1e3:.1f} us, worst {idle5[-1] / 1e3:.1f} us "
              f"(median run {sorted(r[1] for r in runs)[len(runs) // 2] / 1e3:.0f} us).")
    # per launch of each attention entry point (its first kernel and the own-part and merge
    # kernels after it, in dispatch order): the span from the first kernel's start to the
    # last one's end, comparable with the HIP-event time of a launch
    spans, cur = {}, None
    for s, e, k in rows:
        entry = next((en for en, first in ENTRY_FIRST.items() if first in k), None)
        if entry is not None:
            cur = entry
            spans.setdefault(cur, []).append([s, e, e - s])
        elif cur is not None and any(r in k for r in ENTRY_REST):
            sp = spans[cur][-1]
            sp[1] = max(sp[1], e)
            sp[2] += e - s
        else:
            cur = None
    if spans:
        print("\n| entry point | launches | mean launch span us | mean kernel time per launch us |\n|---|---|---|---|")
        for entry, sp in spans.items():
            n = len(sp)
            print(f"| {entry} | {n} | {sum(b - a for a, b, _ in sp) / n / 1e3:.2f} | {sum(t for _, _, t in sp) / n / 1e3:.2f} |")


def achievable_peaks(dev):
    """Measured ceilings beside the published peaks: a plain device copy (4 GiB read and
    4 GiB written, through torch) and a bf16 GEMM (8192^3, through torch and hipBLASLt).
    Median of 10 timed runs after 3 untimed ones."""
    import torch

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    src = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del src, dst
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    t_gemm = timed(lambda: torch.mm(a, b))
    return {"copy_gbs": 2 * (1 << 32) / t_copy / 1e9, "copy_frac_hbm_peak": 2 * (1 << 32) / t_copy / 1e9 / HBM_PEAK_GBS,
            "gemm_bf16_tflops": 2 * n ** 3 / t_gemm / 1e12,
            "gemm_frac_mfma_peak": 2 * n ** 3 / t_gemm / 1e12 / MFMA_BF16_PEAK_TFLOPS}


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the path would shard by KV heads or by requests, with no exchange inside attention)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from prefix_shared_kv_extend_amd import _lib

    _lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calib:
        # plain copy through kv_scatter with identity slots: reads (distinct K and V) and
        # writes 2 x 512 MiB, plus the 128 KiB slot list
        n = 1 << 15
        k = torch.ones((n, 64, 128), dtype=torch.bfloat16, device=dev)
        v = torch.ones_like(k)
        kp = torch.empty_like(k)
        vp = torch.empty_like(k)
        loc = torch.arange(n, dtype=torch.int32, device=dev)
        for _ in range(3):
            _lib.kv_scatter(k, v, loc, kp, vp)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": COPY_READ_BYTES, "copy_calib_bytes_written": COPY_WRITE_BYTES}))
        return

    if args.only:
        print(json.dumps({args.only: side_config(SIDE[args.only], args.reps, Flusher(dev, args.flush_mib))}),
              flush=True)
        return

    h = headline(args, dev)
    job = h.pop("_job")
    h.pop("_inp")
    out = {"metric": METRIC}
    if "wall" in h:
        out.update({"value": h["wall"]["value"], "unit": "attn tokens/s", "n_gpus": 1, "steps": args.steps,
                    "warmup": args.warmup, "ms_per_step": h["wall"]["ms_per_step"]})
    else:
        out.update({"value": None, "unit": "attn tokens/s", "n_gpus": 1, "steps": 0, "warmup": 0,
                    "ms_per_step": None})
    out.update({"higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic: seeded tokens; Q/K/V from a prefix-hash generator (N(0,1)), no model weights",
                "config": h["config"], "hit_rate": h["hit_rate"]})
    if "wall" in h:
        out["ms_stats"] = h["wall"]["ms_stats"]
    if "cold" in h:
        out["extend"] = {"cold": h["cold"]["extend"]}
        out["decode"] = {"cold": h["cold"]["decode"]}
        if "natural" in h:
            out["extend"]["natural"] = h["natural"]["extend"]
            out["decode"]["natural"] = h["natural"]["decode"]
        out["roofline"] = roofline_of(h["cold"], args.traffic)
    if "wall" in h:
        # the runtime never synchronises inside a job, so the tree work of one call overlaps
        # the kernels of the previous ones. host_issue_ms includes time a launch waits for a
        # full GPU queue; the host pass gives the host work alone (each step synchronised).
        # The job is host-bound when that host work takes about as long as the job.
        ov = {"host_issue_ms_per_step": h["wall"]["host_issue_ms"], "wall_ms_per_step": h["wall"]["ms_per_step"]}
        if "host" in h:
            ov["host_work_ms_per_step"] = h["host"]["ms_per_step"]
            ov["host_phases_ms"] = h["host"]["phases_ms"]
            ov["host_bound"] = h["host"]["ms_per_step"] > 0.97 * h["wall"]["ms_per_step"]
        if "natural" in h:
            ov["attention_kernel_ms_per_step"] = (h["natural"]["extend"]["us_per_step"]
                                                  + h["natural"]["decode"]["us_per_step"]) * 1e-3
        out["overlap"] = ov
    if not args.no_side:
        flush = Flusher(dev, args.flush_mib)
        for name, idx in SIDE.items():
            out[name] = side_config(idx, args.reps, flush)
        out["scheduler"] = scheduler_ablation()
        out["host_tier"] = host_tier_measure(dev)
        out["qkv_projection"] = projection_measure(dev)
        out["achievable_peaks"] = achievable_peaks(dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(job, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
