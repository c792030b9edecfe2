"""Benchmark of the RadixAttention hot path on one MI355X.

Workload (the few-shot configuration): one attention layer at Llama-2-7B attention
shape (32 heads MHA, head_dim 128), bf16 inputs, fp32 accumulation, bf16 outputs;
64 requests share a 2000-token prefix and each adds a distinct 50-token suffix;
pool of 2^20 token slots; then 32 decode steps for all 64 requests.

One timed step = the whole job from an empty cache, through the C ABI:
  request 0 cold (match, lock, allocate, fill req_to_token, KV write-back, extend
  attention over 2050 tokens, insert); the other 63 reuse its 2000-token prefix
  (match splits its node) and extend only their 50 suffix tokens; 32 decode
  steps (allocate, fill, write-back, decode attention); finish (insert prompt +
  output, unlock); then evict the whole tree, so the next step starts empty.
Q/K/V for every call are generated before timing and stay resident in HBM.

value = attention tokens per second for the whole step (5200 extend queries +
2048 decode queries, wall clock, host tree work included), from a pass with no
timing events. A second pass over the same steps records a HIP event pair around
every attention call on the stream the kernels run on; it gives the per-phase
kernel times and the roofline of the dominant kernel. The JSON line also carries
the CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COPY_READ_BYTES = 2 * (1 << 15) * 64 * 128 * 2 + (1 << 15) * 4   # --copy-calib: K, V and slot list read
COPY_WRITE_BYTES = 2 * (1 << 15) * 64 * 128 * 2                    # K and V written
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "prefix_shared_kv_extend_amd", "csrc", "kernels", "attention.hip")
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "attn tokens/s (extend, decode) + % MFMA/HBM peak on radix-cached KV"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the sections beside the headline (scheduler, host tier, projection, GQA decode)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--traffic", default=TRAFFIC_JSON, help="counter summary with HBM bytes per launch")
    ap.add_argument("--write-traffic", default=None, metavar="DIR",
                    help="condense rocprofv3 counter runs in DIR into profiles/traffic.json and exit")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain copy kernel of known size (for counter scaling) and exit")
    return ap.parse_args()


class Prepared:
    """Pre-generated inputs for every attention call of one job, in call order."""

    def __init__(self, runner, dev):
        import torch
        self.calls = []
        job = runner.job
        seen = {}

        def grab(kind):
            def cb(si, batch, pairs, o):
                seen.setdefault(si, {})[kind] = list(pairs)
            return cb

        runner.run(on_extend=grab("extend"), on_decode=grab("decode"))
        torch.cuda.synchronize()
        for si in sorted(seen):
            for kind in ("extend", "decode"):
                if kind in seen[si]:
                    q, k, v = runner.qkv(seen[si][kind])
                    o = torch.empty((q.shape[0], job.h_q, job.d), dtype=torch.bfloat16, device=dev)
                    self.calls.append((si, kind, seen[si][kind], q, k, v, o))


def algorithmic(job, prep):
    """Flops of each extend call and unique bytes of each decode call (per launch)."""
    D, hq, hkv = job.d, job.h_q, job.h_kv
    elt = 2
    ext_flops, dec_bytes = [], []
    for si, kind, pairs, q, k, v, o in prep.calls:
        if kind == "extend":
            ext_flops.append(sum(4.0 * D * hq * (p + 1) for _, p in pairs))
        else:
            # distinct slots read: the shared prefix once plus every request's own positions
            lens = [p + 1 for _, p in pairs]
            shared = 2000
            distinct = shared + sum(n - shared for n in lens)
            kv = distinct * 2 * hkv * D * elt
            qo = len(pairs) * hq * D * elt * 2
            idx = sum(lens) * 4
            dec_bytes.append(kv + qo + idx)
    return ext_flops, dec_bytes


REPLAYS = 4


def run_step(runner, prep, timers=None):
    """One job pass. With timers: after each attention call, the same call (identical inputs;
    it only writes its output) is replayed REPLAYS times back to back between one HIP event
    pair on the stream the kernels run on, so the measured time is kernel time, not time
    the GPU spent waiting for the host to issue the next launch."""
    import torch
    from prefix_shared_kv_extend_amd import _lib as L
    rt = runner.rt
    job = runner.job
    it = iter(prep.calls)

    def timed(kind, fn):
        if timers is None:
            return
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(REPLAYS):
            fn()
        e1.record()
        timers.setdefault(kind, []).append((e0, e1))

    for si, st in enumerate(job.steps):
        rt.step = si
        if st.extend:
            eb = rt.begin_extend([(rid, job.requests[rid].prompt) for rid in st.extend])
            _, kind, pairs, q, k, v, o = next(it)
            rt.run_extend(eb, q, k, v, o)
            timed("extend", lambda: L.extend_attention(q, k, v, rt.k_pool, rt.v_pool, rt.rtt, eb.dev["req_pool_idx"],
                                                       eb.dev["prefix_len"], eb.dev["qo_indptr"], o,
                                                       shared_len=eb.dev["shared_len"]))
            rt.end_extend(eb, {rid: job.requests[rid].prompt for rid in eb.rids})
        if st.decode:
            db = rt.begin_decode(st.decode)
            _, kind, pairs, q, k, v, o = next(it)
            rt.run_decode(db, q, k, v, o)
            if timers is not None:
                # replays in the layout the runtime's decode step chose (host hints)
                def dec(ws):
                    return L.decode_attention_hinted(q, rt.k_pool, rt.v_pool, rt.rtt, db.dev["req_pool_idx"],
                                                     db.dev["seq_len"], db.max_seq_len, o, db.seq_len,
                                                     db.shared_len_host, workspace=ws,
                                                     shared_len=db.dev["shared_len"])
                ws = rt._workspace(dec(None))
                timed("decode", lambda: dec(ws))
        if st.finish:
            rt.finish_batch([(rid, runner.full[rid][: rt.seq_len(rid)]) for rid in st.finish])
    rt.tree.evict_lru(rt.num_slots)             # the cache yields everything: next step starts empty


def _sha256(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _counter_means(csv_path, counter):
    """Mean per dispatch of one counter, per kernel name, from a rocprofv3 counter CSV."""
    import csv
    acc = {}
    with open(csv_path) as f:
        for x in csv.DictReader(f):
            if x["Counter_Name"] == counter:
                acc.setdefault(x["Kernel_Name"], []).append(float(x["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


# kernels that make up one launch of each attention entry point (substrings of their names)
ENTRY_KERNELS = {"decode": ("shared_kernel<128, 4, 4>", "own_merge_kernelIDF16bLi128E"),
                 "extend": ("attn_kernelIDF16bLi128ELb0E",)}


def write_traffic(run_dir):
    """Condense rocprofv3 FETCH_SIZE / WRITE_SIZE runs (of this script, and of --copy-calib)
    into profiles/traffic.json: HBM bytes per launch of each attention entry point, each
    counter scaled by what it reads for the plain copy of known size."""
    fetch = _counter_means(os.path.join(run_dir, "pmc_FETCH_SIZE", "bench_counter_collection.csv"), "FETCH_SIZE")
    write = _counter_means(os.path.join(run_dir, "pmc_WRITE_SIZE", "bench_counter_collection.csv"), "WRITE_SIZE")
    cf = _counter_means(os.path.join(run_dir, "copy_FETCH_SIZE", "run_counter_collection.csv"), "FETCH_SIZE")
    cw = _counter_means(os.path.join(run_dir, "copy_WRITE_SIZE", "run_counter_collection.csv"), "WRITE_SIZE")
    copy_f = next(v for k, v in cf.items() if "kv_scatter_kernel" in k)
    copy_w = next(v for k, v in cw.items() if "kv_scatter_kernel" in k)
    f_scale = COPY_READ_BYTES / (copy_f * 1024.0)
    w_scale = COPY_WRITE_BYTES / (copy_w * 1024.0)
    out = {"source_sha256": _sha256(KERNEL_SOURCE), "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w, "entries": {}}
    for entry, keys in ENTRY_KERNELS.items():
        per = {}
        for key in keys:
            kf = [v for k, v in fetch.items() if key in k]
            kw = [v for k, v in write.items() if key in k]
            if kf and kw:
                per[key] = {"fetch_kib": kf[0], "write_kib": kw[0],
                            "bytes": kf[0] * 1024 * f_scale + kw[0] * 1024 * w_scale}
        out["entries"][entry] = {"kernels": per, "bytes_per_launch": sum(p["bytes"] for p in per.values())}
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
    pool writes, then rax_kv_scatter from the contiguous K/V. HIP events around 20 calls of
    each on the current stream."""
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

    def unfused():
        _lib.qkv_project(x, w, h, h, q_out=q, k_ext=k, v_ext=v)
        _lib.kv_scatter(k, v, loc, kp, vp)

    out = {"workload": "cached few-shot extend batch: 3150 tokens, hidden 4096, 32 heads x 128 (W 12288 x 4096)"}
    flops = 2.0 * t * hidden * 3 * h * d
    for name, fn in (("fused", fused), ("gemm_then_scatter", unfused)):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            fn()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / 20
        out[name] = {"us": us, "tflops": flops / (us * 1e-6) / 1e12,
                     "frac_mfma_peak": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    out["saved_us"] = out["gemm_then_scatter"]["us"] - out["fused"]["us"]
    assert _lib.device_errors() == 0
    return out


def decode_side_measure(index, workload, n_steps=8, first_decode=0):
    """Decode attention on one of the decode-heavy workloads (configuration `index` of
    workloads.configs). The steps before the chosen decode step run untimed; then each of
    the next n_steps decode calls (rax_decode_step, as the runtime runs it) is replayed
    REPLAYS times between one HIP event pair through rax_decode_attention_hinted, in the
    layout the decode step chose from its host hints. Algorithmic
    bytes per call: the distinct K/V rows the batch reads (each slot id in the batch's
    req_to_token rows once), Q and O, 4 B per req_to_token entry."""
    import torch
    from prefix_shared_kv_extend_amd import _lib as L
    from prefix_shared_kv_extend_amd.driver import JobRunner
    from workloads import configs
    job = configs.make(index)
    runner = JobRunner(job, out_dtype=torch.bfloat16, record_log=False)
    rt = runner.rt
    first = [i for i, st in enumerate(job.steps) if st.decode][first_decode]
    runner.run(steps=range(first))
    elt = 2
    us, nbytes = [], []

    def on_decode(si, db, pairs, o):
        q = torch.randn((len(db.rids), job.h_q, job.d), device=o.device).to(torch.bfloat16)
        ws = rt._workspace(L.attention_workspace_bytes(True, len(db.rids), job.h_q, job.h_kv, job.d,
                                                       db.max_seq_len))

        def call(w):
            return L.decode_attention_hinted(q, rt.k_pool, rt.v_pool, rt.rtt, db.dev["req_pool_idx"],
                                             db.dev["seq_len"], db.max_seq_len, o, db.seq_len, db.shared_len_host,
                                             workspace=w, shared_len=db.dev["shared_len"])
        ws = rt._workspace(max(call(None), ws.numel()))
        call(ws)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(REPLAYS):
            call(ws)
        b.record()
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) * 1e3 / REPLAYS)
        lens = db.seq_len.astype(np.int64)
        rows = db.dev["req_pool_idx"].long()
        width = int(lens.max())
        keys = rt.rtt[rows, :width]
        inside = torch.arange(width, device=keys.device)[None, :] < torch.as_tensor(lens, device=keys.device)[:, None]
        distinct = int(torch.unique(keys[inside]).numel())
        nbytes.append(distinct * 2 * job.h_kv * job.d * elt + 2 * len(lens) * job.h_q * job.d * elt
                      + int(lens.sum()) * 4)

    runner.run(steps=range(first, first + n_steps), on_decode=on_decode)
    assert L.device_errors() == 0
    gbs = sum(nbytes) / (sum(us) * 1e-6) / 1e9
    return {"workload": workload + "; %d decode steps" % n_steps,
            "us_per_call": sum(us) / len(us), "mb_per_call": sum(nbytes) / len(nbytes) / 1e6,
            "gbs_unique": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS}


def decode_gqa_measure(n_steps=8):
    """Self-consistency decode: 256 branches of U{0..1024} tokens off one 4096-token
    prefix, GQA 64/8 heads x 128, bf16; its first n_steps decode calls."""
    return decode_side_measure(3, "self-consistency: 256 branches of U{0..1024} tokens off a 4096-token prefix, "
                                  "GQA 64/8 x 128, bf16; from the first decode step", n_steps)


def decode_two_level_measure(n_steps=8):
    """Two-level decode: a 1024-token system prefix, 8 exemplar blocks of 512 tokens, 16
    questions of 64 tokens under each (128 requests), MHA 32 x 128, bf16; its first
    n_steps decode calls. A 64-request row block spans four exemplar blocks: their keys
    are computed once per block as deeper runs."""
    return decode_side_measure(2, "two-level: 1024-token system prefix, 8 x 512-token exemplar blocks, "
                                  "16 x 64-token questions each (128 requests), MHA 32 x 128, bf16; "
                                  "from the first decode step", n_steps)


def cpu_baseline(job, seconds):
    """The oracle (fp64 recompute from scratch) on a bounded sample of the same workload."""
    import torch
    from oracle.attention import outputs_from_scratch
    threads = len(os.sched_getaffinity(0))
    torch.set_num_threads(threads)
    rng = np.random.default_rng(0)
    done = 0
    t0 = time.perf_counter()
    reqs = []
    while time.perf_counter() - t0 < seconds:
        rid = int(rng.integers(1, len(job.requests)))
        r = job.requests[rid]
        # all 50 suffix queries of one cached request plus its first decode query
        pos = list(range(2000, r.n)) + [r.n]
        outputs_from_scratch(job.full_tokens(rid), pos, job.h_q, job.h_kv, job.d, job.seed, job.dtype)
        done += len(pos)
        reqs.append(rid)
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "attn tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(reqs)} cached requests x (50 suffix queries + 1 decode query), each recomputed "
                      f"from scratch over its 2051-token sequence in fp64 ({dt:.1f} s)"}


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the path would shard by KV heads or by requests, with no exchange inside attention)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from prefix_shared_kv_extend_amd import _lib
    from prefix_shared_kv_extend_amd.driver import JobRunner
    from workloads import configs

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

    job = configs.make(1)
    runner = JobRunner(job, device="cuda:0", out_dtype=torch.bfloat16, record_log=False)
    prep = Prepared(runner, dev)                       # one untimed pass to learn every call's positions
    runner.rt.tree.evict_lru(runner.rt.num_slots)
    ext_flops, dec_bytes = algorithmic(job, prep)
    n_ext_tok = sum(len(c[2]) for c in prep.calls if c[1] == "extend")
    n_dec_tok = sum(len(c[2]) for c in prep.calls if c[1] == "decode")

    for _ in range(args.warmup):
        run_step(runner, prep)
    torch.cuda.synchronize()

    # pass 1: the job as it runs (no timing events) -> value, ms_per_step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(runner, prep)
    t_issued = time.perf_counter()                     # the host never waits inside the loop
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    host_ms = (t_issued - t0) * 1e3 / args.steps

    # pass 2: the same steps, each attention call replayed back to back between a HIP event
    # pair on the stream the kernels run on -> per-launch kernel times for the roofline
    timers = {}
    torch.cuda.synchronize()
    for _ in range(args.steps):
        run_step(runner, prep, timers)
    torch.cuda.synchronize()

    ext_us = [a.elapsed_time(b) * 1e3 / REPLAYS for a, b in timers.get("extend", [])]
    dec_us = [a.elapsed_time(b) * 1e3 / REPLAYS for a, b in timers.get("decode", [])]
    per_step_ext = sum(ext_us) / args.steps
    per_step_dec = sum(dec_us) / args.steps
    ext_tflops = sum(ext_flops) * args.steps / (sum(ext_us) * 1e-6) / 1e12
    dec_gbs = sum(dec_bytes) * args.steps / (sum(dec_us) * 1e-6) / 1e9
    if per_step_ext >= per_step_dec:
        roof = {"kernel": "extend attention (attn_kernel, bf16, D=128)", "bound": "mfma",
                "achieved": ext_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ext_tflops / MFMA_BF16_PEAK_TFLOPS, "launches_per_step": len(ext_flops),
                "avg_launch_us": sum(ext_us) / len(ext_us)}
    else:
        roof = {"kernel": "decode attention (shared_kernel + own_merge_kernel)", "bound": "hbm",
                "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                "launches_per_step": len(dec_bytes), "avg_launch_us": sum(dec_us) / len(dec_us)}
    roof["traffic"] = load_traffic("extend" if roof["bound"] == "mfma" else "decode", args.traffic)

    out = {
        "metric": METRIC,
        "value": (n_ext_tok + n_dec_tok) * args.steps / (t1 - t0),
        "unit": "attn tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded tokens; Q/K/V from a prefix-hash generator (N(0,1)), no model weights",
        "config": {"workload": "fewshot: 64 requests x (2000 shared + 50 own) tokens, then 32 decode steps; "
                               "1 layer, 32 heads MHA, head_dim 128, pool 2^20 slots",
                   "extend_tokens_per_step": n_ext_tok, "decode_tokens_per_step": n_dec_tok,
                   "prompt_tokens_per_step": sum(r.n for r in job.requests)},
        "extend": {"kernel_us_per_step": per_step_ext, "tok_s_kernel": n_ext_tok / (per_step_ext * 1e-6),
                   "tflops": ext_tflops, "frac_mfma_peak": ext_tflops / MFMA_BF16_PEAK_TFLOPS},
        "decode": {"kernel_us_per_step": per_step_dec, "tok_s_kernel": n_dec_tok / (per_step_dec * 1e-6),
                   "gbs_unique": dec_gbs, "frac_hbm_peak": dec_gbs / HBM_PEAK_GBS},
        "hit_rate": 1.0 - n_ext_tok / sum(r.n for r in job.requests),
        "roofline": roof,
        # host/GPU overlap: the runtime never synchronises inside a step, so the tree work
        # of one call overlaps the kernels of the previous ones; the GPU waits on the host
        # only if issuing a step takes as long as the step itself
        "overlap": {"host_issue_ms_per_step": host_ms, "wall_ms_per_step": ms,
                    "attention_kernel_ms_per_step": (per_step_ext + per_step_dec) * 1e-3,
                    "host_bound": host_ms > 0.97 * ms},
    }
    if not args.no_side:
        out["scheduler"] = scheduler_ablation()
        out["host_tier"] = host_tier_measure(dev)
        out["qkv_projection"] = projection_measure(dev)
        out["decode_gqa"] = decode_gqa_measure()
        out["decode_two_level"] = decode_two_level_measure()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(job, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
