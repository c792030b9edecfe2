"""GPU parity: the HIP path (through the C ABI) against the oracle.

* kv_scatter, the req_to_token fill and the decode append are checked bit for bit.
* Whole traces run through RadixRuntime on the GPU; their host event logs
  (matches, evictions, allocations, inserts), final slot rows and tree dumps
  must equal the oracle's replay exactly, and attention outputs must agree with
  fp64 attention recomputed from scratch over each full sequence within
  max-abs 1e-5 (fp32 inputs) or 1e-2 (bf16 inputs, fp32 accumulation).
* Small traces are checked at every output; the full-size configurations are
  checked on sampled outputs (the oracle recomputes each sample from scratch).
"""
import os
import sys

import numpy as np
import pytest
import torch

from oracle.attention import outputs_from_scratch
from oracle.runner import run_trace
from workloads import configs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from prefix_shared_kv_extend_amd import _lib
    _lib.lib()          # fails loudly if librax.so is missing
    yield


def _collect(job, runner_kw=None, pick=None, progress=0):
    """Run the job on the GPU; keep outputs chosen by pick(kind, step, rid, pos) -> bool."""
    from prefix_shared_kv_extend_amd.driver import JobRunner
    got = {}

    def keep(kind, si, pairs, o):
        idx = [i for i, (rid, p) in enumerate(pairs) if pick is None or pick(kind, si, rid, p)]
        if idx:
            sel = o[torch.tensor(idx, device=o.device)].float().cpu().numpy()
            for j, i in enumerate(idx):
                got[pairs[i]] = sel[j]

    r = JobRunner(job, **(runner_kw or {}))
    r.run(on_extend=lambda si, eb, pairs, o: keep("extend", si, pairs, o),
          on_decode=lambda si, db, pairs, o: keep("decode", si, pairs, o), progress=progress)
    torch.cuda.synchronize()
    return r, got


def _check_outputs(job, got, tol):
    by_rid = {}
    for (rid, p), o in got.items():
        by_rid.setdefault(rid, []).append((p, o))
    worst = 0.0
    for rid, items in by_rid.items():
        pos = [p for p, _ in items]
        ref = outputs_from_scratch(job.full_tokens(rid), pos, job.h_q, job.h_kv, job.d, job.seed, job.dtype)
        for i, (p, o) in enumerate(items):
            err = float(np.abs(o.astype(np.float64) - ref[i]).max())
            worst = max(worst, err)
            assert err <= tol, f"rid {rid} pos {p}: max abs err {err:.3g} > {tol}"
    return worst


def _check_host(job, runner, host_slots=0):
    ref = run_trace(job, host_slots=host_slots)
    assert len(runner.log) == len(ref["log"])
    for a, b in zip(runner.log, ref["log"]):
        assert a == b
    assert runner.final_rows == ref["rows"]
    assert runner.rt.tree.dump() == ref["dump"]
    from prefix_shared_kv_extend_amd import _lib
    assert _lib.device_errors() == 0


# ------------------------------------------------------------------ data movement
def test_kv_scatter_bit_exact():
    from prefix_shared_kv_extend_amd import _lib
    say("kv_scatter: bf16 [777, 8, 128] and fp32 [33, 4, 64] into shuffled slots")
    g = torch.Generator().manual_seed(1)
    for dt, (n, h, d), S in ((torch.bfloat16, (777, 8, 128), 5000), (torch.float32, (33, 4, 64), 100)):
        k = torch.randn((n, h, d), generator=g).to(dt).cuda()
        v = torch.randn((n, h, d), generator=g).to(dt).cuda()
        loc = torch.randperm(S, generator=g)[:n].to(torch.int32)
        kp = torch.zeros((S, h, d), dtype=dt, device="cuda")
        vp = torch.zeros_like(kp)
        _lib.kv_scatter(k, v, loc.cuda(), kp, vp)
        torch.cuda.synchronize()
        kp, vp, loc = kp.cpu(), vp.cpu(), loc.long()
        assert torch.equal(kp[loc], k.cpu()) and torch.equal(vp[loc], v.cpu())
        untouched = torch.ones(S, dtype=torch.bool)
        untouched[loc] = False
        assert int(kp[untouched].abs().sum()) == 0 and int(vp[untouched].abs().sum()) == 0
    assert _lib.device_errors() == 0


def test_extend_write_equals_separate_calls():
    """rax_extend_write (the rows and the K/V write-back in one launch) against
    rax_req_to_token_write followed by rax_kv_scatter with the same arguments, bit for bit:
    bf16 [1500, 8, 128] rows into shuffled slots with 9 ragged requests' rows; then each half
    alone (no K/V rows; no req_to_token entries); then an out-of-range slot and row, skipped
    and flagged as by the separate calls."""
    from prefix_shared_kv_extend_amd import _lib
    say("extend_write: rows + K/V write-back in one launch vs the two calls")
    g = torch.Generator().manual_seed(7)
    n, h, d, S, B, W = 1500, 8, 128, 6000, 9, 700
    lens = torch.randint(1, 300, (B,), generator=g)
    ip = torch.zeros(B + 1, dtype=torch.int32)
    ip[1:] = torch.cumsum(lens, 0)
    total = int(ip[-1])
    rows = torch.randperm(B + 4, generator=g)[:B].to(torch.int32)
    start = torch.randint(0, W - 300, (B,), generator=g).to(torch.int32)
    src = torch.randint(0, S, (total,), generator=g).to(torch.int32)
    k = torch.randn((n, h, d), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((n, h, d), generator=g).to(torch.bfloat16).cuda()
    loc = torch.randperm(S, generator=g)[:n].to(torch.int32).cuda()
    dev = [t.cuda() for t in (rows, start, ip, src)]

    def run(fused, kk, vv, ll, tot):
        rtt = torch.full((B + 4, W), -1, dtype=torch.int32, device="cuda")
        kp = torch.zeros((S, h, d), dtype=torch.bfloat16, device="cuda")
        vp = torch.zeros_like(kp)
        if fused:
            _lib.extend_write(rtt, *dev, tot, kk, vv, ll, kp, vp)
        else:
            _lib.req_to_token_write(rtt, *dev, tot)
            _lib.kv_scatter(kk, vv, ll, kp, vp)
        torch.cuda.synchronize()
        return rtt.cpu(), kp.cpu(), vp.cpu(), _lib.device_errors()

    empty = (k[:0], v[:0], loc[:0])
    for args in ((k, v, loc, total), (*empty, total), (k, v, loc, 0)):
        a, b = run(True, *args), run(False, *args)
        assert all(torch.equal(x, y) for x, y in zip(a[:3], b[:3])) and a[3] == b[3] == 0
    # out of range: one slot past the pool, one row start past the row width
    bad_loc = loc.clone()
    bad_loc[5] = S
    start[3] = W
    dev[1] = start.cuda()
    a, b = run(True, k, v, bad_loc, total), run(False, k, v, bad_loc, total)
    assert all(torch.equal(x, y) for x, y in zip(a[:3], b[:3]))
    assert a[3] == b[3] == (_lib.DEVERR_SLOT | _lib.DEVERR_ROW)


def test_kv_scatter_out_of_range_slot_is_skipped_and_flagged():
    from prefix_shared_kv_extend_amd import _lib
    say("kv_scatter: slot ids -1 and S are skipped by the kernel's own bounds check")
    S, h, d = 16, 2, 64
    k = torch.ones((3, h, d), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((S, h, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    _lib.kv_scatter(k, k, torch.tensor([-1, 5, S], dtype=torch.int32, device="cuda"), kp, vp)
    assert _lib.device_errors() == _lib.DEVERR_SLOT
    assert float(kp.sum()) == h * d and float(kp[5].sum()) == h * d
    assert _lib.device_errors() == 0                  # cleared by the read


def test_req_to_token_write_bit_exact():
    from prefix_shared_kv_extend_amd import _lib
    say("req_to_token_write: 5 requests, ragged spans")
    rtt = torch.full((8, 50), -7, dtype=torch.int32, device="cuda")
    rows = [3, 0, 7, 1, 5]
    start = [0, 10, 49, 2, 0]
    lens = [4, 0, 1, 9, 50]
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    src = np.arange(indptr[-1], dtype=np.int32) * 3 + 1
    c = lambda x: torch.tensor(np.asarray(x, dtype=np.int32), device="cuda")
    _lib.req_to_token_write(rtt, c(rows), c(start), c(indptr), c(src), int(indptr[-1]))
    want = np.full((8, 50), -7, dtype=np.int32)
    for r in range(5):
        want[rows[r], start[r]: start[r] + lens[r]] = src[indptr[r]: indptr[r + 1]]
    assert np.array_equal(rtt.cpu().numpy(), want)
    assert _lib.device_errors() == 0


def test_decode_append_bit_exact_and_errors():
    """rax_decode_append: slots lowest-free-first, rows appended, lengths on both sides,
    K/V rows in the pools; 300 requests (more than one kernel-argument batch of 256);
    rejected calls change nothing."""
    from prefix_shared_kv_extend_amd import _lib
    say("decode_append: 300 requests into a 600-slot pool, then ENOMEM and EINVAL")
    S, R, W, h, d, n = 600, 320, 40, 4, 64, 300
    t = _lib.Tree(S)
    t.alloc_slots(300)                                   # slots 0..299 taken: the new ones are 300..599
    g = torch.Generator().manual_seed(7)
    rows_np = torch.randperm(R, generator=g)[:n].numpy().astype(np.int32)
    lens = torch.randint(0, W - 1, (n,), generator=g).numpy().astype(np.int32)
    k = torch.randn((n, h, d), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((n, h, d), generator=g).to(torch.bfloat16).cuda()
    kp = torch.zeros((S, h, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    rtt = torch.full((R, W), -5, dtype=torch.int32, device="cuda")
    rows = torch.tensor(rows_np, device="cuda")
    sl_dev = torch.zeros(n, dtype=torch.int32, device="cuda")
    seq = lens.copy()
    new, freed = t.decode_append(seq, rtt, rows, sl_dev, k, v, kp, vp)
    torch.cuda.synchronize()
    assert np.array_equal(new, np.arange(300, 600, dtype=np.int32)) and len(freed) == 0
    assert np.array_equal(seq, lens + 1) and np.array_equal(sl_dev.cpu().numpy(), lens + 1)
    want = np.full((R, W), -5, dtype=np.int32)
    want[rows_np, lens] = new
    assert np.array_equal(rtt.cpu().numpy(), want)
    kc, vc = kp.cpu(), vp.cpu()
    assert torch.equal(kc[300:], k.cpu()) and torch.equal(vc[300:], v.cpu())
    assert int(kc[:300].abs().sum()) == 0 and int(vc[:300].abs().sum()) == 0
    assert _lib.device_errors() == 0
    # no free slot and nothing evictable: ENOMEM, lengths untouched
    before = seq.copy()
    with pytest.raises(_lib.RaxError) as e:
        t.decode_append(seq[:1].copy(), rtt, rows[:1], sl_dev[:1], k[:1], v[:1], kp, vp)
    assert e.value.status == _lib.ENOMEM and np.array_equal(seq, before)
    # a row already at full width: EINVAL before any slot is taken
    t.free_slots([0])
    full = np.array([W], dtype=np.int32)
    with pytest.raises(_lib.RaxError) as e:
        t.decode_append(full, rtt, rows[:1], sl_dev[:1], k[:1], v[:1], kp, vp)
    assert e.value.status == _lib.EINVAL and full[0] == W and t.free_count() == 1
    torch.cuda.synchronize()
    assert np.array_equal(rtt.cpu().numpy(), want)


# ------------------------------------------------------------- whole small traces
SMALL = {
    "tiny_fp32_d64": lambda: configs.tiny(),
    "tiny_fp32_d128": lambda: configs.tiny(n_req=4, prefix=130, suffix=7, n_decode=5, h=4, d=128),
    "fewshot_bf16_ragged": lambda: configs.fewshot(n_req=5, prefix=300, suffix=37, n_decode=3, h=4,
                                                   num_slots=4096),
    "fewshot_bf16_d64_many": lambda: configs.fewshot(n_req=70, prefix=65, suffix=3, n_decode=2, h=2, d=64,
                                                     num_slots=8192),
    "two_level_bf16": lambda: configs.two_level(system=100, n_blocks=3, block=70, n_q=4, q=9, n_decode=3,
                                                h=4, num_slots=8192),
    "self_consistency_gqa8": lambda: configs.self_consistency(prefix=200, n_branch=12, max_branch=90,
                                                              n_decode=4, h_q=16, h_kv=2, num_slots=8192),
    "self_consistency_gqa16_zero_branch": lambda: configs.self_consistency(prefix=70, n_branch=40,
                                                                           max_branch=2, n_decode=2, h_q=16,
                                                                           h_kv=1, num_slots=4096),
    "multi_turn_evicting": lambda: configs.multi_turn(n_sessions=12, max_depth=3, median=40, lo=4, hi=150,
                                                      system=30, h_q=8, h_kv=2, max_running=6,
                                                      max_extend_tokens=400),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_trace_every_output(name):
    job = SMALL[name]()
    say(f"trace {name}: {job.dtype} h_q={job.h_q} h_kv={job.h_kv} d={job.d} "
        f"requests={len(job.requests)} steps={len(job.steps)}")
    runner, got = _collect(job)
    _check_host(job, runner)
    worst = _check_outputs(job, got, TOL[job.dtype])
    say(f"  checked {len(got)} outputs, worst max-abs {worst:.3g}")
    if name == "multi_turn_evicting":
        assert any(e[0] == "evict" for e in runner.log)
    if name == "self_consistency_gqa16_zero_branch":
        assert 0 in job.notes["branch_lens"]


@pytest.mark.parametrize("host_slots", [300, 20000])
def test_small_trace_host_tier_every_output(host_slots):
    """Evicting multi-turn trace with a host tier: events and dumps equal the oracle's replay
    (rules H1-H5), and every output, including those over promoted prefixes, matches
    attention recomputed from scratch."""
    job = SMALL["multi_turn_evicting"]()
    say(f"trace multi_turn_evicting with a host tier of {host_slots} rows")
    runner, got = _collect(job, runner_kw=dict(host_slots=host_slots))
    _check_host(job, runner, host_slots)
    worst = _check_outputs(job, got, TOL[job.dtype])
    st = runner.rt.tree.stats()
    say(f"  checked {len(got)} outputs, worst max-abs {worst:.3g}; demoted {st['demoted_tokens']} "
        f"promoted {st['promoted_tokens']}")
    assert st["demoted_tokens"] > 0 and st["promoted_tokens"] > 0 and st["pending_moves"] == 0
    plain = run_trace(job)
    assert run_trace(job, host_slots=host_slots)["computed"] < plain["computed"]


def test_kv_moves_bit_exact():
    """Demotion copies pool rows to the pinned host tier and promotion copies them back,
    bit for bit, in the tree's order (bf16 [*, 8, 128] and fp32 [*, 4, 64])."""
    from prefix_shared_kv_extend_amd import _lib
    g = torch.Generator().manual_seed(3)
    for dt, h, d in ((torch.bfloat16, 8, 128), (torch.float32, 4, 64)):
        say(f"kv moves: {dt} rows [{h}, {d}]")
        S, H = 600, 700
        kp = torch.randn((S, h, d), generator=g).to(dt).cuda()
        vp = torch.randn((S, h, d), generator=g).to(dt).cuda()
        kh = torch.zeros((H, h, d), dtype=dt, pin_memory=True)
        vh = torch.zeros((H, h, d), dtype=dt, pin_memory=True)
        t = _lib.Tree(S)
        t.set_host_tier(H, kh, vh)
        seqs = [list(range(i * 1000, i * 1000 + 150)) for i in range(4)]
        slots = [t.alloc_slots(150) for _ in seqs]
        for q, sl in zip(seqs, slots):
            t.insert(q, sl)
        want_k = {i: kp[torch.from_numpy(sl).long().cuda()].cpu() for i, sl in enumerate(slots)}
        want_v = {i: vp[torch.from_numpy(sl).long().cuda()].cpu() for i, sl in enumerate(slots)}
        freed = t.evict_lru(450)                       # three sequences go to the host
        assert len(freed) == 450 and t.stats()["host_tokens"] == 450
        t.run_moves(kp, vp)
        torch.cuda.synchronize()
        dump = {d_[5][0]: d_ for d_ in t.dump()}
        for i, q in enumerate(seqs):
            sl = np.array(dump[q[0]][6])
            if sl[0] < 0:
                idx = torch.from_numpy(-1 - sl).long()
                assert torch.equal(kh[idx], want_k[i]) and torch.equal(vh[idx], want_v[i])
        kp[torch.from_numpy(freed).long().cuda()] = 0     # the freed rows get reused
        vp[torch.from_numpy(freed).long().cuda()] = 0
        ip = np.cumsum([0] + [150] * 4)
        done, fr = t.promote_batch(np.concatenate([np.asarray(q, np.int32) for q in seqs]), ip)
        assert int(done.sum()) == 450
        t.run_moves(kp, vp)
        torch.cuda.synchronize()
        for i, q in enumerate(seqs):
            m, sl, _ = t.match_prefix(q)
            if m == 150:
                idx = torch.from_numpy(sl).long().cuda()
                assert torch.equal(kp[idx].cpu(), want_k[i]) and torch.equal(vp[idx].cpu(), want_v[i])
        assert t.stats()["host_tokens"] + t.stats()["cached_tokens"] == 600
    assert _lib.device_errors() == 0


def test_bf16_output_dtype():
    job = configs.fewshot(n_req=3, prefix=100, suffix=20, n_decode=2, h=4, num_slots=2048)
    say("fewshot with bf16 outputs")
    runner, got = _collect(job, runner_kw=dict(out_dtype=torch.bfloat16))
    _check_outputs(job, got, TOL["bf16"])


# ------------------------------------------------------------- full-size configs
def _pick_sampled(job, rng, per_step=3):
    """Extend: per_step random requests of every extend batch plus its first and last, at
    their last position and every 97th. Decode: per_step random requests at every 8th
    step and the last, and per_step fixed requests (the first decode batch's first, middle
    and last) at every decode step."""
    ext = {}
    dec = {}
    fixed = set()
    for si, st in enumerate(job.steps):
        if st.extend:
            ext[si] = set(rng.choice(st.extend, size=min(per_step, len(st.extend)), replace=False).tolist())
            ext[si] |= {st.extend[0], st.extend[-1]}
        if st.decode:
            dec[si] = set(rng.choice(st.decode, size=min(per_step, len(st.decode)), replace=False).tolist())
            if not fixed:
                fixed = {st.decode[0], st.decode[len(st.decode) // 2], st.decode[-1]}

    def pick(kind, si, rid, p):
        if kind == "extend":
            r = job.requests[rid]
            return rid in ext.get(si, ()) and (p == r.n - 1 or p % 97 == 0)
        return rid in fixed or (rid in dec.get(si, ()) and (si % 8 == 0 or si == len(job.steps) - 1))
    return pick


@pytest.mark.parametrize("index", [1, 2, 3])
def test_full_config_sampled(index):
    job = configs.make(index)
    say(f"config {index} ({job.name}) full size: requests={len(job.requests)} steps={len(job.steps)}")
    rng = np.random.default_rng(index)
    runner, got = _collect(job, pick=_pick_sampled(job, rng), progress=16)
    _check_host(job, runner)
    worst = _check_outputs(job, got, TOL[job.dtype])
    say(f"  checked {len(got)} sampled outputs, worst max-abs {worst:.3g}")


_MT = {}


def _multi_turn_plan(job):
    """Sampled outputs of the full multi-turn trace: one extend and one decode request on
    every 50th step and on every 50th step with an eviction, split in three parts; and
    three fixed long-context requests (100..300 generated tokens each) at every decode
    step and the last position of their extend."""
    from prefix_shared_kv_extend_amd.driver import tree_replay
    log, _, tree, _ = tree_replay(job)
    tree.close()
    ev_steps = sorted({e[1] for e in log if e[0] == "evict"})
    steps = sorted(set(range(0, len(job.steps), 50)) | set(ev_steps[::50]))
    rng = np.random.default_rng(4)
    chosen = {}
    for si in steps:
        st = job.steps[si]
        c = []
        if st.extend:
            c.append(("extend", int(rng.choice(st.extend))))
        if st.decode:
            c.append(("decode", int(rng.choice(st.decode))))
        chosen[si] = c
    fixed = [r.rid for r in job.requests if 100 <= len(r.output) <= 300 and r.n >= 1000][:3]
    return steps, chosen, fixed, ev_steps


def _multi_turn_run():
    """One GPU run of the full multi-turn trace, shared by the tests below (cached)."""
    if "got" in _MT:
        return _MT
    job = configs.make(4)
    steps, chosen, fixed, ev_steps = _multi_turn_plan(job)
    say(f"config 4 (multi_turn) full size: requests={len(job.requests)} steps={len(job.steps)} "
        f"pool={job.num_slots}; {len(steps)} sampled steps ({len(ev_steps)} steps evict), fixed requests {fixed}")
    fixed_set = set(fixed)

    def pick(kind, si, rid, p):
        if rid in fixed_set:
            return kind == "decode" or p == job.requests[rid].n - 1
        if (kind, rid) not in chosen.get(si, ()):
            return False
        return kind == "decode" or p == job.requests[rid].n - 1 or p % 211 == 0

    from prefix_shared_kv_extend_amd import _lib
    runner, got = _collect(job, pick=pick, progress=1000)
    _MT.update(job=job, steps=steps, chosen=chosen, fixed=fixed, got=got, log=runner.log,
               rows=runner.final_rows, dump=runner.rt.tree.dump(), errors=_lib.device_errors())
    del runner
    torch.cuda.empty_cache()
    return _MT


def test_full_multi_turn_host_log():
    mt = _multi_turn_run()
    say("  GPU run done; replaying the trace in the oracle")
    ref = run_trace(mt["job"])
    assert mt["errors"] == 0
    assert len(mt["log"]) == len(ref["log"])
    for a, b in zip(mt["log"], ref["log"]):
        assert a == b
    assert mt["rows"] == ref["rows"] and mt["dump"] == ref["dump"]
    say(f"  host log identical ({len(ref['log'])} events, {sum(1 for e in ref['log'] if e[0] == 'evict')} evictions)")


@pytest.mark.parametrize("part", range(3))
def test_full_multi_turn_sampled(part):
    mt = _multi_turn_run()
    job = mt["job"]
    mine = set(mt["steps"][part::3])
    keep = {(k, r) for si in mine for k, r in mt["chosen"].get(si, ())}
    # the outputs the run kept for the requests chosen at this part's steps
    rids = {r for _, r in keep} - set(mt["fixed"])
    got = {(rid, p): o for (rid, p), o in mt["got"].items() if rid in rids}
    worst = _check_outputs(job, got, TOL[job.dtype])
    say(f"  part {part}: {len(mine)} steps, checked {len(got)} sampled outputs, worst max-abs {worst:.3g}")
    assert got


def test_full_multi_turn_fixed_requests_every_step():
    mt = _multi_turn_run()
    job = mt["job"]
    got = {(rid, p): o for (rid, p), o in mt["got"].items() if rid in mt["fixed"]}
    for rid in mt["fixed"]:
        r = job.requests[rid]
        assert sum(1 for (x, p) in got if x == rid and p >= r.n) == len(r.output)
    worst = _check_outputs(job, got, TOL[job.dtype])
    say(f"  fixed requests {mt['fixed']}: {len(got)} outputs (every decode step), worst max-abs {worst:.3g}")


# ------------------------------------------------------------- QKV projection (fused write-back)
@pytest.mark.parametrize("t,hidden,h_q,h_kv,d", [(300, 256, 4, 2, 128), (77, 512, 8, 2, 64), (1, 128, 1, 1, 128),
                                                  (1100, 256, 1, 1, 128), (1300, 512, 8, 2, 64),
                                                  (800, 128, 32, 32, 128), (1500, 128, 32, 32, 128)])
def test_qkv_project_small(t, hidden, h_q, h_kv, d):
    """Every output of the fused projection against the fp64 oracle (bf16 rounding of fp32
    sums: max-abs 2e-2 at values of order 1), and the pool rows bit for bit equal to the
    contiguous K/V outputs; untouched pool rows stay zero. From 1024 tokens the kernel takes
    256 x 256 tiles: 1100 tokens (a ragged last token block) with 384 output features (the
    second feature block half past the end), and 1300 tokens with 768. With 12288 output
    features, 800 tokens make 672 tiles of 128 x 128 and 1500 tokens 288 of 256 x 256, so
    the last partial round (160 and 32 tiles) runs as half tiles, the ragged last token
    block among them."""
    from oracle.projection import qkv_project
    from prefix_shared_kv_extend_amd import _lib
    from workloads.gen import projection_inputs
    say(f"qkv projection: T={t} hidden={hidden} h_q={h_q} h_kv={h_kv} d={d}")
    n_out = (h_q + 2 * h_kv) * d
    x, w = projection_inputs(11, t, hidden, n_out)
    S = 3 * t + 5
    loc = torch.randperm(S, generator=torch.Generator().manual_seed(2))[:t].to(torch.int32)
    kp = torch.zeros((S, h_kv, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    q, k, v = _lib.qkv_project(x.to(torch.bfloat16).cuda(), w.to(torch.bfloat16).cuda(), h_q, h_kv,
                               out_loc=loc.cuda(), k_pool=kp, v_pool=vp)
    torch.cuda.synchronize()
    rq, rk, rv = qkv_project(x.numpy(), w.numpy(), h_q, h_kv, d)
    for got, ref in ((q, rq), (k, rk), (v, rv)):
        err = float(np.abs(got.float().cpu().numpy() - ref).max())
        assert err <= 2e-2, err
    kp, vp, loc = kp.cpu(), vp.cpu(), loc.long()
    assert torch.equal(kp[loc], k.cpu()) and torch.equal(vp[loc], v.cpu())
    rest = torch.ones(S, dtype=torch.bool)
    rest[loc] = False
    assert int(kp[rest].abs().sum()) == 0 and int(vp[rest].abs().sum()) == 0
    assert _lib.device_errors() == 0


def test_qkv_project_full_size_sampled():
    """The cached few-shot extend batch's projection (3150 tokens, hidden 4096, 32 heads x
    128): sampled token rows against the oracle; the pool copy bit-exact."""
    from oracle.projection import qkv_project_rows
    from prefix_shared_kv_extend_amd import _lib
    from workloads.gen import projection_inputs
    t, hidden, h, d = 3150, 4096, 32, 128
    say(f"qkv projection full size: T={t} hidden={hidden} heads={h} d={d}")
    x, w = projection_inputs(12, t, hidden, 3 * h * d)
    loc = torch.arange(t, dtype=torch.int32) * 3 + 1
    kp = torch.zeros((3 * t + 2, h, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    q, k, v = _lib.qkv_project(x.to(torch.bfloat16).cuda(), w.to(torch.bfloat16).cuda(), h, h,
                               out_loc=loc.cuda(), k_pool=kp, v_pool=vp)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 1000, 2047, 3071, 3072, 3149]
    rq, rk, rv = qkv_project_rows(x.numpy(), w.numpy(), rows, h, h, d)
    for got, ref in ((q, rq), (k, rk), (v, rv)):
        err = float(np.abs(got[rows].float().cpu().numpy() - ref).max())
        assert err <= 2e-2, err
    assert torch.equal(kp[loc.long().cuda()], k) and torch.equal(vp[loc.long().cuda()], v)
    assert _lib.device_errors() == 0


def test_qkv_project_errors_and_flagged_slots():
    from prefix_shared_kv_extend_amd import _lib
    say("qkv projection: argument errors, out-of-range slot flagged and skipped")
    x = torch.ones((4, 96), dtype=torch.bfloat16, device="cuda")          # hidden % 64 != 0
    w = torch.ones((384, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.RaxError) as e:
        _lib.qkv_project(x, w, 1, 1)
    assert e.value.status == _lib.EINVAL
    x = torch.ones((4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((384, 64), dtype=torch.bfloat16, device="cuda") / 64
    kp = torch.zeros((8, 1, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    q, k, v = _lib.qkv_project(x, w, 1, 1, out_loc=torch.tensor([0, 8, -1, 3], dtype=torch.int32, device="cuda"),
                               k_pool=kp, v_pool=vp)
    assert _lib.device_errors() == _lib.DEVERR_SLOT
    assert float(kp[0].float().sum()) == 128 and float(kp[3].float().sum()) == 128
    assert float(kp.float().sum()) == 256 and float(q.float().sum()) == 4 * 128


def test_decode_step_folded_append_equals_separate_calls():
    """rax_decode_step carries the append in the first attention kernel (bf16, D = 128): the
    slots, rows, lengths, pools and outputs equal those of rax_decode_append followed by
    rax_decode_attention_hinted (the same layout) on an identical runtime, bit for bit, over
    several steps (70 requests, GQA 16/4, five row blocks); plain rax_decode_attention, laid
    out from the longest sequence, agrees within the bf16 tolerance."""
    from prefix_shared_kv_extend_amd import _lib
    from prefix_shared_kv_extend_amd.runtime import RadixRuntime
    say("decode step with the append folded in vs separate append + attention (bf16, g = 4)")
    h_q, h_kv, d, B = 16, 4, 128, 70
    rng = np.random.default_rng(5)
    pre = rng.integers(0, 50, 120)
    prompts = [np.concatenate([pre, rng.integers(0, 50, int(rng.integers(1, 30)))]).astype(np.int32)
               for _ in range(B)]
    gen = torch.Generator().manual_seed(9)

    def rnd(*shape):
        return torch.randn(shape, generator=gen).to(torch.bfloat16).cuda()

    rts = []
    for _ in range(2):
        rt = RadixRuntime(16384, h_q, h_kv, d, torch.bfloat16, B, 400)
        rts.append((rt, rt.begin_extend(list(enumerate(prompts)))))
    t = rts[0][1].total_q
    q, k, v = rnd(t, h_q, d), rnd(t, h_kv, d), rnd(t, h_kv, d)
    for rt, eb in rts:
        rt.run_extend(eb, q, k, v, torch.empty((t, h_q, d), dtype=torch.bfloat16, device="cuda"))
        rt.end_extend(eb)
    (ra, _), (rb, _) = rts
    rids = list(range(B))
    for step in range(3):
        qd, kd, vd = rnd(B, h_q, d), rnd(B, h_kv, d), rnd(B, h_kv, d)
        oa = torch.empty((B, h_q, d), dtype=torch.bfloat16, device="cuda")
        ra.run_decode(ra.begin_decode(rids), qd, kd, vd, oa)
        rb.begin_decode(rids)
        ds = rb._dec_cache
        new, _ = rb.tree.decode_append(ds.lens, rb.rtt, ds.inv["req_pool_idx"], ds.inv["seq_len"], kd, vd,
                                       rb.k_pool, rb.v_pool)
        rb.rows[ds.req_rows, ds.lens - 1] = new
        mx = int(ds.lens.max())
        ob = torch.empty_like(oa)
        # the same layout as the decode step: sized from host copies of the lengths and hints
        hinted = lambda w: _lib.decode_attention_hinted(qd, rb.k_pool, rb.v_pool, rb.rtt, ds.inv["req_pool_idx"],
                                                        ds.inv["seq_len"], mx, ob, ds.lens, ds.hints, workspace=w,
                                                        shared_len=ds.inv["shared_len"])
        hinted(torch.empty(hinted(None), dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"step {step}"
        # and the plain call (layout from the longest sequence) within the bf16 tolerance
        oc = torch.empty_like(oa)
        ws = torch.empty(_lib.attention_workspace_bytes(True, B, h_q, h_kv, d, mx), dtype=torch.uint8, device="cuda")
        _lib.decode_attention(qd, rb.k_pool, rb.v_pool, rb.rtt, ds.inv["req_pool_idx"], ds.inv["seq_len"], mx, oc,
                              workspace=ws, shared_len=ds.inv["shared_len"])
        torch.cuda.synchronize()
        assert float((oa.float() - oc.float()).abs().max()) <= TOL["bf16"], f"step {step}"
        assert np.array_equal(ra._dec_cache.lens, ds.lens)
        assert torch.equal(ra._dec_cache.inv["seq_len"], ds.inv["seq_len"])
    assert torch.equal(ra.rtt, rb.rtt) and np.array_equal(ra.rows, rb.rows)
    assert torch.equal(ra.k_pool, rb.k_pool) and torch.equal(ra.v_pool, rb.v_pool)
    assert _lib.device_errors() == 0


def test_decode_step_above_append_limit_every_output():
    """A decode step of 300 requests, more than the 256 whose append one attention launch
    can carry: rax_decode_step appends in a launch of its own, and the attention, laid out
    from the host's lengths and hints, runs without a host work list (requests in batch
    order). Runtime path (GQA 16/4, bf16, a 96-token prefix shared by all prompts), two
    steps; after each, the new tokens' K/V rows in the pools equal the inputs bit for bit,
    and every output is compared with fp64 attention over the request's keys read back
    from the pools (oracle.attention.attend)."""
    from oracle.attention import attend
    from prefix_shared_kv_extend_amd import _lib
    from prefix_shared_kv_extend_amd.runtime import RadixRuntime
    h_q, h_kv, d, B = 16, 4, 128, 300
    say(f"decode step above the folded-append limit: {B} requests, GQA {h_q}/{h_kv}")
    rng = np.random.default_rng(31)
    pre = rng.integers(0, 50, 96)
    prompts = [np.concatenate([pre, rng.integers(0, 50, int(rng.integers(1, 40)))]).astype(np.int32)
               for _ in range(B)]
    gen = torch.Generator().manual_seed(17)

    def rnd(*shape):
        return torch.randn(shape, generator=gen).to(torch.bfloat16).cuda()

    rt = RadixRuntime(32768, h_q, h_kv, d, torch.bfloat16, B, 256)
    # the first prompt alone, so that the others find the prefix in the tree
    for part in (list(enumerate(prompts))[:1], list(enumerate(prompts))[1:]):
        eb = rt.begin_extend(part)
        t = eb.total_q
        rt.run_extend(eb, rnd(t, h_q, d), rnd(t, h_kv, d), rnd(t, h_kv, d),
                      torch.empty((t, h_q, d), dtype=torch.bfloat16, device="cuda"))
        rt.end_extend(eb)
    assert int(np.min(eb.prefix_len)) >= len(pre)
    rids = list(range(B))
    worst = 0.0
    for step in range(2):
        qd, kd, vd = rnd(B, h_q, d), rnd(B, h_kv, d), rnd(B, h_kv, d)
        o = torch.empty((B, h_q, d), dtype=torch.bfloat16, device="cuda")
        db = rt.begin_decode(rids)
        rt.run_decode(db, qd, kd, vd, o)
        torch.cuda.synchronize()
        assert _lib.device_errors() == 0
        ds = rt._dec_cache
        assert np.array_equal(ds.lens, db.seq_len)
        kf, vf = rt.k_pool.cpu(), rt.v_pool.cpu()
        newest = torch.as_tensor(rt.rows[ds.req_rows, ds.lens - 1].astype(np.int64))
        assert torch.equal(kf[newest], kd.cpu()) and torch.equal(vf[newest], vd.cpu()), f"step {step}"
        kf, vf, qf, got = kf.float().numpy(), vf.float().numpy(), qd.float().cpu().numpy(), o.float().cpu().numpy()
        for i in range(B):
            sl = rt.rows[ds.req_rows[i], : ds.lens[i]]
            err = float(np.abs(got[i] - attend(qf[i], kf[sl], vf[sl])).max())
            worst = max(worst, err)
            assert err <= TOL["bf16"], f"step {step}, request {i}: max abs err {err:.3g}"
    say(f"  worst max-abs {worst:.3g} over {B} requests x 2 steps")


@pytest.mark.parametrize("h_q,h_kv,P,n_req", [(4, 2, 150, 12), (32, 4, 150, 12), (64, 4, 150, 12),
                                             (12, 3, 150, 12), (16, 1, 150, 12),
                                             (16, 2, 2100, 256), (32, 8, 150, -72), (32, 16, 150, -64)])
def test_decode_query_head_groups_direct(h_q, h_kv, P, n_req):
    """Decode attention with query-head groups (own keys on MFMA tiles) on hand-built rows:
    a P-key prefix shared by all requests (hinted), then own ranges of 0..2600 keys, so
    that chunks are empty, shorter than a tile, exactly one or two tiles, ragged, several
    per (request, KV head), and longer than one round of tiles. The sixth case has 64 row
    blocks and a 2100-key prefix, so the shared part runs in 4-wave workgroups with two
    tiles per round and several rounds per split. An odd number of KV heads (3, and 1)
    takes the own part's one-head workgroups. The last two (n_req < 0: -n_req
    requests) give every request 1100..1400 own keys: with 72 x 8 (request, KV head)
    pairs, two chunks each, so many items of requests with several chunks that these merge
    in the merge kernel (in the other cases the own part's launch merges them itself); with
    64 x 16 pairs, enough to fill the GPU, one chunk of more than 1024 keys per request and
    no merge. Outputs against fp64 attention over each request's keys
    (oracle.attention.attend): every request, or 64 spread ones."""
    from oracle.attention import attend
    from prefix_shared_kv_extend_amd import _lib
    say(f"decode, query-head groups {h_q}/{h_kv}, {n_req} requests: own ranges 0..2600 keys past a {P}-key "
        f"shared prefix")
    d, S = 128, 1 << 17
    base = [0, 1, 63, 64, 65, 127, 128, 129, 300, 1100, 2600, 7]
    if n_req < 0:
        own = [1100 + (i * 97) % 301 for i in range(-n_req)]
    else:
        own = (base * (n_req // len(base) + 1))[:n_req] if n_req <= len(base) else \
            [base[i % len(base)] if i % 16 == 0 else int(i % 41) for i in range(n_req)]
    B = len(own)
    W = P + max(own) + 2
    gen = torch.Generator().manual_seed(23 + h_q + P)
    k_pool = torch.randn((S, h_kv, d), generator=gen).to(torch.bfloat16)
    v_pool = torch.randn((S, h_kv, d), generator=gen).to(torch.bfloat16)
    q = torch.randn((B, h_q, d), generator=gen).to(torch.bfloat16)
    perm = torch.randperm(S, generator=gen).numpy().astype(np.int32)
    rtt = np.full((B + 3, W), -1, dtype=np.int32)
    rows = np.arange(B, dtype=np.int32) + 2                 # rows 0, 1 stay unused
    prefix_slots = perm[:P]
    used = P
    lens = []
    for i, n in enumerate(own):
        ln = P + n + 1                                      # the newest key is always in the own part
        rtt[rows[i], :P] = prefix_slots
        rtt[rows[i], P:ln] = perm[used: used + ln - P]
        used += ln - P
        lens.append(ln)
    assert used <= S
    lens = np.array(lens, dtype=np.int32)
    hints = np.full(B, P, dtype=np.int32)
    dev = lambda x: torch.as_tensor(x).cuda()
    ws = torch.empty(_lib.attention_workspace_bytes(True, B, h_q, h_kv, d, int(lens.max())), dtype=torch.uint8,
                     device="cuda")
    ob = torch.empty((B, h_q, d), dtype=torch.bfloat16, device="cuda")
    _lib.decode_attention(dev(q), dev(k_pool), dev(v_pool), dev(rtt), dev(rows), dev(lens), int(lens.max()), ob,
                          workspace=ws, shared_len=dev(hints))
    # the same call laid out from host copies (the own part as a work queue of waves)
    oh = torch.empty_like(ob)
    hinted = lambda w: _lib.decode_attention_hinted(dev(q), dev(k_pool), dev(v_pool), dev(rtt), dev(rows),
                                                    dev(lens), int(lens.max()), oh, lens, hints, workspace=w,
                                                    shared_len=dev(hints))
    hinted(torch.empty(hinted(None), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert _lib.device_errors() == 0
    outs = (ob.float().cpu().numpy(), oh.float().cpu().numpy())
    kf, vf, qf = k_pool.float().numpy(), v_pool.float().numpy(), q.float().numpy()
    worst = 0.0
    check = range(B) if B <= 64 else sorted(set(np.linspace(0, B - 1, 64).astype(int).tolist()))
    for i in check:
        sl = rtt[rows[i], : lens[i]]
        ref = attend(qf[i], kf[sl], vf[sl])
        for got in outs:
            err = float(np.abs(got[i] - ref).max())
            worst = max(worst, err)
            assert err <= TOL["bf16"], f"request {i} (own {own[i]}): max abs err {err:.3g}"
    say(f"  worst max-abs {worst:.3g} over {len(check)} requests, plain and hinted layouts")


@pytest.mark.parametrize("h_q,h_kv,d,dt", [(32, 8, 128, "bf16"), (16, 16, 128, "bf16"), (8, 8, 64, "f32")])
def test_decode_long_request_many_own_chunks(h_q, h_kv, d, dt):
    """Decode where one request holds 20,000 own keys past a 100-key shared prefix, beside
    requests of 3000, 64, 1 and 0 own keys: the long request's own part is cut into many
    chunks (more than the four of shorter requests, more than the eight the MHA own part
    merges by itself), whose partials the merge combines with the shared part's splits.
    GQA 32/8 and MHA in bf16 (D = 128), MHA in fp32 (D = 64); plain and hinted layouts;
    every output against fp64 attention over the request's keys (oracle.attention.attend)."""
    from oracle.attention import attend
    from prefix_shared_kv_extend_amd import _lib
    say(f"decode, one request of 20000 own keys: {h_q}/{h_kv} heads, d={d}, {dt}")
    P, own = 100, [20000, 1, 0, 3000, 64]
    B = len(own)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    lens = np.array([P + n + 1 for n in own], dtype=np.int32)
    S = int(lens.sum()) + 64
    W = int(lens.max()) + 3
    gen = torch.Generator().manual_seed(41 + h_q + d)
    k_pool = torch.randn((S, h_kv, d), generator=gen).to(tdt)
    v_pool = torch.randn((S, h_kv, d), generator=gen).to(tdt)
    q = torch.randn((B, h_q, d), generator=gen).to(tdt)
    perm = torch.randperm(S, generator=gen).numpy().astype(np.int32)
    rtt = np.full((B + 2, W), -1, dtype=np.int32)
    rows = np.array([3, 0, 5, 1, 2], dtype=np.int32)
    used = P
    for i in range(B):
        rtt[rows[i], :P] = perm[:P]
        rtt[rows[i], P:lens[i]] = perm[used: used + lens[i] - P]
        used += lens[i] - P
    assert used <= S
    hints = np.full(B, P, dtype=np.int32)
    dev = lambda x: torch.as_tensor(x).cuda()
    ws = torch.empty(_lib.attention_workspace_bytes(True, B, h_q, h_kv, d, int(lens.max())), dtype=torch.uint8,
                     device="cuda")
    ob = torch.empty((B, h_q, d), dtype=torch.float32, device="cuda")
    _lib.decode_attention(dev(q), dev(k_pool), dev(v_pool), dev(rtt), dev(rows), dev(lens), int(lens.max()), ob,
                          workspace=ws, shared_len=dev(hints))
    oh = torch.empty_like(ob)
    hinted = lambda w: _lib.decode_attention_hinted(dev(q), dev(k_pool), dev(v_pool), dev(rtt), dev(rows),
                                                    dev(lens), int(lens.max()), oh, lens, hints, workspace=w,
                                                    shared_len=dev(hints))
    hinted(torch.empty(hinted(None), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert _lib.device_errors() == 0
    kf, vf, qf = k_pool.double().numpy(), v_pool.double().numpy(), q.double().numpy()
    worst = 0.0
    for i in range(B):
        sl = rtt[rows[i], : lens[i]]
        ref = attend(qf[i], kf[sl], vf[sl])
        for got in (ob.cpu().numpy(), oh.cpu().numpy()):
            err = float(np.abs(got[i] - ref).max())
            worst = max(worst, err)
            assert err <= TOL[dt], f"request {i} (own {own[i]}): max abs err {err:.3g}"
    say(f"  worst max-abs {worst:.3g} over {B} requests, plain and hinted layouts")


@pytest.mark.parametrize("d,B", [(64, 150), (128, 131)])
def test_decode_fp32_mha_many_requests_direct(d, B):
    """fp32 MHA decode with more than 128 requests, so row blocks are full and there are
    several of them: a shared prefix (hinted for most neighbours, with some hints cut
    short), own ranges of 0..300 keys. Every output against fp64 attention over the
    request's keys (oracle.attention.attend) within 1e-5."""
    from oracle.attention import attend
    from prefix_shared_kv_extend_amd import _lib
    h, S, P = 4, 1 << 15, 97
    say(f"decode fp32 MHA, {B} requests, d={d}: {P}-key prefix, own ranges 0..300")
    gen = torch.Generator().manual_seed(977 + d)
    perm = torch.randperm(S, generator=gen).numpy().astype(np.int32)
    own = [(i * 37) % 301 for i in range(B)]
    lens = np.array([P + n + 1 for n in own], dtype=np.int32)
    W = int(lens.max()) + 1
    rtt = np.full((B + 1, W), -1, dtype=np.int32)
    rows = (np.arange(B, dtype=np.int32) * 7) % (B + 1)      # shuffled, distinct rows
    used = P
    for i in range(B):
        rtt[rows[i], :P] = perm[:P]
        rtt[rows[i], P:lens[i]] = perm[used: used + lens[i] - P]
        used += lens[i] - P
    assert used <= S and len(set(rows.tolist())) == B
    hints = np.array([P if i % 9 else P // 2 for i in range(B)], dtype=np.int32)
    k_pool = torch.randn((S, h, d), generator=gen)
    v_pool = torch.randn((S, h, d), generator=gen)
    q = torch.randn((B, h, d), generator=gen)
    dev = lambda x: torch.as_tensor(x).cuda()
    ws = torch.empty(_lib.attention_workspace_bytes(True, B, h, h, d, int(lens.max())), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((B, h, d), dtype=torch.float32, device="cuda")
    _lib.decode_attention(dev(q), dev(k_pool), dev(v_pool), dev(rtt), dev(rows), dev(lens), int(lens.max()), o,
                          workspace=ws, shared_len=dev(hints))
    torch.cuda.synchronize()
    assert _lib.device_errors() == 0
    got = o.cpu().numpy()
    kf, vf, qf = k_pool.numpy(), v_pool.numpy(), q.numpy()
    worst = 0.0
    for i in range(B):
        sl = rtt[rows[i], : lens[i]]
        err = float(np.abs(got[i] - attend(qf[i], kf[sl], vf[sl])).max())
        worst = max(worst, err)
        assert err <= TOL["f32"], f"request {i} (own {own[i]}): max abs err {err:.3g}"
    say(f"  worst max-abs {worst:.3g} over {B} requests")


def test_decode_step_rejects_strided_and_host_tensors():
    """rax_decode_step's binding checks every per-step tensor before the native call."""
    from prefix_shared_kv_extend_amd import _lib
    say("decode_step binding: strided q and host k_new are refused")
    h, d, B = 4, 128, 3
    t = _lib.Tree(64)
    kp = torch.zeros((64, h, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    rtt = torch.zeros((4, 16), dtype=torch.int32, device="cuda")
    rows = torch.arange(B, dtype=torch.int32, device="cuda")
    lens = np.zeros(B, dtype=np.int32)
    prep = t.decode_step_prepare(lens, rtt, rows, torch.zeros(B, dtype=torch.int32, device="cuda"), kp, vp, h)
    q = torch.zeros((B, h, d), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((B, h, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    wide = torch.zeros((B, h, 2 * d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        t.decode_step(prep, wide[:, :, :d], kn, kn, o, None)
    with pytest.raises(ValueError):
        t.decode_step(prep, q, kn.cpu(), kn, o, None)
    assert t.free_count() == 64                              # nothing was allocated


@pytest.mark.parametrize("dt,h_q,h_kv,d,reqs", [
    ("bf16", 32, 8, 128, [(1800, 300)]),
    ("bf16", 32, 8, 128, [(1500, 200), (0, 77), (1700, 64)]),
    ("bf16", 4, 4, 128, [(2100, 130), (900, 1)]),
    ("f32", 8, 2, 64, [(1300, 150), (640, 33)]),
    ("f32", 4, 4, 128, [(1100, 90)]),
])
def test_extend_key_split_direct(dt, h_q, h_kv, d, reqs):
    """Extend calls of few long requests, whose key ranges are split over several workgroups
    (partials merged by log-sum-exp): hand-built prefixes in shuffled pool slots and
    suffixes in k_ext/v_ext. Every output against fp64 attention over the request's keys
    (oracle.attention.attend), with and without the workspace that enables the split."""
    from oracle.attention import attend
    from prefix_shared_kv_extend_amd import _lib
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    say(f"extend key split: {dt} {h_q}/{h_kv} d={d}, (prefix, suffix) = {reqs}")
    S = 1 << 14
    gen = torch.Generator().manual_seed(331 + h_q + d + len(reqs))
    perm = torch.randperm(S, generator=gen).numpy().astype(np.int32)
    B = len(reqs)
    W = max(m + n for m, n in reqs) + 5
    rtt = np.full((B + 2, W), -1, dtype=np.int32)
    rows = np.arange(B, dtype=np.int32) + 1
    used = 0
    for i, (m, n) in enumerate(reqs):
        rtt[rows[i], :m] = perm[used: used + m]
        used += m
    qo = np.zeros(B + 1, dtype=np.int32)
    qo[1:] = np.cumsum([n for _, n in reqs])
    T = int(qo[-1])
    prefix = np.array([m for m, _ in reqs], dtype=np.int32)
    max_kv = int(max(m + n for m, n in reqs))
    k_pool = torch.randn((S, h_kv, d), generator=gen).to(tdt)
    v_pool = torch.randn((S, h_kv, d), generator=gen).to(tdt)
    q = torch.randn((T, h_q, d), generator=gen).to(tdt)
    k_ext = torch.randn((T, h_kv, d), generator=gen).to(tdt)
    v_ext = torch.randn((T, h_kv, d), generator=gen).to(tdt)
    need = _lib.attention_workspace_bytes(False, T, h_q, h_kv, d, max_kv)
    assert need > 0, "the case must take the split path"
    dev = lambda x: torch.as_tensor(x).cuda()
    args = [dev(q), dev(k_ext), dev(v_ext), dev(k_pool), dev(v_pool), dev(rtt), dev(rows), dev(prefix), dev(qo)]
    outs = []
    for ws in (torch.empty(need, dtype=torch.uint8, device="cuda"), None):
        o = torch.empty((T, h_q, d), dtype=torch.float32, device="cuda")
        _lib.extend_attention(*args, o, workspace=ws, max_kv_len=max_kv)
        outs.append(o)
    torch.cuda.synchronize()
    assert _lib.device_errors() == 0
    kf, vf, qf = k_pool.double().numpy(), v_pool.double().numpy(), q.double().numpy()
    kef, vef = k_ext.double().numpy(), v_ext.double().numpy()
    got = [o.cpu().numpy() for o in outs]
    worst = 0.0
    for r, (m, n) in enumerate(reqs):
        sl = rtt[rows[r], :m]
        for i in range(n):
            t = int(qo[r]) + i
            K = np.concatenate([kf[sl], kef[qo[r]: t + 1]])
            V = np.concatenate([vf[sl], vef[qo[r]: t + 1]])
            ref = attend(qf[t], K, V)
            for g in got:
                err = float(np.abs(g[t] - ref).max())
                worst = max(worst, err)
                assert err <= TOL[dt], f"request {r} query {i}: max abs err {err:.3g}"
    say(f"  worst max-abs {worst:.3g} over {T} queries, split and unsplit")


# (h_q, h_kv, groups): each group is (requests, extra shared keys past the block prefix).
# Row blocks hold 64 / (h_q / h_kv) requests, so groups fall inside, across and exactly on
# block boundaries.
_RUN_CASES = [
    # MHA, 150 requests (3 blocks): runs of 1..30 requests, extra prefixes short of a tile,
    # exactly one, ragged, and several rounds of tiles; a group with no extra keys
    (4, 4, [(1, 0), (2, 1), (3, 63), (16, 64), (17, 65), (5, 0), (30, 700), (2, 129), (40, 200),
            (1, 500), (33, 1300)]),
    # query-head groups (own keys on MFMA tiles): 8 and 16 requests per block
    (64, 8, [(2, 100), (3, 64), (1, 0), (5, 900), (8, 1000), (4, 30), (2, 0), (7, 300)]),
    (16, 4, [(3, 200), (13, 520), (4, 1), (1, 0), (6, 64)]),
    # 64 requests in 32 pairs, each pair sharing 1000 keys past the block's: the extra
    # tiles exceed the per-block cap, so only the first pairs are computed as runs
    (4, 4, [(2, 1000)] * 32),
]


@pytest.mark.parametrize("case", range(len(_RUN_CASES)))
def test_decode_deeper_runs_direct(case):
    """Decode attention on hand-built two-level rows: a block prefix shared by every
    request (hinted), then groups of consecutive requests sharing more keys (hinted to
    their predecessor), then own keys. Groups of two or more requests become runs whose
    extra keys the shared-part kernel computes once for the group's rows, up to a per-block
    cap; their own parts start past the group's keys. Outputs against fp64 attention over
    each request's keys (oracle.attention.attend), every request."""
    from oracle.attention import attend
    from prefix_shared_kv_extend_amd import _lib
    h_q, h_kv, groups = _RUN_CASES[case]
    say(f"decode, deeper runs, case {case}: {h_q}/{h_kv} heads, {sum(n for n, _ in groups)} requests in "
        f"{len(groups)} groups")
    d, S, P = 128, 1 << 16, 300
    own_cycle = [0, 1, 5, 63, 64, 65, 130, 7, 260, 33]
    gen = torch.Generator().manual_seed(101 + case)
    perm = torch.randperm(S, generator=gen).numpy().astype(np.int32)
    used = P
    rows_keys, hints = [], []
    for gi, (n, extra) in enumerate(groups):
        ext = perm[used: used + extra]
        used += extra
        for j in range(n):
            own = own_cycle[(gi * 3 + j) % len(own_cycle)]
            mine = perm[used: used + own + 1]           # the newest key is always own
            used += own + 1
            rows_keys.append(np.concatenate([perm[:P], ext, mine]))
            hints.append(P + extra if j > 0 else P)
    assert used <= S
    B = len(rows_keys)
    lens = np.array([len(k) for k in rows_keys], dtype=np.int32)
    W = int(lens.max()) + 3
    rtt = np.full((B + 2, W), -1, dtype=np.int32)
    rows = np.arange(B, dtype=np.int32)[::-1].copy() + 1   # rows in reverse, row 0 unused
    for i, k in enumerate(rows_keys):
        rtt[rows[i], : len(k)] = k
    hints = np.array(hints, dtype=np.int32)
    k_pool = torch.randn((S, h_kv, d), generator=gen).to(torch.bfloat16)
    v_pool = torch.randn((S, h_kv, d), generator=gen).to(torch.bfloat16)
    q = torch.randn((B, h_q, d), generator=gen).to(torch.bfloat16)
    dev = lambda x: torch.as_tensor(x).cuda()
    ws = torch.empty(_lib.attention_workspace_bytes(True, B, h_q, h_kv, d, int(lens.max())), dtype=torch.uint8,
                     device="cuda")
    ob = torch.empty((B, h_q, d), dtype=torch.bfloat16, device="cuda")
    _lib.decode_attention(dev(q), dev(k_pool), dev(v_pool), dev(rtt), dev(rows), dev(lens), int(lens.max()), ob,
                          workspace=ws, shared_len=dev(hints))
    torch.cuda.synchronize()
    assert _lib.device_errors() == 0
    got = ob.float().cpu().numpy()
    # the same call laid out from host copies of the lengths and hints
    oh = torch.empty_like(ob)
    hinted = lambda w: _lib.decode_attention_hinted(dev(q), dev(k_pool), dev(v_pool), dev(rtt), dev(rows),
                                                    dev(lens), int(lens.max()), oh, lens, hints, workspace=w,
                                                    shared_len=dev(hints))
    need = hinted(None)
    hinted(torch.empty(max(need, 1), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert _lib.device_errors() == 0
    got_h = oh.float().cpu().numpy()
    kf, vf, qf = k_pool.float().numpy(), v_pool.float().numpy(), q.float().numpy()
    worst = 0.0
    for i in range(B):
        sl = rtt[rows[i], : lens[i]]
        ref = attend(qf[i], kf[sl], vf[sl])
        for out in (got, got_h):
            err = float(np.abs(out[i] - ref).max())
            worst = max(worst, err)
            assert err <= TOL["bf16"], f"request {i}: max abs err {err:.3g}"
    say(f"  worst max-abs {worst:.3g} over {B} requests, plain and hinted layouts")
