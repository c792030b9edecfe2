"""Request lifecycle over librax: the host side of RadixAttention's hot path.

Per batch (2312.07104_SGLang notes, App. A.2: match every request, form the batch
evicting when memory is short, run it, update the tree; hustzhy SGLang post,
§2.3 (2): traverse -> reuse -> compute -> insert):

  extend   match each prompt in the tree and lock the matched node
           (rax_match_prefix_batch); allocate slots for all unmatched suffixes at
           once (rax_alloc_slots_evict); fill the requests' req_to_token rows on the
           device; write the new tokens' K/V into the pool (rax_kv_scatter); run
           extend attention over reused prefix + causal suffix; then insert every
           prompt (rax_insert_batch) and move the locks to the new nodes.
  decode   allocate one slot per request, append it to the rows, write the new
           tokens' K/V, run decode attention over the whole rows: one native call
           (rax_decode_step) whose argument block is built once per decode batch.
  finish   insert prompt + generated tokens, unlock.

With a host tier (host_slots > 0; hustzhy SGLang post, §6.1, HiCache's host-memory
level) eviction demotes KV to a pinned host buffer instead of dropping it; an extend
batch first promotes its requests' host-resident prefixes back to the pool
(rax_promote_batch), and every demotion and promotion runs as a copy kernel on the
stream before the pool slots they free are written (rax_run_moves; the decode append
runs its own).

A match that covers the whole prompt is cut by one token so the request has a
query to run. Consecutive requests' common slot prefix (the depth of the lowest
common ancestor of their tree nodes, rax_lca_depths) is passed to the kernels as
`shared_len`, so K/V tiles they share are loaded once for all of them.

All arithmetic runs in librax (host tree in C++, attention and data movement in
HIP kernels). This module sequences the calls, keeps a host mirror of the
req_to_token table, and moves each call's int32 metadata to the device in one
pinned copy.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from operator import itemgetter

import numpy as np
import torch

from . import _lib as L


def _take(d: dict, keys) -> list:
    """[d[k] for k in keys], looked up in C (itemgetter): the per-request tables are read
    for whole batches of up to 256 requests on every batch change."""
    if not keys:
        return []
    got = itemgetter(*keys)(d)
    return list(got) if len(keys) > 1 else [got]


@dataclass
class ExtendBatch:
    rids: list
    prefix_len: np.ndarray        # m per request (after the full-match cut)
    q_len: np.ndarray
    qo_indptr: np.ndarray
    total_q: int
    tokens: np.ndarray = None     # prompts, flat
    tok_indptr: np.ndarray = None
    max_kv_len: int = 0           # the most keys a query row sees (the longest prompt)
    dev: dict = field(default_factory=dict)
    rtt_total: int = 0            # req_to_token entries of the batch's rows (run_extend writes them)


@dataclass
class DecodeBatch:
    rids: list
    seq_len: np.ndarray
    max_seq_len: int
    dev: dict = field(default_factory=dict)
    key: tuple = None
    shared_len_host: np.ndarray = None  # host copy of dev["shared_len"]


@dataclass
class _DecodeState:
    """The running decode batch while its composition is unchanged."""
    key: tuple                    # request ids, in batch order
    req_rows: np.ndarray          # their req_to_token rows
    inv: dict                     # device int32 views: req_pool_idx, shared_len, seq_len
    lens: np.ndarray              # host lengths (slots in each row), updated by every step
    prep: tuple                   # rax_decode_step argument block (Tree.decode_step_prepare)
    max_len: int = 0              # lens.max(), kept in step with lens
    pos: dict = None              # request id -> its index in the batch (built on first use)
    hints: np.ndarray = None      # host copy of inv["shared_len"]


class RadixRuntime:
    def __init__(self, num_slots: int, h_q: int, h_kv: int, d: int, dtype: torch.dtype,
                 max_reqs: int, max_ctx: int, device: str = "cuda", log: list | None = None,
                 host_slots: int = 0):
        self.tree = L.Tree(num_slots)
        self.num_slots = num_slots
        self.h_q, self.h_kv, self.d, self.dtype = h_q, h_kv, d, dtype
        self.device = torch.device(device)
        self.k_pool = torch.zeros((num_slots, h_kv, d), dtype=dtype, device=self.device)
        self.v_pool = torch.zeros((num_slots, h_kv, d), dtype=dtype, device=self.device)
        self.host_slots = int(host_slots)
        self.k_host = self.v_host = None
        if self.host_slots:
            self.k_host = torch.zeros((self.host_slots, h_kv, d), dtype=dtype, pin_memory=True)
            self.v_host = torch.zeros((self.host_slots, h_kv, d), dtype=dtype, pin_memory=True)
            self.tree.set_host_tier(self.host_slots, self.k_host, self.v_host)
        self.rtt = torch.zeros((max_reqs, max_ctx), dtype=torch.int32, device=self.device)
        self._seq_dev = torch.zeros(max_reqs, dtype=torch.int32, device=self.device)  # decode lengths on the device
        self.rows = np.zeros((max_reqs, max_ctx), dtype=np.int32)   # host mirror of rtt
        self.max_ctx = max_ctx
        self.free_rows = list(range(max_reqs - 1, -1, -1))
        self.row_of: dict[int, int] = {}
        self.len_of: dict[int, int] = {}     # current sequence length (slots in the row)
        self.n_prompt: dict[int, int] = {}
        self.node_of: dict[int, int] = {}    # locked tree node
        self.node_by_row = np.zeros(max_reqs, dtype=np.int64)  # the same, by req_to_token row
        self.trusted_of: dict[int, int] = {}  # row positions before it hold the tree's slots
        self.log = log
        self.step = 0                        # label of the current step in the event log (set by the caller)
        self.timers = None                   # {"extend": [...], "decode": [...]} of (start, end) events, if set
        self.pre_attention = None            # called right before each attention call is issued, if set
        self._ws = torch.empty(0, dtype=torch.uint8, device=self.device)
        self._dec_cache = None               # _DecodeState while the decode batch is unchanged

    # ------------------------------------------------------------------ helpers
    def _upload(self, parts: dict) -> dict:
        """One pinned host buffer -> one device copy; returns named int32 device views."""
        names = list(parts)
        arrs = [np.asarray(parts[k], dtype=np.int32).reshape(-1) for k in names]
        sizes = [a.size for a in arrs]
        total = sum(sizes)
        host = torch.empty(max(total, 1), dtype=torch.int32, pin_memory=True)
        if total:
            np.concatenate(arrs, out=host.numpy()[:total])
        dev = host.to(self.device, non_blocking=True)
        return dict(zip(names, torch.split(dev[:total], sizes)))

    def _workspace(self, nbytes: int):
        if nbytes == 0:
            return None
        if self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self._ws

    def _event_pair(self, kind):
        """When timing is on: record a start event now on the current stream, return (start, end)."""
        if self.timers is None:
            return None
        pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        pair[0].record()
        self.timers.setdefault(kind, []).append(pair)
        return pair

    def _log(self, *ev):
        if self.log is not None:
            self.log.append(ev)

    def seq_len(self, rid: int) -> int:
        """Current number of slots in the request's row."""
        ds = self._dec_cache
        if ds is not None:
            if ds.pos is None:
                ds.pos = dict(zip(ds.key, range(len(ds.key))))
            i = ds.pos.get(rid)
            if i is not None:
                return int(ds.lens[i])
        return self.len_of[rid]

    def slot_row(self, rid: int) -> np.ndarray:
        return self.rows[self.row_of[rid], : self.seq_len(rid)].copy()

    # ------------------------------------------------------------------- extend
    def begin_extend(self, batch) -> ExtendBatch:
        """batch: list of (rid, prompt int32 array). Tree side + req_to_token fill."""
        rids = [rid for rid, _ in batch]
        prompts = [np.asarray(p, dtype=np.int32) for _, p in batch]
        n = np.array([len(p) for p in prompts], dtype=np.int64)
        if len(n) and int(n.max()) > self.max_ctx:
            raise ValueError("prompt longer than the req_to_token rows")
        ip = np.zeros(len(rids) + 1, dtype=np.int64)
        ip[1:] = np.cumsum(n)
        toks = np.concatenate(prompts) if prompts else np.zeros(0, np.int32)
        if self.host_slots:
            done, pfreed = self.tree.promote_batch(toks, ip)
            self._log("promote", self.step, tuple(done.tolist()), tuple(pfreed.tolist()))
        pslots, m, nodes = self.tree.match_prefix_batch(toks, ip, cut_full=True, lock=True)
        if self.log is not None:
            for i, rid in enumerate(rids):
                self._log("match", rid, int(m[i]), int(nodes[i]))
        q_len = (n - m).astype(np.int32)
        new, freed = self.tree.alloc_slots_evict(int(q_len.sum()))
        if self.log is not None:
            if len(freed):
                self._log("evict", self.step, tuple(freed.tolist()))
            self._log("alloc", self.step, tuple(new.tolist()))
        # slot of every prompt position: the tree's for the matched prefix (already in
        # pslots), a new one after it; plain lists in the per-request loop (numpy scalar
        # indexing costs more than the row copies)
        src = pslots
        off = 0
        req_rows = [0] * len(rids)
        ipl, ml, ql, nl = ip.tolist(), m.tolist(), q_len.tolist(), nodes.tolist()
        for i, rid in enumerate(rids):
            row = self.free_rows.pop()
            a, b, mi, qi = ipl[i], ipl[i + 1], ml[i], ql[i]
            if qi:
                src[a + mi: b] = new[off: off + qi]
                off += qi
            self.rows[row, : b - a] = src[a: b]
            self.row_of[rid] = row
            self.len_of[rid] = b - a
            self.n_prompt[rid] = b - a
            self.node_of[rid] = nl[i]
            self.trusted_of[rid] = mi
            req_rows[i] = row
        req_rows = np.array(req_rows, dtype=np.int32)
        self.node_by_row[req_rows] = nodes
        qo = np.zeros(len(rids) + 1, dtype=np.int32)
        qo[1:] = np.cumsum(q_len)
        eb = ExtendBatch(rids, m.astype(np.int32), q_len, qo, int(qo[-1]), toks, ip,
                         max_kv_len=int(n.max()) if len(n) else 0)
        eb.dev = self._upload(dict(
            req_pool_idx=req_rows, prefix_len=eb.prefix_len, qo_indptr=qo,
            shared_len=self.tree.lca_depths(nodes), out_loc=new, rtt_start=np.zeros(len(rids)),
            rtt_indptr=ip, rtt_src=src))
        # the rows are filled by run_extend's launch, together with the K/V write-back
        eb.rtt_total = int(ip[-1])
        if self.host_slots:
            self.tree.run_moves(self.k_pool, self.v_pool)   # before the scatter writes the freed slots
        self._sync_decode_lengths()
        self._dec_cache = None
        return eb

    def run_extend(self, eb: ExtendBatch, q, k_ext, v_ext, o) -> None:
        """Write the suffix K/V into the pool and run extend attention (q/k/v/o on the device)."""
        if eb.total_q == 0:
            L.req_to_token_write(self.rtt, eb.dev["req_pool_idx"], eb.dev["rtt_start"], eb.dev["rtt_indptr"],
                                 eb.dev["rtt_src"], eb.rtt_total)
            return
        # the requests' req_to_token rows and the suffix K/V rows in one launch
        L.extend_write(self.rtt, eb.dev["req_pool_idx"], eb.dev["rtt_start"], eb.dev["rtt_indptr"], eb.dev["rtt_src"],
                       eb.rtt_total, k_ext, v_ext, eb.dev["out_loc"], self.k_pool, self.v_pool)
        if self.pre_attention is not None:
            self.pre_attention()
        ws = self._workspace(L.attention_workspace_bytes(False, eb.total_q, self.h_q, self.h_kv, self.d,
                                                         eb.max_kv_len))
        ev = self._event_pair("extend")
        L.extend_attention(q, k_ext, v_ext, self.k_pool, self.v_pool, self.rtt, eb.dev["req_pool_idx"],
                           eb.dev["prefix_len"], eb.dev["qo_indptr"], o, shared_len=eb.dev["shared_len"],
                           workspace=ws, max_kv_len=eb.max_kv_len)
        if ev:
            ev[1].record()

    def end_extend(self, eb: ExtendBatch, prompts=None) -> None:
        """Insert every prompt; requests switch to the tree's copy of any duplicate slots."""
        rids, ip = eb.rids, eb.tok_indptr
        rows = _take(self.row_of, rids)
        n_prompt = _take(self.n_prompt, rids)
        slots = np.concatenate([self.rows[row, :n] for row, n in zip(rows, n_prompt)]) \
            if rids else np.zeros(0, np.int32)
        # each walk starts where the request's prefix matched (its locked node): the
        # matched slots are the tree's already
        old = _take(self.node_of, rids)
        tslots, existing, nodes = self.tree.insert_batch_from(old, _take(self.trusted_of, rids), eb.tokens, slots, ip)
        if self.log is not None:
            for i, rid in enumerate(rids):
                self._log("insert", rid, int(existing[i]), int(nodes[i]))
        diff = np.nonzero(tslots != slots)[0]
        if len(diff):
            req_i = np.searchsorted(ip, diff, side="right") - 1
            pos = diff - ip[req_i]
            fix_rows = np.array(rows, dtype=np.int32)[req_i]
            self.rows[fix_rows, pos] = tslots[diff]
            k = len(diff)
            dv = self._upload(dict(rows=fix_rows, start=pos, indptr=np.arange(k + 1), src=tslots[diff]))
            L.req_to_token_write(self.rtt, dv["rows"], dv["start"], dv["indptr"], dv["src"], k)
        self.tree.lock_ref_batch(nodes, +1)
        self.tree.lock_ref_batch(old, -1)
        self.node_of.update(zip(rids, nodes.tolist()))
        self.node_by_row[np.asarray(rows, dtype=np.int64)] = nodes
        self.trusted_of.update(zip(rids, n_prompt))   # duplicates switched to the tree's above
        self._sync_decode_lengths()
        self._dec_cache = None

    # ------------------------------------------------------------------- decode
    def _sync_decode_lengths(self):
        """Write the decode batch's cached lengths back to the per-request table."""
        if self._dec_cache is not None:
            self.len_of.update(zip(self._dec_cache.key, self._dec_cache.lens.tolist()))

    def begin_decode(self, rids) -> DecodeBatch:
        """Describe the next decode step of `rids` (one new token each): db.seq_len holds the
        lengths after the step, so token i of the batch sits at position db.seq_len[i] - 1.
        Nothing changes until run_decode."""
        key = tuple(rids)
        ds = self._dec_cache
        if ds is None or ds.key != key:
            self._sync_decode_lengths()
            req_rows = np.array(_take(self.row_of, rids), dtype=np.int32)
            hints = self.tree.lca_depths(self.node_by_row[req_rows])
            inv = self._upload(dict(req_pool_idx=req_rows, shared_len=hints))
            inv["seq_len"] = self._seq_dev[: len(rids)]   # written by every step's append
            lens = np.array(_take(self.len_of, rids), dtype=np.int32)
            prep = self.tree.decode_step_prepare(lens, self.rtt, inv["req_pool_idx"], inv["seq_len"], self.k_pool,
                                                 self.v_pool, self.h_q, shared_len=inv["shared_len"],
                                                 shared_len_host=hints)
            ds = self._dec_cache = _DecodeState(key, req_rows, inv, lens, prep, int(lens.max()) if len(lens) else 0,
                                                None, hints)
        seq_len = ds.lens + 1
        max_seq = ds.max_len + 1 if len(seq_len) else 0
        if max_seq > self.max_ctx:
            raise ValueError("sequence longer than the req_to_token rows")
        db = DecodeBatch(list(rids), seq_len, max_seq, ds.inv, ds.key, ds.hints)
        return db

    def run_decode(self, db: DecodeBatch, q, k_new, v_new, o) -> None:
        """One decode step in one native call (rax_decode_step): allocate the new tokens'
        slots, append them to the rows, write their K/V into the pools, run decode attention."""
        ds = self._dec_cache
        if ds is None or db.key is not ds.key:
            raise ValueError("run_decode: batch differs from the last begin_decode")
        if self.pre_attention is not None:
            self.pre_attention()
        ev = self._event_pair("decode")
        new, freed, need = self.tree.decode_step(ds.prep, q, k_new, v_new, o, self._ws)
        if new is None:                      # workspace too small: nothing was done
            new, freed, need = self.tree.decode_step(ds.prep, q, k_new, v_new, o, self._workspace(need))
        if ev:
            ev[1].record()
        if self.log is not None:
            if len(freed):
                self._log("evict", self.step, tuple(freed.tolist()))
            self._log("alloc", self.step, tuple(new.tolist()))
        ds.max_len += 1                      # every request gained one token
        self.rows[ds.req_rows, ds.lens - 1] = new

    # ------------------------------------------------------------------- finish
    def finish(self, rid: int, tokens) -> np.ndarray:
        """Insert prompt + generated tokens of one request, unlock; returns the tree's slots."""
        return self.finish_batch([(rid, tokens)])[0]

    def finish_batch(self, items) -> list:
        """items: list of (rid, tokens). Insert each, unlock each; returns the tree's slot rows."""
        if not items:
            return []
        self._sync_decode_lengths()
        rids = [rid for rid, _ in items]
        toks = [np.asarray(t, dtype=np.int32) for _, t in items]
        for rid, t in zip(rids, toks):
            if len(t) != self.len_of[rid]:
                raise ValueError("finish: tokens and slot row differ in length")
        ip = np.zeros(len(rids) + 1, dtype=np.int64)
        ip[1:] = np.cumsum([len(t) for t in toks])
        rows, lens, locked = _take(self.row_of, rids), _take(self.len_of, rids), _take(self.node_of, rids)
        slots = np.concatenate([self.rows[row, :n] for row, n in zip(rows, lens)])
        # from each request's locked node (its prompt's; the row holds the tree's slots up
        # to its trusted length)
        tslots, existing, nodes = self.tree.insert_batch_from(locked, _take(self.trusted_of, rids),
                                                              np.concatenate(toks), slots, ip)
        if self.log is not None:
            for i, rid in enumerate(rids):
                self._log("insert", rid, int(existing[i]), int(nodes[i]))
        self.tree.lock_ref_batch(locked, -1)
        out = []
        for i, rid in enumerate(rids):
            self.free_rows.append(self.row_of.pop(rid))
            del self.len_of[rid], self.n_prompt[rid], self.node_of[rid], self.trusted_of[rid]
            out.append(tslots[ip[i]: ip[i + 1]])
        self._dec_cache = None
        return out

    @property
    def reqs(self):
        """Running request ids (those holding a req_to_token row)."""
        return self.row_of
