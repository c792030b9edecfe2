"""Request lifecycle over librax: the host side of RadixAttention's hot path.

Per batch (2312.07104_SGLang notes, App. A.2: match every request, form the batch
evicting when memory is short, run it, update the tree; hustzhy SGLang post,
§2.3 (2): traverse -> reuse -> compute -> insert):

  extend   match each prompt in the tree (rax_match_prefix) and lock the matched
           node; allocate slots for all unmatched suffixes at once
           (rax_alloc_slots_evict); fill the requests' req_to_token rows on the
           device; write the new tokens' K/V into the pool (rax_kv_scatter); run
           extend attention over reused prefix + causal suffix; then insert each
           prompt (rax_insert) and move the lock to the new node.
  decode   allocate one slot per request, append it to the row, write the new
           token's K/V, run decode attention over the whole row.
  finish   insert prompt + generated tokens, unlock.

A match that covers the whole prompt is cut by one token so the request has a
query to run. Consecutive requests' common slot prefix (the depth of the lowest
common ancestor of their tree nodes, rax_lca_depth) is passed to the kernels as
`shared_len`, so K/V tiles they share are loaded once for all of them.

All arithmetic runs in librax (host tree in C++, attention and data movement in
HIP kernels). This module only sequences the calls and moves int32 metadata to
the device in one pinned copy per call.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import _lib as L


@dataclass
class ReqState:
    rid: int
    row: int                      # req_to_token row
    n_prompt: int
    slots: list                   # host copy of the request's slot row
    node: int                     # locked tree node


@dataclass
class ExtendBatch:
    rids: list
    prefix_len: np.ndarray        # m per request (after the full-match cut)
    q_len: np.ndarray
    qo_indptr: np.ndarray
    total_q: int
    dev: dict = field(default_factory=dict)


@dataclass
class DecodeBatch:
    rids: list
    seq_len: np.ndarray
    max_seq_len: int
    dev: dict = field(default_factory=dict)


class RadixRuntime:
    def __init__(self, num_slots: int, h_q: int, h_kv: int, d: int, dtype: torch.dtype,
                 max_reqs: int, max_ctx: int, device: str = "cuda", log: list | None = None):
        self.tree = L.Tree(num_slots)
        self.num_slots = num_slots
        self.h_q, self.h_kv, self.d, self.dtype = h_q, h_kv, d, dtype
        self.device = torch.device(device)
        self.k_pool = torch.zeros((num_slots, h_kv, d), dtype=dtype, device=self.device)
        self.v_pool = torch.zeros((num_slots, h_kv, d), dtype=dtype, device=self.device)
        self.rtt = torch.zeros((max_reqs, max_ctx), dtype=torch.int32, device=self.device)
        self.max_ctx = max_ctx
        self.free_rows = list(range(max_reqs - 1, -1, -1))
        self.reqs: dict[int, ReqState] = {}
        self.log = log
        self.step = 0                 # label of the current step in the event log (set by the caller)
        self.timers = None            # {"extend": [...], "decode": [...]} of (start, end) events, if set
        self._ws = torch.empty(0, dtype=torch.uint8, device=self.device)

    # ------------------------------------------------------------------ helpers
    def _upload(self, parts: dict) -> dict:
        """One pinned host buffer -> one device copy; returns named int32 device views."""
        names = list(parts)
        arrs = [np.ascontiguousarray(parts[k], dtype=np.int32).ravel() for k in names]
        total = sum(a.size for a in arrs)
        host = torch.empty(max(total, 1), dtype=torch.int32, pin_memory=True)
        hv = host.numpy()
        off = 0
        spans = {}
        for k, a in zip(names, arrs):
            hv[off: off + a.size] = a
            spans[k] = (off, a.size)
            off += a.size
        dev = host.to(self.device, non_blocking=True)
        return {k: dev[o: o + n] for k, (o, n) in spans.items()}

    def _workspace(self, nbytes: int):
        if nbytes == 0:
            return None
        if self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self._ws

    def _shared_len(self, rids) -> np.ndarray:
        out = np.zeros(len(rids), dtype=np.int32)
        for i in range(1, len(rids)):
            out[i] = self.tree.lca_depth(self.reqs[rids[i - 1]].node, self.reqs[rids[i]].node)
        return out

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

    # ------------------------------------------------------------------- extend
    def begin_extend(self, batch) -> ExtendBatch:
        """batch: list of (rid, prompt int32 array). Tree side + req_to_token fill."""
        rids, m_list, pre = [], [], []
        for rid, prompt in batch:
            prompt = np.asarray(prompt, dtype=np.int32)
            m, pslots, node = self.tree.match_prefix(prompt)
            if m == len(prompt):
                m -= 1
                pslots = pslots[:m]
            self._log("match", rid, m, node)
            self.tree.lock_ref(node, +1)
            if len(prompt) > self.max_ctx:
                raise ValueError("prompt longer than the req_to_token rows")
            self.reqs[rid] = ReqState(rid, self.free_rows.pop(), len(prompt), [], node)
            rids.append(rid)
            m_list.append(m)
            pre.append(pslots)
        n_list = [self.reqs[r].n_prompt for r in rids]
        q_len = np.array([n - m for n, m in zip(n_list, m_list)], dtype=np.int32)
        new, freed = self.tree.alloc_slots_evict(int(q_len.sum()))
        if len(freed):
            self._log("evict", self.step, tuple(freed.tolist()))
        self._log("alloc", self.step, tuple(new.tolist()))
        rows_src, off = [], 0
        for i, rid in enumerate(rids):
            st = self.reqs[rid]
            own = new[off: off + q_len[i]]
            off += q_len[i]
            st.slots = pre[i].tolist() + own.tolist()
            rows_src.append(np.concatenate([pre[i], own]))
        qo = np.zeros(len(rids) + 1, dtype=np.int32)
        qo[1:] = np.cumsum(q_len)
        src_indptr = np.zeros(len(rids) + 1, dtype=np.int32)
        src_indptr[1:] = np.cumsum(n_list)
        eb = ExtendBatch(rids, np.array(m_list, dtype=np.int32), q_len, qo, int(qo[-1]))
        eb.dev = self._upload(dict(
            req_pool_idx=[self.reqs[r].row for r in rids], prefix_len=eb.prefix_len, qo_indptr=qo,
            shared_len=self._shared_len(rids), out_loc=new, rtt_start=np.zeros(len(rids)),
            rtt_indptr=src_indptr, rtt_src=np.concatenate(rows_src) if rows_src else np.zeros(0)))
        L.req_to_token_write(self.rtt, eb.dev["req_pool_idx"], eb.dev["rtt_start"], eb.dev["rtt_indptr"],
                             eb.dev["rtt_src"], int(src_indptr[-1]))
        return eb

    def run_extend(self, eb: ExtendBatch, q, k_ext, v_ext, o) -> None:
        """Write the suffix K/V into the pool and run extend attention (q/k/v/o on the device)."""
        if eb.total_q == 0:
            return
        L.kv_scatter(k_ext, v_ext, eb.dev["out_loc"], self.k_pool, self.v_pool)
        ev = self._event_pair("extend")
        L.extend_attention(q, k_ext, v_ext, self.k_pool, self.v_pool, self.rtt, eb.dev["req_pool_idx"],
                           eb.dev["prefix_len"], eb.dev["qo_indptr"], o, shared_len=eb.dev["shared_len"])
        if ev:
            ev[1].record()

    def end_extend(self, eb: ExtendBatch, prompts: dict) -> None:
        """Insert every prompt; requests switch to the tree's copy of any duplicate slots."""
        fix_rows, fix_pos, fix_val = [], [], []
        for rid in eb.rids:
            st = self.reqs[rid]
            prompt = np.asarray(prompts[rid], dtype=np.int32)
            existing, node, tslots = self.tree.insert(prompt, np.asarray(st.slots[: st.n_prompt], np.int32))
            self._log("insert", rid, existing, node)
            ts = tslots.tolist()
            if ts != st.slots[: st.n_prompt]:
                for p in range(st.n_prompt):
                    if ts[p] != st.slots[p]:
                        fix_rows.append(st.row)
                        fix_pos.append(p)
                        fix_val.append(ts[p])
                st.slots[: st.n_prompt] = ts
            self.tree.lock_ref(node, +1)
            self.tree.lock_ref(st.node, -1)
            st.node = node
        if fix_val:
            k = len(fix_val)
            dv = self._upload(dict(rows=fix_rows, start=fix_pos, indptr=np.arange(k + 1), src=fix_val))
            L.req_to_token_write(self.rtt, dv["rows"], dv["start"], dv["indptr"], dv["src"], k)

    # ------------------------------------------------------------------- decode
    def begin_decode(self, rids) -> DecodeBatch:
        new, freed = self.tree.alloc_slots_evict(len(rids))
        if len(freed):
            self._log("evict", self.step, tuple(freed.tolist()))
        self._log("alloc", self.step, tuple(new.tolist()))
        seq_len = np.empty(len(rids), dtype=np.int32)
        for i, rid in enumerate(rids):
            st = self.reqs[rid]
            st.slots.append(int(new[i]))
            seq_len[i] = len(st.slots)
        if int(seq_len.max()) > self.max_ctx:
            raise ValueError("sequence longer than the req_to_token rows")
        db = DecodeBatch(list(rids), seq_len, int(seq_len.max()))
        db.dev = self._upload(dict(
            req_pool_idx=[self.reqs[r].row for r in rids], seq_len=seq_len, shared_len=self._shared_len(rids),
            out_loc=new, rtt_start=seq_len - 1, rtt_indptr=np.arange(len(rids) + 1)))
        L.req_to_token_write(self.rtt, db.dev["req_pool_idx"], db.dev["rtt_start"], db.dev["rtt_indptr"],
                             db.dev["out_loc"], len(rids))
        return db

    def run_decode(self, db: DecodeBatch, q, k_new, v_new, o) -> None:
        L.kv_scatter(k_new, v_new, db.dev["out_loc"], self.k_pool, self.v_pool)
        ws = self._workspace(L.attention_workspace_bytes(True, len(db.rids), self.h_q, self.h_kv, self.d,
                                                         db.max_seq_len))
        ev = self._event_pair("decode")
        L.decode_attention(q, self.k_pool, self.v_pool, self.rtt, db.dev["req_pool_idx"], db.dev["seq_len"],
                           db.max_seq_len, o, workspace=ws, shared_len=db.dev["shared_len"])
        if ev:
            ev[1].record()

    # ------------------------------------------------------------------- finish
    def finish(self, rid: int, tokens) -> list:
        """Insert prompt + generated tokens, unlock; returns the tree's slots for them."""
        st = self.reqs.pop(rid)
        toks = np.asarray(tokens, dtype=np.int32)
        if len(toks) != len(st.slots):
            raise ValueError("finish: tokens and slot row differ in length")
        existing, node, tslots = self.tree.insert(toks, np.asarray(st.slots, dtype=np.int32))
        self._log("insert", rid, existing, node)
        self.tree.lock_ref(st.node, -1)
        self.free_rows.append(st.row)
        return tslots.tolist()

    def slot_row(self, rid: int) -> list:
        return list(self.reqs[rid].slots)
