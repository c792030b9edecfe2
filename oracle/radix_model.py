"""Plain model of the radix-tree KV cache: segments over a per-token trie.

TEST INFRASTRUCTURE (oracle). Only tests/, the smoke check and the bench's CPU
baseline leg may use this module. It shares no code with the C++ tree.

What the pages fix (cited by page title and section):
  * Tree of token sequences whose edges carry variable-length labels, the KV of
    every token kept in one token-granular pool (2312.07104_SGLang notes, §3
    "RadixAttention core idea"; hustzhy SGLang post, §2.2-2.3).
  * Match = longest cached prefix; insert merges a finished request into the tree
    as new edges / leaves; a node shared only up to a divergence point is split
    in two (bowenzhou SGLang review, "Work loop: insert, match, split, evict";
    Figure 3 steps 4 and 7 as narrated in the notes and in the unite.ai article).
  * Ref counts: a node is pinned while running requests depend on it; only at
    count 0 may it be freed (notes §3; bowenzhou review, same section).
  * Eviction is LRU over leaves; ancestors survive until they become leaves
    themselves (notes §3; hustzhy post §2.3 (3); bowenzhou review).
  * Cached and running KV share one pool (notes §3; papers.lqhl.me review,
    "Core method").

Readings where the pages are silent (each a choice; the C++ tree follows the
same rules so results compare bit for bit):
  R4  A match that ends inside a node splits that node at once; the upper part is
      a new node (new id, same ref count, same tick), the lower part keeps its id.
  R5  A logical clock advances by one on every match or insert call; every node on
      the matched/inserted path (after any split) takes the new tick. Ties between
      evictable leaves break by the smaller node id.
  R6  Eviction removes whole leaves with ref 0, least recent first, until at least
      the requested number of tokens is freed or nothing is evictable. Freed slots
      are reported leaf by leaf, each leaf's tokens in sequence order.
  R7  Insert over an already cached position keeps the tree's slot; the caller's
      slot there, if different, goes back to the free set.
  R8  The allocator hands out the lowest free slot ids first, in ascending order;
      a request it cannot satisfy takes nothing.
Node ids: root is 0; every new node takes the next integer.

Host-memory tier (hustzhy SGLang post, §6.1, HiCache: GPU memory keeps the hottest KV,
host memory the next level; the pages give no mechanics, so every rule below is a
reading):
  H1  With a tier of host_slots rows, eviction demotes instead of dropping: the LRU
      candidate is a device node with ref 0 and no device child; its tokens take the
      lowest free host slots, one move (0, device slot, host slot) each in token
      order, and the node stays in the tree as a host node. If the tier is short,
      host nodes with no children and ref 0 are dropped first, least recent first
      (tie: smaller id); if it is still short, the node and all its (host)
      descendants are dropped and only its own device slots are reported freed.
  H2  Host nodes only have host descendants. Match and the cached-prefix length
      walk device nodes only; a host node cannot be locked (ESTATE).
  H3  Promotion of a request: walk its device prefix; if that ends inside a device
      node there is nothing to do. Otherwise follow its tokens through host nodes
      one node at a time: split where they diverge inside a node, make room on the
      device by eviction (H1) for the node's tokens while that node and the device
      path above it are pinned, take the lowest free device slots (stop if short),
      record one move (1, host slot, device slot) per token and free the host slots.
  H4  Insert adopts host nodes on its path: the caller's slots become the node's
      device slots, its host slots are freed, nothing moves. Only the device-cached
      prefix counts as "existing" (its duplicate caller slots are returned).
  H5  Moves are kept in decision order; running them in that order reproduces the
      data even where a slot freed by one move is taken by a later one.

Representation: one trie vertex per cached token (token, slot, segment id);
a segment (= radix node) is a maximal run of trie vertices between branch points
as created by inserts and splits. Every query is answered by walking the trie;
eviction candidates are found by scanning all segments.
"""
from __future__ import annotations

import heapq


class CacheError(Exception):
    """Raised for states the C-ABI reports as an error code."""

    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


class _Vertex:
    __slots__ = ("tok", "slot", "parent", "children", "seg", "depth")

    def __init__(self, tok, slot, parent, seg, depth):
        self.tok = tok
        self.slot = slot
        self.parent = parent
        self.children = {}
        self.seg = seg
        self.depth = depth          # number of tokens from the root up to and including this one


class _Segment:
    __slots__ = ("id", "top", "bottom", "ref", "tick", "parent", "host")

    def __init__(self, sid, top, bottom, ref, tick, parent, host=False):
        self.id = sid
        self.top = top              # first vertex (None for root)
        self.bottom = bottom        # last vertex  (None for root)
        self.ref = ref
        self.tick = tick
        self.parent = parent        # parent segment id (-1 for root)
        self.host = host            # KV in the host tier (vertex slots are host slot ids)


class RadixCacheModel:
    def __init__(self, num_slots: int, host_slots: int = 0):
        self.num_slots = int(num_slots)
        self.host_slots = int(host_slots)
        self.hfree = list(range(self.host_slots))          # lowest first, like the device pool
        heapq.heapify(self.hfree)
        self.moves = []                                     # (kind, src, dst) in decision order (H5)
        self.root_v = _Vertex(None, None, None, 0, 0)
        self.segs = {0: _Segment(0, None, None, 0, 0, -1)}
        self.next_id = 1
        self.clock = 0
        self.free = list(range(self.num_slots))
        heapq.heapify(self.free)
        self.free_set = set(self.free)

    # ------------------------------------------------------------ allocator (R8)
    def alloc(self, n: int) -> list:
        if n > len(self.free):
            raise CacheError("ENOMEM", f"need {n}, free {len(self.free)}")
        out = [heapq.heappop(self.free) for _ in range(n)]
        for s in out:
            self.free_set.discard(s)
        return out

    def free_slots(self, slots) -> None:
        slots = [int(s) for s in slots]
        for s in slots:
            if s < 0 or s >= self.num_slots or s in self.free_set:
                raise CacheError("EINVAL", f"bad free of slot {s}")
        for s in slots:
            heapq.heappush(self.free, s)
            self.free_set.add(s)

    def num_free(self) -> int:
        return len(self.free)

    # ------------------------------------------------------------------ helpers
    def _seg_len(self, s: _Segment) -> int:
        return 0 if s.top is None else s.bottom.depth - s.top.depth + 1

    def _seg_vertices(self, s: _Segment) -> list:
        out = []
        v = s.bottom
        while v is not None and v.depth >= s.top.depth:
            out.append(v)
            v = v.parent
        out.reverse()
        return out

    def _is_leaf(self, s: _Segment) -> bool:
        return s.id != 0 and len(s.bottom.children) == 0

    def _path_segments(self, sid: int) -> list:
        out = []
        while sid != -1:
            out.append(sid)
            sid = self.segs[sid].parent
        return out

    def _split(self, v: _Vertex) -> int:
        """Make ``v`` the bottom of its segment (R4); return the upper segment's id."""
        s = self.segs[v.seg]
        if s.bottom is v:
            return s.id
        up = _Segment(self.next_id, s.top, v, s.ref, s.tick, s.parent, s.host)
        self.next_id += 1
        self.segs[up.id] = up
        u = v
        while u is not None and u.depth >= s.top.depth:
            u.seg = up.id
            u = u.parent
        # the lower part keeps s's id; it now starts below v
        below = [c for c in v.children.values()]
        assert len(below) == 1
        s.top = below[0]
        s.parent = up.id
        return up.id

    def _walk(self, tokens) -> tuple:
        """Device-cached prefix (H2): (last vertex, slots)."""
        v = self.root_v
        slots = []
        for t in tokens:
            c = v.children.get(int(t))
            if c is None or self.segs[c.seg].host:
                break
            v = c
            slots.append(v.slot)
        return v, slots

    def _tick_path(self, sid: int) -> None:
        for p in self._path_segments(sid):
            if p != 0:
                self.segs[p].tick = self.clock

    # --------------------------------------------------------------- operations
    def match(self, tokens) -> tuple:
        """Longest cached prefix: (m, slots[m], node id). Splits and ticks (R4, R5)."""
        self.clock += 1
        v, slots = self._walk(tokens)
        node = 0 if v is self.root_v else self._split(v)
        self._tick_path(node)
        return len(slots), slots, node

    def insert(self, tokens, slots) -> tuple:
        """Cache tokens with their slots: (existing, node id, tree slots). R4, R5, R7."""
        tokens = [int(t) for t in tokens]
        slots = [int(s) for s in slots]
        if len(tokens) != len(slots):
            raise CacheError("EINVAL", "length mismatch")
        self.clock += 1
        v, tree_slots = self._walk(tokens)
        m = len(tree_slots)
        node = 0 if v is self.root_v else self._split(v)
        dup = [slots[i] for i in range(m) if slots[i] != tree_slots[i]]
        out_slots = list(tree_slots)
        existing = m
        # H4: host vertices on the path take the caller's slots
        path = []
        while m + len(path) < len(tokens):
            c = (path[-1] if path else v).children.get(tokens[m + len(path)])
            if c is None:
                break
            path.append(c)
        if path:
            node = self._split(path[-1])
            for i, x in enumerate(path):
                self.segs[x.seg].host = False
                heapq.heappush(self.hfree, x.slot)
                x.slot = slots[m + i]
                out_slots.append(x.slot)
            m += len(path)
            v = path[-1]
        if m < len(tokens):
            seg = _Segment(self.next_id, None, None, 0, self.clock, node)
            self.next_id += 1
            self.segs[seg.id] = seg
            parent_v = v
            for i in range(m, len(tokens)):
                nv = _Vertex(tokens[i], slots[i], parent_v, seg.id, parent_v.depth + 1)
                parent_v.children[tokens[i]] = nv
                if seg.top is None:
                    seg.top = nv
                parent_v = nv
                out_slots.append(slots[i])
            seg.bottom = parent_v
            node = seg.id
        self._tick_path(node)
        if dup:
            self.free_slots(dup)
        return existing, node, out_slots

    def lock_ref(self, node: int, delta: int) -> None:
        if delta not in (1, -1):
            raise CacheError("EINVAL", f"bad delta {delta}")
        if node not in self.segs:
            raise CacheError("ESTATE", f"unknown node {node}")
        if self.segs[node].host:
            raise CacheError("ESTATE", "host nodes cannot be pinned (H2)")
        path = [p for p in self._path_segments(node) if p != 0]
        if delta < 0 and any(self.segs[p].ref + delta < 0 for p in path):
            raise CacheError("ESTATE", "unlock below zero")
        for p in path:
            self.segs[p].ref += delta

    def _children(self, sid: int) -> list:
        """Child segments: those whose first vertex hangs below this segment's last one."""
        s = self.segs[sid]
        below = self.root_v if s.top is None else s.bottom
        return [self.segs[c.seg] for c in below.children.values()]

    def _remove_subtree(self, s: _Segment) -> None:
        """Unlink segment s and everything below it; host slots go back to the tier."""
        del s.top.parent.children[s.top.tok]
        stack = [s]
        while stack:
            x = stack.pop()
            stack.extend(self._children(x.id))
            if x.host:
                for v in self._seg_vertices(x):
                    heapq.heappush(self.hfree, v.slot)
            del self.segs[x.id]

    def _drop_host_leaves(self, need: int) -> None:
        while len(self.hfree) < need:
            cands = [s for s in self.segs.values() if s.host and s.ref == 0 and not self._children(s.id)]
            if not cands:
                return
            self._remove_subtree(min(cands, key=lambda x: (x.tick, x.id)))

    def evict(self, num_tokens: int) -> list:
        """Free >= num_tokens device slots, LRU device leaves first (R6); with a host tier
        the leaf is demoted rather than dropped (H1)."""
        freed = []
        while len(freed) < num_tokens:
            cands = [s for s in self.segs.values()
                     if s.id != 0 and not s.host and s.ref == 0
                     and all(c.host for c in self._children(s.id))]
            if not cands:
                break
            s = min(cands, key=lambda x: (x.tick, x.id))
            verts = self._seg_vertices(s)
            freed.extend(x.slot for x in verts)
            if self.host_slots > 0:
                self._drop_host_leaves(len(verts))
            if self.host_slots > 0 and len(self.hfree) >= len(verts):
                for x in verts:
                    h = heapq.heappop(self.hfree)
                    self.moves.append((0, x.slot, h))
                    x.slot = h
                s.host = True
            else:
                self._remove_subtree(s)
        if freed:
            self.free_slots(freed)
        return freed

    def promote(self, tokens) -> tuple:
        """H3: bring the host continuation of the request's device prefix back to the
        device. Returns (tokens promoted, device slots freed by evictions)."""
        tokens = [int(t) for t in tokens]
        v, slots = self._walk(tokens)
        i = len(slots)
        freed = []
        if v is not self.root_v and self.segs[v.seg].bottom is not v:
            return 0, freed                         # ends or diverges inside a device node
        locked = None if v is self.root_v else v.seg
        if locked is not None:
            self.lock_ref(locked, +1)
        done = 0
        while i < len(tokens):
            c = v.children.get(tokens[i])
            if c is None:
                break
            seg = self.segs[c.seg]                  # a host node, entered at its top
            verts = self._seg_vertices(seg)
            k = 1
            while k < len(verts) and i + k < len(tokens) and verts[k].tok == tokens[i + k]:
                k += 1
            u = self.segs[self._split(verts[k - 1])]
            u.ref += 1                              # not droppable while making room
            short = k - self.num_free()
            if short > 0:
                freed.extend(self.evict(short))
            u.ref -= 1
            if self.num_free() < k:
                break
            dev = self.alloc(k)
            for x, d in zip(verts[:k], dev):
                self.moves.append((1, x.slot, d))
                heapq.heappush(self.hfree, x.slot)
                x.slot = d
            u.host = False
            self.lock_ref(u.id, +1)
            if locked is not None:
                self.lock_ref(locked, -1)
            locked = u.id
            done += k
            i += k
            v = verts[k - 1]
            if k < len(verts):
                break
        if locked is not None:
            self.lock_ref(locked, -1)
        return done, freed

    def take_moves(self) -> list:
        out, self.moves = self.moves, []
        return out

    def lca_depth(self, a: int, b: int) -> int:
        """Token depth of the deepest node that is an ancestor of (or equal to) both nodes."""
        if a not in self.segs or b not in self.segs:
            raise CacheError("ESTATE", "unknown node")
        pa = self._path_segments(a)
        pb = set(self._path_segments(b))
        for s in pa:
            if s in pb:
                return 0 if s == 0 else self.segs[s].bottom.depth
        return 0

    # ------------------------------------------------------------ introspection
    def dump(self) -> list:
        """Preorder list of (id, parent, length, ref, tick, tokens, slots); children by first token."""
        out = []
        children = {}
        for s in self.segs.values():
            if s.id != 0:
                children.setdefault(s.parent, []).append(s)

        def rec(sid):
            kids = sorted(children.get(sid, []), key=lambda c: c.top.tok)
            for c in kids:
                vs = self._seg_vertices(c)
                out.append((c.id, c.parent, len(vs), c.ref, c.tick, tuple(x.tok for x in vs),
                            tuple(-1 - x.slot if c.host else x.slot for x in vs)))
                rec(c.id)

        rec(0)
        return out

    def stats(self) -> dict:
        cached = sum(self._seg_len(s) for s in self.segs.values() if not s.host)
        locked = sum(self._seg_len(s) for s in self.segs.values() if s.ref > 0)
        host = sum(self._seg_len(s) for s in self.segs.values() if s.host)
        return dict(cached=cached, locked=locked, evictable=cached - locked,
                    nodes=len(self.segs) - 1, free=len(self.free), host=host, host_free=len(self.hfree))
