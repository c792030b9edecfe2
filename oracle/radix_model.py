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
    __slots__ = ("id", "top", "bottom", "ref", "tick", "parent")

    def __init__(self, sid, top, bottom, ref, tick, parent):
        self.id = sid
        self.top = top              # first vertex (None for root)
        self.bottom = bottom        # last vertex  (None for root)
        self.ref = ref
        self.tick = tick
        self.parent = parent        # parent segment id (-1 for root)


class RadixCacheModel:
    def __init__(self, num_slots: int):
        self.num_slots = int(num_slots)
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
        up = _Segment(self.next_id, s.top, v, s.ref, s.tick, s.parent)
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
        v = self.root_v
        slots = []
        for t in tokens:
            c = v.children.get(int(t))
            if c is None:
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
        return m, node, out_slots

    def lock_ref(self, node: int, delta: int) -> None:
        if delta not in (1, -1):
            raise CacheError("EINVAL", f"bad delta {delta}")
        if node not in self.segs:
            raise CacheError("ESTATE", f"unknown node {node}")
        path = [p for p in self._path_segments(node) if p != 0]
        if delta < 0 and any(self.segs[p].ref + delta < 0 for p in path):
            raise CacheError("ESTATE", "unlock below zero")
        for p in path:
            self.segs[p].ref += delta

    def evict(self, num_tokens: int) -> list:
        """Free >= num_tokens slots by removing LRU leaves with ref 0 (R6)."""
        freed = []
        while len(freed) < num_tokens:
            cands = [s for s in self.segs.values() if self._is_leaf(s) and s.ref == 0]
            if not cands:
                break
            s = min(cands, key=lambda x: (x.tick, x.id))
            verts = self._seg_vertices(s)
            freed.extend(x.slot for x in verts)
            top = s.top
            del top.parent.children[top.tok]
            del self.segs[s.id]
        if freed:
            self.free_slots(freed)
        return freed

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
                out.append((c.id, c.parent, len(vs), c.ref, c.tick,
                            tuple(x.tok for x in vs), tuple(x.slot for x in vs)))
                rec(c.id)

        rec(0)
        return out

    def stats(self) -> dict:
        cached = sum(self._seg_len(s) for s in self.segs.values())
        locked = sum(self._seg_len(s) for s in self.segs.values() if s.ref > 0)
        return dict(cached=cached, locked=locked, evictable=cached - locked,
                    nodes=len(self.segs) - 1, free=len(self.free))
