"""Naive per-token trie: the plainest longest-prefix match.

TEST INFRASTRUCTURE (oracle). Only tests/, the smoke check and the bench's CPU
baseline leg may use this module.

Follows the "traverse" step of the request loop in the hustzhy SGLang post,
§2.3 (2): from the root, find the longest cached prefix of the request. One
trie node per token, so no path compression and no splitting: the radix-tree
node boundaries are not modelled here (see radix_model.py), only which token
prefixes are cached.
"""
from __future__ import annotations


class NaiveTrie:
    def __init__(self):
        self.root: dict = {}
        self._count = 0

    def insert(self, tokens) -> int:
        """Add every prefix of ``tokens``; return how many prefixes were already present."""
        node = self.root
        existing = 0
        for t in tokens:
            t = int(t)
            if t in node:
                existing += 1
            else:
                node[t] = {}
                self._count += 1
            node = node[t]
        return existing

    def match(self, tokens) -> int:
        """Length of the longest prefix of ``tokens`` present in the trie."""
        node = self.root
        m = 0
        for t in tokens:
            t = int(t)
            if t not in node:
                break
            node = node[t]
            m += 1
        return m

    def num_nodes(self) -> int:
        """Number of distinct non-empty prefixes stored (= sum of radix edge lengths)."""
        return self._count
