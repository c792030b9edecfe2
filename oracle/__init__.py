"""CPU oracle for the RadixAttention hot path.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import anything under oracle/. The HIP path never routes
through it, and it shares no code with the HIP path (only the seeded input
generators in workloads/).

Parts: a naive per-token trie (trie.py), a plain segment model of the radix
tree with splits, ref counts, ticks, leaf-first LRU eviction and the slot
allocator (radix_model.py), a trace replayer (runner.py), hit-rate counts
(counts.py) and fp64 causal attention recomputed from scratch (attention.py).
Every function is pinned by tests/test_oracle_*.py; none is "parity unpinned".
"""
