"""Cache hit rate and computed-token counts.

TEST INFRASTRUCTURE (oracle).

Two definitions from the pages, which must agree:
  * hit rate = cached prompt tokens / prompt tokens (2312.07104_SGLang notes,
    §3 "Cache-aware scheduling");
  * hit rate = 1 - C / sum of prefill tokens, with C the number of tokens whose
    KV had to be computed (same notes, App. A.3, proof of Theorem 3.1).
Theorem 3.1 (same notes §3 and App. A.3; bowenzhou SGLang review): with a cache
at least as large as the longest request, visiting requests in the radix tree's
depth-first order computes every tree edge exactly once, so C equals the total
edge length, i.e. the number of distinct token prefixes.
"""
from __future__ import annotations


def hit_rate_cached(matched, prompt_lens) -> float:
    return sum(matched) / sum(prompt_lens)


def hit_rate_computed(computed: int, prompt_lens) -> float:
    return 1.0 - computed / sum(prompt_lens)


def computed_tokens(matched, prompt_lens) -> int:
    return sum(n - m for m, n in zip(matched, prompt_lens))


def no_cache_tokens(prompt_lens) -> int:
    return sum(prompt_lens)
