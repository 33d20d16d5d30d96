"""Oracle: prompt-lookup (n-gram) drafting.

Test infrastructure only (see ``oracle/__init__.py``).

goinfer, "Turn nine in under half a second", section "What we got wrong":
the n-gram form of speculation drafts its tokens by copying what followed an
earlier occurrence of the latest tokens in the prompt itself, and a single
verify pass then accepts or rejects the draft.

Readings (the page says no more):
  * the guess continues the most recent earlier occurrence of the longest
    suffix of the token history that occurred before: suffix lengths are
    tried from max_ngram down to min_ngram, and for each length the
    occurrences starting at p = n-g-1, n-g-2, ..., 0 (overlapping the suffix
    is allowed, the suffix itself is not an occurrence);
  * the draft is the up to k tokens that followed that occurrence
    (tokens[p+g : p+g+k], shorter at the end of the history);
  * no occurrence of any length: an empty draft (a plain decode step).
"""
from __future__ import annotations


def ngram_draft(tokens, k: int, max_ngram: int = 3, min_ngram: int = 1) -> list[int]:
    """Draft tokens for the history `tokens` (a sequence of ints)."""
    t = [int(x) for x in tokens]
    n = len(t)
    if k <= 0:
        return []
    for g in range(min(max_ngram, n - 1), min_ngram - 1, -1):
        suffix = t[n - g:]
        for p in range(n - g - 1, -1, -1):
            if t[p:p + g] == suffix:
                return t[p + g:p + g + k]
    return []
