"""Pins of the prompt-lookup drafting oracle (goinfer, 'Turn nine in under
half a second', section 'What we got wrong'): hand-worked cases and an
independent string-search formulation on random histories."""
import json
import os

import numpy as np
import pytest

from oracle.ngram import ngram_draft

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_hand.json")


def test_hand_worked_cases():
    for c in json.load(open(GOLDEN))["cases"]:
        got = ngram_draft(c["tokens"], c["k"], c["max_ngram"], c["min_ngram"])
        assert got == c["draft"], c["why"]


def _by_rfind(tokens, k, max_ngram, min_ngram):
    """Same reading through str.rfind on a separator-joined history: the
    latest earlier occurrence of the suffix string, then the tokens after."""
    n = len(tokens)
    if k <= 0:
        return []
    text = "," + ",".join(str(x) for x in tokens) + ","
    for g in range(min(max_ngram, n - 1), min_ngram - 1, -1):
        pat = "," + ",".join(str(x) for x in tokens[n - g:]) + ","
        end_of_history_match = len(text) - len(pat)  # the suffix itself
        pos = text.rfind(pat, 0, end_of_history_match + len(pat) - 1)
        if pos >= 0 and pos < end_of_history_match:
            start_tok = text[:pos + 1].count(",") - 1  # token index of the match
            return list(tokens[start_tok + g:start_tok + g + k])
    return []


@pytest.mark.parametrize("seed", range(40))
def test_matches_string_search(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(0, 60))
    vocab = int(g.integers(2, 6))
    tokens = g.integers(0, vocab, n).tolist()
    k = int(g.integers(0, 7))
    lo = int(g.integers(1, 4))
    hi = lo + int(g.integers(0, 3))
    assert ngram_draft(tokens, k, hi, lo) == _by_rfind(tokens, k, hi, lo)


def test_longest_suffix_wins_over_later_shorter_match():
    # [1,2] occurred at 0 (followed by 8); [2] alone latest at 3 (followed by 9)
    t = [1, 2, 8, 2, 9, 1, 2]
    assert ngram_draft(t, 1, 2, 1) == [8]
    assert ngram_draft(t, 1, 1, 1) == [9]
