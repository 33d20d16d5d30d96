"""Oracle: greedy acceptance of a speculative verify step, the KV rollback it
implies, and the rolling-acceptance gate.

Test infrastructure only (see ``oracle/__init__.py``).

thinkspread, "The economics of speculative decoding: +41% on 9B, break-even
on 35B":
  * opening section: a draft head proposes k tokens, the full model checks
    them in one pass over m = k + 1 rows, and the runtime keeps the ones that
    were right;
  * "Gating: enable it only where it pays": when the rolling acceptance drops
    under a threshold (0.60 on that page) the runtime falls back to ordinary
    decoding;
  * "Closing the ledger": the cost model verify(m) = a + b*m prices whether
    speculation pays.

Readings (the pages do not spell these out):
  * "right" is greedy matching: row i of the verify logits predicts the token
    after input i; draft token i+1 is kept while it equals that row's argmax,
    and the first mismatch ends the run. The step then emits the argmax of the
    row after the last kept draft (the correction, or a bonus token when every
    draft was kept).
  * argmax ties go to the lowest token id; a NaN counts as larger than any
    number (the first NaN wins), as numpy's argmax does.
  * the verify appended m rows at positions P .. P+k; the kept ones are the
    last accepted input plus the accepted drafts, so the cache is cut back to
    P + accepted + 1 positions.
  * acceptance of a step = accepted / k; the rolling acceptance is the mean
    over the last `window` steps (fewer at the start), taken as (sum of the
    accepted counts) / (k * steps), and once it is below the threshold the
    request stops speculating (k = 0) for good.
  * the break-even acceptance of depth k under verify(m) = a + b*m, with a
    per-position acceptance alpha that is the same at every depth, is the
    alpha where the expected tokens per verify step, 1 + alpha + ... +
    alpha^k, times the cost of a one-row step equals the cost of a k+1 row
    step; the draft head's own cost is left out.
"""
from __future__ import annotations

import numpy as np


def argmax_rows(logits) -> np.ndarray:
    """Per-row argmax of an [m][V] array (ties: lowest index; NaN wins)."""
    x = np.asarray(logits, dtype=np.float64)
    return np.argmax(x, axis=1).astype(np.int64)


def greedy_accept(logits, draft):
    """(accepted, next_token, per-row argmax) of one verify step.

    logits: [m][V] rows for the inputs (last accepted token, draft_1 ..
    draft_k); draft: the k = m - 1 drafted token ids."""
    t = argmax_rows(logits)
    m = t.shape[0]
    draft = np.asarray(draft, dtype=np.int64)
    assert draft.shape == (m - 1,)
    accepted = 0
    while accepted < m - 1 and draft[accepted] == t[accepted]:
        accepted += 1
    return accepted, int(t[accepted]), t


def rollback_len(P: int, accepted: int) -> int:
    """Cached positions kept after a verify that started at P."""
    return P + accepted + 1


def expected_tokens(alpha: float, k: int) -> float:
    """Tokens emitted per verify step at per-position acceptance alpha."""
    return sum(alpha ** i for i in range(k + 1))


def break_even_acceptance(a: float, b: float, k: int) -> float:
    """alpha in [0, 1] where expected_tokens(alpha, k) * (a + b) = a + b*(k+1),
    by bisection (the left side grows with alpha); 1.0 if even alpha = 1 does
    not pay, 0.0 if k = 0."""
    if k <= 0:
        return 0.0
    need = (a + b * (k + 1)) / (a + b)
    if expected_tokens(1.0, k) < need:
        return 1.0
    lo, hi = 0.0, 1.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if expected_tokens(mid, k) < need:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


class RollingGate:
    """Rolling-acceptance gate of one request ("Gating: enable it only where
    it pays")."""

    def __init__(self, k: int, min_accept: float = 0.60, window: int = 8):
        assert k >= 0 and window >= 1
        self.k = k
        self.min_accept = min_accept
        self.window = window
        self.accepted: list[int] = []

    def rolling(self) -> float:
        recent = self.accepted[-self.window:]
        return sum(recent) / (self.k * len(recent)) if recent else 1.0

    def step(self, accepted: int) -> int:
        """Record one verify step with `accepted` of k drafts kept; returns
        the depth for the next step (k, or 0 once the gate has closed)."""
        if self.k == 0:
            return 0
        assert 0 <= accepted <= self.k
        self.accepted.append(int(accepted))
        if self.rolling() < self.min_accept:
            self.k = 0
        return self.k
