"""Oracle: the resident KV-slot store and the slot-selection rule.

Test infrastructure only (see ``oracle/__init__.py``).

Sources (goinfer, "Turn nine in under half a second"):
  * section "How it works": a new prompt goes to the stored conversation with
    the longest common start, provided that start is longer than what that
    conversation has in common with the other stored ones (so a shared system
    prompt cannot pull in another conversation); the conversation is cut back
    to the common point and only the remainder is prefilled. A model held on
    the GPU keeps up to --kv-sessions slots; a request reuses the slot already
    holding the start of its prompt, else takes an empty slot, else the least
    recently used one. The reuse count is reported to the caller.
  * section "What we got wrong": a matching rule that let two alternating
    conversations take each other's session reused only the 7-token template
    start and never kept more than one session.
  * section "Use it": --kv-sessions 0 switches reuse off; the memory check may
    grant fewer slots than requested.

Reading (listed in the design doc). With T_s the tokens of slot s, L_s = LCP(p, T_s)
and O_s the largest LCP of T_s with any other occupied slot (0 if none), slot
s is *eligible* when it is occupied, L_s > 0, L_s > O_s, and either L_s = |T_s|
(the slot holds the start of the prompt) or some other slot is occupied. The
last clause keeps a lone slot from being taken over by a conversation that
only shares its header, which is the failure the pages report. A repeated
prompt reuses at most n - 1 tokens so that its last token still runs through
the model (section "What we got wrong", the one-token-short bug).

Only tokens whose K/V rows are resident in every layer take part in matching:
T_s is the committed prompt of slot s cut to min over layers of kv_len[s].
A slot counts as empty only while no prompt has been selected into it: one
handed to a conversation stays claimed while its prefill is still pending, so
several prompts can be placed before any of them is prefilled.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


def lcp(a, b) -> int:
    """Length of the longest common prefix of two token sequences."""
    n = min(len(a), len(b))
    i = 0
    while i < n and int(a[i]) == int(b[i]):
        i += 1
    return i


@dataclass
class SlotOracle:
    """Host model of the slot store: token lists, LRU ticks and per-layer
    cached lengths; optionally the cached K/V rows themselves."""
    n_slots: int
    n_layers: int = 1
    reuse: bool = True
    literal_rule: bool = False   # the one-sentence rule without the lone-slot clause
    tokens: List[Optional[np.ndarray]] = field(default_factory=list)
    tick: List[int] = field(default_factory=list)
    kv_len: List[List[int]] = field(default_factory=list)
    committed: List[int] = field(default_factory=list)
    clock: int = 0

    def __post_init__(self):
        self.tokens = [None] * self.n_slots
        self.tick = [0] * self.n_slots
        self.kv_len = [[0] * self.n_layers for _ in range(self.n_slots)]
        self.committed = [0] * self.n_slots

    # -- the decision rule -------------------------------------------------
    def resident(self, s: int) -> np.ndarray:
        """Tokens of slot s whose K/V rows are cached in every layer."""
        if self.tokens[s] is None:
            return np.zeros(0, dtype=np.int64)
        return self.tokens[s][:min(self.kv_len[s])]

    def occupied(self, s: int) -> bool:
        return len(self.resident(s)) > 0

    def eligible(self, prompt) -> List[int]:
        occ = [s for s in range(self.n_slots) if self.occupied(s)]
        out = []
        for s in occ:
            ts = self.resident(s)
            ls = lcp(prompt, ts)
            others = [lcp(ts, self.resident(t)) for t in occ if t != s]
            os_ = max(others) if others else 0
            if ls <= 0 or ls <= os_:
                continue
            if not self.literal_rule and not (ls == len(ts) or others):
                continue
            out.append(s)
        return out

    def select(self, prompt):
        """Choose a slot for ``prompt``; commit it; return (slot, reused)."""
        prompt = np.asarray(prompt, dtype=np.int64)
        n = len(prompt)
        if n <= 0:
            raise ValueError("empty prompt")
        el = self.eligible(prompt)
        assert len(el) <= 1, "LCP is ultrametric: at most one slot can be eligible"
        if el:
            s = el[0]
            r = min(lcp(prompt, self.resident(s)), n - 1)
        else:
            empty = [t for t in range(self.n_slots) if self.committed[t] == 0]
            if empty:
                s, r = empty[0], 0
            else:
                s = min(range(self.n_slots), key=lambda t: (self.tick[t], t))
                r = min(lcp(prompt, self.resident(s)), n - 1)
        if not self.reuse:
            r = 0
        self.clock += 1
        self.tick[s] = self.clock
        self.tokens[s] = prompt.copy()
        self.kv_len[s] = [r] * self.n_layers
        self.committed[s] = n
        return s, r

    def truncate(self, s: int, length: int):
        """Cut slot s back to ``length`` cached positions in every layer; the
        committed prompt is kept, so extend can refill it."""
        if length < 0 or length > min(self.kv_len[s]):
            raise ValueError("truncate can only shorten")
        self.kv_len[s] = [length] * self.n_layers

    def extend(self, s: int, layer: int, m: int):
        """Account for m new rows in (slot, layer); returns the prefix P."""
        p = self.kv_len[s][layer]
        if p + m > self.committed[s]:
            raise ValueError("extend beyond the committed prompt")
        self.kv_len[s][layer] = p + m
        return p


def unique_argmax_rule(prompt, slot_tokens) -> Optional[int]:
    """Equivalent statement of the literal rule: the slot whose common start
    with the prompt is strictly the largest over all occupied slots (and > 0).
    Used to cross-check ``SlotOracle.eligible`` with ``literal_rule=True``."""
    ls = [(lcp(prompt, t) if t is not None and len(t) else -1) for t in slot_tokens]
    best = max(ls) if ls else -1
    if best <= 0 or ls.count(best) != 1:
        return None
    return ls.index(best)
