"""A token-by-token constrained decoder on the library's kernels.

This is the baseline parallel constrained decoding is measured against: the
answer is written one token per decoder pass, field after field, each field
seeing the answers before it, as a model writing the JSON itself would
("Parallel Constrained Decoding from Scratch", "The problem: most of a JSON
answer is not an answer": every scaffold token and every label token costs a
pass).  Scaffold tokens are forced.  At a label token the next token is the
most likely of the tokens that continue some spelling of some label (the
children of the trie node reached so far; a single child is forced), until a
spelling is complete; its label is the field's answer.

Every pass is one library call on a growing state (pcd_extend or
pcd_extend_decide): one new output token, one decoder pass.  The state runs
one or two tokens behind the text written so far: a pass that must read the
next-token distribution after the newest token processes that token as the
one-token scaffold of a field (not appended) and appends the token before it,
so each output token costs exactly one pass.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence


@dataclasses.dataclass
class GreedyResult:
    labels: List[int]          # per field, the label written
    tokens: List[int]          # every output token, in order
    passes: int                # decoder passes after the prefill


@dataclasses.dataclass
class _OneToken:
    """A field of one scaffold token whose candidates are single tokens."""
    scaffold: List[int]
    candidates: List[List[int]]


def _spellings(f) -> List[List[List[int]]]:
    sp = getattr(f, "spellings", None)
    if sp is None:
        return [[[int(t) for t in c]] for c in f.candidates]
    return [[[int(t) for t in c] for c in lab] for lab in sp]


def decode(model, prefix: Sequence[int], fields, capacity: int = 0) -> GreedyResult:
    """Greedy constrained decoding of `fields` after `prefix`, one decoder
    pass per output token.  `capacity`: tokens the state's buffer holds
    (default: the prefix plus every scaffold and the longest spelling of each
    field)."""
    prefix = [int(t) for t in prefix]
    if capacity <= 0:
        capacity = len(prefix) + sum(len(f.scaffold) + max(len(s) for lab in _spellings(f) for s in lab)
                                     for f in fields)
    st = model.prefill(prefix[:-1], capacity=capacity) if len(prefix) > 1 else model.new_state(capacity)
    pending = [prefix[-1]]        # written, not yet in the state (one or two tokens)
    out: List[int] = []
    labels: List[int] = []
    passes = 0

    def forced(x: int):
        nonlocal pending, passes
        st.extend(pending)
        pending = [x]
        out.append(x)
        passes += 1

    def choose(allowed: List[int]) -> int:
        nonlocal pending, passes
        r = model.extend_decide(st, pending[:-1], [_OneToken([pending[-1]], [[a] for a in allowed])])
        c = allowed[int(r["argmax"][0])]
        pending = [pending[-1], c]
        out.append(c)
        passes += 1
        return c

    for f in fields:
        for x in f.scaffold:
            forced(int(x))
        spells = [(k, s) for k, lab in enumerate(_spellings(f)) for s in lab]
        written: List[int] = []
        while True:
            live = [(k, s) for k, s in spells if s[:len(written)] == written]
            done = [k for k, s in live if len(s) == len(written)]
            if done:
                labels.append(done[0])
                break
            allowed: List[int] = []
            for _, s in live:
                if s[len(written)] not in allowed:
                    allowed.append(s[len(written)])
            if len(allowed) == 1:
                forced(allowed[0])
                written.append(allowed[0])
            else:
                written.append(choose(allowed))
    st.close()
    return GreedyResult(labels, out, passes)
