"""Canonical plan of a PCD request (oracle; test infrastructure only).

What the plan encodes, and where the pages say it:
  * One row per field: the field's scaffold tokens (the text of the row up to
    the point where its labels part ways), appended after the shared prefix
    ([Scratch], "The idea: parallel constrained decoding", steps 2-3; [README],
    "The technique").  The readout position is the row's last token.
  * Candidates whose first tokens collide are told apart by following the
    shared branch inside the same batched pass and multiplying along the path
    ([Scratch], "When one token is not enough"; [TechRef] section 4, stage 5).
    Every candidate token sequence is known in advance, so the continuation
    rows are teacher-forced ([FirstPr], "Multi-token candidates").

Canonical trie per field: nodes are created by inserting the candidates in
declaration order, so the children of a node are ordered by the first
declaration index that reaches them; nodes are numbered breadth-first.
Readout nodes are the root plus every non-root node with two or more
candidates below it.  A candidate c is scored on the edges c[0..u(c)], where
u(c) is the first index at which c's token prefix c[0..u] belongs to no other
candidate.

Branch tokens, per request then per field: the scaffold tokens in order, then
the field's non-root readout nodes in BFS order (each carries its edge token).
Token positions are those a from-scratch run of prefix + scaffold + path would
give: P + offset.  Each branch token sees the whole prefix of its request plus
the branch tokens listed as its ancestors (itself included).

Spellings ([Scratch], "Small models quote their booleans"): a label may be
written several ways (a bare and a quoted boolean); a label is the set of its
spellings, and its probability is the sum of its spellings' path products.
The trie is built over every spelling of every label of the field, inserted
label by label and, within a label, in the order given; u(c) is taken over
spellings, so a spelling is followed until no other spelling (of any label)
shares its tokens.  A field without explicit spellings has one spelling per
candidate.

Scoring modes (the rules the pages describe for multi-token labels):
  path  - the default: full-vocabulary log p of c[0..u(c)] summed
          ([Scratch], "When one token is not enough");
  exact - every token of the spelling, to its end ([Scratch], same section:
          scoring a label to the end of its line); each non-leaf trie node is
          then a readout;
  level - per level, a softmax over the node's child tokens only, multiplied
          down to u(c) ([README], "The technique" and "Caveats": confidence
          as the product of per-level probabilities);
  mean  - the exact sum divided by the spelling's token count ([FirstPr],
          "Multi-token candidates": length normalisation).

Validation (a reading of the pages' limits): every field needs a non-empty
scaffold and 2..255 candidates ([TechRef], "At a glance" and the schema
checklist); candidates must be non-empty, distinct, and no candidate may be a
proper prefix of another (with token ids only, the end of a label is unknown,
so callers end each label with an explicit terminator token).  With
spellings, the same holds for all spellings of a field taken together, each
label needs at least one spelling, and a field has at most 1024 spellings.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence

import numpy as np

MAX_CANDIDATES = 255
MAX_SPELLINGS = 1024
MODES = ("path", "exact", "level", "mean")


def field_spellings(f) -> List[List[List[int]]]:
    """Per label, its spellings (token lists): the field's ``spellings`` when
    given, else one spelling per candidate."""
    sp = getattr(f, "spellings", None)
    if sp is None:
        return [[[int(t) for t in c]] for c in f.candidates]
    return [[[int(t) for t in c] for c in lab] for lab in sp]


def field_mode(f) -> str:
    return getattr(f, "mode", None) or "path"


class PlanError(ValueError):
    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


@dataclasses.dataclass
class TrieNode:
    token: int
    parent: int
    depth: int
    cands: List[int]
    children: List[int]


def build_trie(cands: Sequence[Sequence[int]]) -> List[TrieNode]:
    """Trie over candidate token sequences, nodes in BFS order (node 0 = root)."""
    nodes = [TrieNode(-1, -1, 0, [], [])]
    child_of = {}
    for ci, c in enumerate(cands):
        cur = 0
        nodes[0].cands.append(ci)
        for t in c:
            key = (cur, int(t))
            if key not in child_of:
                nodes.append(TrieNode(int(t), cur, nodes[cur].depth + 1, [], []))
                child_of[key] = len(nodes) - 1
                nodes[cur].children.append(len(nodes) - 1)
            cur = child_of[key]
            nodes[cur].cands.append(ci)
    # renumber breadth-first
    order = [0]
    i = 0
    while i < len(order):
        order.extend(nodes[order[i]].children)
        i += 1
    new_id = {old: new for new, old in enumerate(order)}
    out = []
    for old in order:
        n = nodes[old]
        out.append(TrieNode(n.token, new_id.get(n.parent, -1), n.depth, list(n.cands),
                            [new_id[c] for c in n.children]))
    return out


def validate_field(scaffold, labels, vocab_size: int, mode: str = "path"):
    """labels: per label, its spellings (token lists)."""
    if mode not in MODES:
        raise PlanError("ARG", f"unknown scoring mode {mode!r}")
    if len(scaffold) == 0:
        raise PlanError("EMPTY", "empty scaffold")
    if not (2 <= len(labels) <= MAX_CANDIDATES):
        raise PlanError("NCAND", f"{len(labels)} candidates (allowed 2..{MAX_CANDIDATES})")
    if any(len(lab) == 0 for lab in labels):
        raise PlanError("EMPTY", "a label without spellings")
    cands = [c for lab in labels for c in lab]
    if len(cands) > MAX_SPELLINGS:
        raise PlanError("NCAND", f"{len(cands)} spellings (allowed up to {MAX_SPELLINGS})")
    for t in list(scaffold) + [t for c in cands for t in c]:
        if not (0 <= int(t) < vocab_size):
            raise PlanError("TOKEN", f"token id {t} outside [0, {vocab_size})")
    seen = set()
    for c in cands:
        if len(c) == 0:
            raise PlanError("EMPTY", "empty candidate")
        tc = tuple(int(t) for t in c)
        if tc in seen:
            raise PlanError("DUP", f"duplicate candidate {list(tc)}")
        seen.add(tc)
    for a in seen:
        for b in seen:
            if len(a) < len(b) and b[:len(a)] == a:
                raise PlanError("PREFIX", f"candidate {list(a)} is a proper prefix of {list(b)}")


@dataclasses.dataclass
class Plan:
    """Flat integer arrays (int32) describing one batched branch pass."""
    tok: np.ndarray        # [Tb] branch token ids
    pos: np.ndarray        # [Tb] absolute positions
    req: np.ndarray        # [Tb] request index of each branch token
    tfield: np.ndarray     # [Tb] global field index of each branch token
    anc_off: np.ndarray    # [Tb+1]
    anc: np.ndarray        # ancestors (branch token indices, ascending, self last)
    ro_tok: np.ndarray     # [R] branch token index read out
    ro_field: np.ndarray   # [R]
    g_off: np.ndarray      # [R+1]
    g_tok: np.ndarray      # [G] child token ids gathered at each readout
    f_ro_root: np.ndarray  # [F] readout index of each field's root
    f_cand_off: np.ndarray  # [F+1] candidate (label) range of each field (global candidate index)
    f_mode: np.ndarray     # [F] scoring mode, an index into MODES
    c_spell_off: np.ndarray  # [C+1] spelling range of each candidate
    s_path_off: np.ndarray  # [S+1]
    s_path: np.ndarray     # gather indices scored for each spelling, depth order
    n_requests: int

    @property
    def n_branch(self) -> int:
        return len(self.tok)

    @property
    def n_readouts(self) -> int:
        return len(self.ro_tok)

    @property
    def n_gather(self) -> int:
        return len(self.g_tok)

    def arrays(self):
        return {k: getattr(self, k) for k in (
            "tok", "pos", "req", "tfield", "anc_off", "anc", "ro_tok", "ro_field", "g_off", "g_tok",
            "f_ro_root", "f_cand_off", "f_mode", "c_spell_off", "s_path_off", "s_path")}


def build_plan(requests, vocab_size: int) -> Plan:
    """requests: list of (prefix_len, fields) with fields a list of objects
    carrying ``scaffold`` and ``candidates`` (and optionally ``spellings``,
    per label a list of token lists, and ``mode``, one of MODES)."""
    tok, pos, req, tfield, anc_off, anc = [], [], [], [], [0], []
    ro_tok, ro_field, g_off, g_tok = [], [], [0], []
    f_ro_root, f_cand_off, f_mode, c_spell_off, s_path_off, s_path = [], [0], [], [0], [0], []
    gf = 0
    for r, (P, fields) in enumerate(requests):
        for f in fields:
            sc = [int(t) for t in f.scaffold]
            labels = field_spellings(f)
            mode = field_mode(f)
            validate_field(sc, labels, vocab_size, mode)
            spells = [c for lab in labels for c in lab]
            to_end = mode in ("exact", "mean")
            nodes = build_trie(spells)
            base = len(tok)
            # scaffold tokens
            for j, t in enumerate(sc):
                tok.append(t); pos.append(P + j); req.append(r); tfield.append(gf)
                anc.extend(range(base, base + j + 1)); anc_off.append(len(anc))
            last_scaffold = base + len(sc) - 1
            # non-root readout nodes, BFS order: nodes the labels still share, or
            # (scoring to the end) every node some spelling continues from
            is_ro = [i == 0 or (len(n.children) > 0 if to_end else len(n.cands) >= 2)
                     for i, n in enumerate(nodes)]
            branch_of = {0: last_scaffold}
            for i, n in enumerate(nodes):
                if i == 0 or not is_ro[i]:
                    continue
                bi = len(tok)
                branch_of[i] = bi
                tok.append(n.token); pos.append(P + len(sc) + n.depth - 1); req.append(r); tfield.append(gf)
                path = []
                a = i
                while a != 0:
                    path.append(branch_of[a])
                    a = nodes[a].parent
                anc.extend(list(range(base, base + len(sc))) + sorted(path)); anc_off.append(len(anc))
            # readouts and gathers
            gidx = {}
            for i, n in enumerate(nodes):
                if not is_ro[i]:
                    continue
                ri = len(ro_tok)
                if i == 0:
                    f_ro_root.append(ri)
                ro_tok.append(branch_of[i]); ro_field.append(gf)
                for ch in n.children:
                    gidx[(i, nodes[ch].token)] = len(g_tok)
                    g_tok.append(nodes[ch].token)
                g_off.append(len(g_tok))
            # spelling paths: edges c[0..u(c)], or every edge when scoring to the end
            for lab in labels:
                for c in lab:
                    cur = 0
                    for t in c:
                        s_path.append(gidx[(cur, t)])
                        nxt = [ch for ch in nodes[cur].children if nodes[ch].token == t][0]
                        if len(nodes[nxt].cands) == 1 and not to_end:
                            break
                        cur = nxt
                    s_path_off.append(len(s_path))
                c_spell_off.append(c_spell_off[-1] + len(lab))
            f_cand_off.append(f_cand_off[-1] + len(labels))
            f_mode.append(MODES.index(mode))
            gf += 1
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return Plan(i32(tok), i32(pos), i32(req), i32(tfield), i32(anc_off), i32(anc), i32(ro_tok), i32(ro_field),
                i32(g_off), i32(g_tok), i32(f_ro_root), i32(f_cand_off), i32(f_mode), i32(c_spell_off),
                i32(s_path_off), i32(s_path), len(requests))
