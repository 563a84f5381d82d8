"""PCD end to end in fp64 (oracle; test infrastructure only).

Steps, in the order the pages give them ([TechRef] section 4 "The algorithm";
[README] "The technique"; [Scratch] "The idea: parallel constrained decoding"):
  1. prefill the shared prefix once and keep its K/V;
  2. share that K/V with every field row (here: every branch token attends the
     whole cached prefix of its request; nothing is recomputed);
  3. one batched pass over all branch tokens (field scaffolds plus the
     teacher-forced trie continuation tokens);
  4. at each readout row, the full-vocabulary next-token distribution, of
     which only the candidate tokens are kept;
  5. combine: per candidate the sum of log-probabilities along its scored
     path, a softmax over the field's candidates at temperature T, and the
     candidate mass.

Combine, written out (the default "path" scoring; plan.py lists the other
modes and the spelling sets):
  logscore(c) = sum_{i=0}^{u(c)} log p(c[i] | prefix + scaffold + c[<i])
  q           = softmax(logscore / T)           ([TechRef] section 4, stage 4)
  mass        = sum over distinct first tokens t of p(t | prefix + scaffold)
                ([Scratch], "And you get confidence for free")
  argmax      = largest logscore, ties to the lowest declaration index
                ([TechRef], "Notes on the softmax" leaves ties open; the
                first-declared candidate wins here)
  margin      = top-1 minus top-2 logscore, in nats (T = 1).
For single-token candidates, q is the subset softmax of the logits, which
equals p_S / mass: the full-vocabulary normaliser cancels ([FirstPr], "The
subset softmax is exact").
With spelling sets, a label's logscore is log of the sum over its spellings
of exp(spelling score); q, argmax and margin are taken over labels.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

from .decoder import Decoder, causal_mask
from .plan import MODES, Plan, build_plan, build_trie, field_mode, field_spellings


@dataclasses.dataclass
class FieldResult:
    prob: np.ndarray       # [K] candidate probabilities (sum to 1)
    logscore: np.ndarray   # [K]
    mass: float
    argmax: int
    margin: float


@dataclasses.dataclass
class DecideResult:
    plan: Plan
    lse: np.ndarray        # [R] full-vocabulary log-sum-exp per readout row
    z: np.ndarray          # [G] gathered logits
    fields: List[FieldResult]
    passes: Dict[str, int]
    token_by_token_steps: int


def prefill(dec: Decoder, prefix: Sequence[int], n_layers: Optional[int] = None):
    """Step 1: one causal pass over the prefix at positions 0..P-1; returns the
    per-layer (K, V) after RoPE, each [Hkv, P, hd]."""
    P = len(prefix)
    _, kv = dec.forward(list(prefix), np.arange(P), causal_mask(P), None, n_layers)
    return kv


def branch(dec: Decoder, plan: Plan, prefix_kv: List, n_layers: Optional[int] = None) -> np.ndarray:
    """Steps 2-3: every branch token of every request in one pass.  Token t sees
    the whole cached prefix of its request and the branch tokens listed as its
    ancestors.  Requests are independent, so each request's tokens run as one
    group against its own prefix K/V.  Returns residual rows x [Tb, d]."""
    Tb = plan.n_branch
    x = np.zeros((Tb, dec.sh.d_model), dec.dt)
    for r in range(plan.n_requests):
        idx = np.nonzero(plan.req == r)[0]
        if len(idx) == 0:
            continue
        local = {int(g): i for i, g in enumerate(idx)}
        mask = np.zeros((len(idx), len(idx)), bool)
        for i, g in enumerate(idx):
            for a in plan.anc[plan.anc_off[g]:plan.anc_off[g + 1]]:
                mask[i, local[int(a)]] = True
        xr, _ = dec.forward(plan.tok[idx], plan.pos[idx], mask, prefix_kv[r], n_layers)
        x[idx] = xr
    return x


def readout(dec: Decoder, plan: Plan, x: np.ndarray):
    """Step 4: full logits at each readout row, their log-sum-exp, and the
    logits of each readout's child tokens."""
    z_full = dec.logits(x[plan.ro_tok])
    lse = Decoder.logsumexp(z_full)
    z = np.empty(plan.n_gather, dec.dt)
    for r in range(plan.n_readouts):
        for g in range(plan.g_off[r], plan.g_off[r + 1]):
            z[g] = z_full[r, plan.g_tok[g]]
    return lse, z


def combine_field(edge_logp: np.ndarray, paths: List[Sequence[int]], root_edges: Sequence[int],
                  temperature: float = 1.0, labels: Optional[Sequence[int]] = None,
                  mean: bool = False) -> FieldResult:
    """Step 5 for one field.  edge_logp[g] is the log-probability of gather g
    under the field's scoring mode; paths[c] lists the gather indices scored
    for spelling c; root_edges lists the gathers of the root readout (its
    distinct first tokens), whose probabilities must be full-vocabulary ones.

    ``mean``: a spelling's score is the mean of its edge log-probabilities.
    ``labels`` (optional) groups spellings that write one label: a label's
    probability sums its spellings' path products ([Scratch], "Small models
    quote their booleans").  With labels given, ``prob``/``logscore`` are per
    label."""
    ls = np.array([sum(edge_logp[g] for g in p) / (len(p) if mean else 1) for p in paths], dtype=np.float64)
    if labels is not None:
        nl = max(labels) + 1
        ls = np.array([np.log(sum(np.exp(ls[c]) for c in range(len(ls)) if labels[c] == k)) for k in range(nl)])
    s = ls / temperature
    s = s - s.max()
    q = np.exp(s) / np.exp(s).sum()
    mass = float(sum(np.exp(edge_logp[g]) for g in root_edges))
    best = int(np.argmax(ls))  # numpy returns the first maximum
    srt = np.sort(ls)[::-1]
    margin = float(srt[0] - srt[1]) if len(srt) > 1 else float("inf")
    return FieldResult(q, ls, mass, best, margin)


def combine(plan: Plan, lse: np.ndarray, z: np.ndarray, temperature: float = 1.0) -> List[FieldResult]:
    ro_of_g = np.repeat(np.arange(plan.n_readouts), np.diff(plan.g_off))
    edge_full = z - lse[ro_of_g]
    # "level": each readout's child logits softmaxed among themselves
    sub = np.array([Decoder.logsumexp(z[plan.g_off[r]:plan.g_off[r + 1]][None])[0] if plan.g_off[r + 1] > plan.g_off[r]
                    else 0.0 for r in range(plan.n_readouts)])
    edge_level = z - sub[ro_of_g]
    out = []
    for f in range(len(plan.f_ro_root)):
        mode = MODES[plan.f_mode[f]]
        c0, c1 = plan.f_cand_off[f], plan.f_cand_off[f + 1]
        s0, s1 = plan.c_spell_off[c0], plan.c_spell_off[c1]
        paths = [plan.s_path[plan.s_path_off[k]:plan.s_path_off[k + 1]] for k in range(s0, s1)]
        labels = [c - c0 for c in range(c0, c1) for _ in range(plan.c_spell_off[c], plan.c_spell_off[c + 1])]
        r = plan.f_ro_root[f]
        res = combine_field(edge_level if mode == "level" else edge_full, paths,
                            range(plan.g_off[r], plan.g_off[r + 1]), temperature, labels, mean=mode == "mean")
        # mass is a full-vocabulary quantity in every mode
        res.mass = float(sum(np.exp(edge_full[g]) for g in range(plan.g_off[r], plan.g_off[r + 1])))
        out.append(res)
    return out


def answer_tokens(f, label: int) -> List[int]:
    """The tokens written for a field's label: its first spelling."""
    return field_spellings(f)[label][0]


def token_by_token_steps(requests, results: List[FieldResult]) -> int:
    """Sequential passes a token-by-token decoder would need for the same
    fields: every scaffold token and every token of the chosen label is one
    pass ([Scratch], "The problem: most of a JSON answer is not an answer")."""
    n, i = 0, 0
    for _, fields in requests:
        for f in fields:
            n += len(f.scaffold) + len(answer_tokens(f, results[i].argmax))
            i += 1
    return n


def decide(dec: Decoder, requests, temperature: float = 1.0, prefix_kv=None,
           n_layers: Optional[int] = None) -> DecideResult:
    """requests: list of (prefix tokens, fields).  Runs steps 1-5."""
    plan = build_plan([(len(p), f) for p, f in requests], dec.sh.vocab_size)
    if prefix_kv is None:
        prefix_kv = [prefill(dec, p, n_layers) for p, _ in requests]
    x = branch(dec, plan, prefix_kv, n_layers)
    lse, z = readout(dec, plan, x)
    res = combine(plan, lse, z, temperature)
    steps = token_by_token_steps([(len(p), f) for p, f in requests], res)
    return DecideResult(plan, lse, z, res, {"prefill": 1, "branch": 1}, steps)


def decide_sequenced(dec: Decoder, prefix: Sequence[int], fields, n_first: int, temperature: float = 1.0,
                     n_layers: Optional[int] = None):
    """The first-field round ([Scratch] "The idea: parallel constrained
    decoding": the first field is decided, its answer written into the
    prompt, and the remaining fields decided against it).  Reading taken: the
    answer of a field is its scaffold followed by its argmax candidate, the
    first n_first fields' answers are appended in field order, and the rest
    are decided against that extended prefix.  Returns (first result, rest
    result, extended prefix)."""
    first = decide(dec, [(list(prefix), fields[:n_first])], temperature, n_layers=n_layers)
    ext = list(prefix)
    for f, r in zip(fields[:n_first], first.fields):
        ext += list(f.scaffold) + answer_tokens(f, r.argmax)
    rest = decide(dec, [(ext, fields[n_first:])], temperature, n_layers=n_layers)
    return first, rest, ext


# ----------------------------------------------------------------------------
# independent references built on plain causal runs (no cache, no batching)
# ----------------------------------------------------------------------------

def next_token_logp(dec: Decoder, seq: Sequence[int], n_layers: Optional[int] = None) -> np.ndarray:
    """log p(. | seq) from one plain causal run of the whole sequence."""
    T = len(seq)
    x, _ = dec.forward(list(seq), np.arange(T), causal_mask(T), None, n_layers)
    z = dec.logits(x[-1:])[0]
    return z - Decoder.logsumexp(z[None])[0]


def scratch_readouts(dec: Decoder, requests, n_layers: Optional[int] = None):
    """For every readout node v: log p(child | prefix + scaffold + path(v)) from
    a from-scratch causal run, in the plan's gather order, and the from-scratch
    log-sum-exp of the logits."""
    plan = build_plan([(len(p), f) for p, f in requests], dec.sh.vocab_size)
    edge = np.empty(plan.n_gather)
    lse = np.empty(plan.n_readouts)
    r = 0
    for prefix, fields in requests:
        for f in fields:
            to_end = field_mode(f) in ("exact", "mean")
            nodes = build_trie([c for lab in field_spellings(f) for c in lab])
            for i, n in enumerate(nodes):
                if not (i == 0 or (len(n.children) > 0 if to_end else len(n.cands) >= 2)):
                    continue
                path = []
                a = i
                while a != 0:
                    path.append(nodes[a].token)
                    a = nodes[a].parent
                seq = list(prefix) + list(f.scaffold) + path[::-1]
                T = len(seq)
                x, _ = dec.forward(seq, np.arange(T), causal_mask(T), None, n_layers)
                z = dec.logits(x[-1:])[0]
                l = Decoder.logsumexp(z[None])[0]
                lse[r] = l
                for g in range(plan.g_off[r], plan.g_off[r + 1]):
                    edge[g] = z[plan.g_tok[g]] - l
                r += 1
    return plan, edge, lse


def greedy_decode(dec: Decoder, prefix, fields, n_layers: Optional[int] = None):
    """The token-by-token baseline, from scratch: fields in order, each
    written after the text so far ([Scratch], "The problem: most of a JSON
    answer is not an answer").  Scaffold tokens are copied; at each label
    token the allowed tokens are the next tokens of the spellings that agree
    with what was written (in first-appearance order), and the one with the
    largest log p(. | text) is written (ties to the first); a single allowed
    token is written without a choice.  Stops a field when a spelling is
    complete.  Returns (label per field, output tokens, output token count)."""
    text = [int(t) for t in prefix]
    labels, out = [], []
    for f in fields:
        text += [int(t) for t in f.scaffold]
        out += [int(t) for t in f.scaffold]
        spells = [(k, list(s)) for k, lab in enumerate(field_spellings(f)) for s in lab]
        w: List[int] = []
        while True:
            live = [(k, s) for k, s in spells if s[:len(w)] == w]
            done = [k for k, s in live if len(s) == len(w)]
            if done:
                labels.append(done[0])
                break
            allowed = []
            for _, s in live:
                if s[len(w)] not in allowed:
                    allowed.append(s[len(w)])
            if len(allowed) == 1:
                c = allowed[0]
            else:
                lp = next_token_logp(dec, text, n_layers)
                c = max(allowed, key=lambda t: (lp[t], -allowed.index(t)))
            w.append(c)
            text.append(c)
            out.append(c)
    return labels, out, len(out)


def greedy_first_token(dec: Decoder, prefix, field, n_layers: Optional[int] = None) -> int:
    """Brute-force constrained greedy step for one field decided on its own:
    run prefix + scaffold from scratch and take the allowed first token with
    the largest logit; returns the index of the first candidate starting with
    it."""
    lp = next_token_logp(dec, list(prefix) + list(field.scaffold), n_layers)
    firsts = [c[0] for c in field.candidates]
    best = max(range(len(firsts)), key=lambda i: (lp[firsts[i]], -i))
    return best


def enumerate_scores(dec: Decoder, prefix, field, n_layers: Optional[int] = None, mode: Optional[str] = None,
                     spellings=None) -> np.ndarray:
    """Brute force, per label: each spelling scored from separately computed
    from-scratch conditionals log p(c[i] | prefix + scaffold + c[<i]), with no
    trie: u(c) is found by comparing token prefixes of the spellings directly,
    and (mode "level") a level's sub-vocabulary is the set of next tokens of
    the spellings that share c[<i].  A label's score is log of the sum of
    exp(spelling score) over its spellings."""
    mode = mode or field_mode(field)
    labels = spellings if spellings is not None else field_spellings(field)
    allsp = [list(c) for lab in labels for c in lab]
    ctx = list(prefix) + list(field.scaffold)
    out = []
    for lab in labels:
        tot = []
        for c in lab:
            c = list(c)
            s = 0.0
            for i in range(len(c)):
                lp = next_token_logp(dec, ctx + c[:i], n_layers)
                if mode == "level":
                    sibs = sorted({o[i] for o in allsp if len(o) > i and o[:i] == c[:i]})
                    s += lp[c[i]] - np.log(sum(np.exp(lp[t]) for t in sibs))
                else:
                    s += lp[c[i]]
                if mode in ("path", "level") and not any(o[:i + 1] == c[:i + 1] for o in allsp if o != c):
                    break
            if mode == "mean":
                s /= len(c)
            tot.append(s)
        out.append(np.log(sum(np.exp(v) for v in tot)))
    return np.array(out)
