"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None of them retypes the oracle's own
formula: each checks the oracle against a value a page prints, a closed form,
an invariant, brute force, or an independent library implementation of the
same network.  The last group plants mistakes in a copy of the oracle and
checks that at least one pin catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest

import pcd_inputs as pi
from oracle import decoder as odec
from oracle import pcd as opcd
from oracle import plan as oplan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def tiny():
    w = pi.make_weights(pi.SHAPES["tiny"], 1000)
    return odec.Decoder(w, np.float64)


@pytest.fixture(scope="module")
def cfg0():
    return pi.make_workload("cfg0")


@pytest.fixture(scope="module")
def cfg0t():
    return pi.make_workload("cfg0t")


def _reqs(wl):
    return [(r.prefix, r.fields) for r in wl.requests]


# ---------------------------------------------------------------------------
# worked numbers printed on the pages
# ---------------------------------------------------------------------------

def test_softmax_worked_example():
    """Technical Reference, section 4 ("Notes on the softmax"): logits 4.1 and
    1.8 give about 0.91/0.09 at T=1 and 0.76/0.24 at T=2."""
    g = _golden("softmax_worked_example.json")
    fields = [pi.Field([5], [[10], [11]])]
    plan = oplan.build_plan([(3, fields)], 64)
    # the oracle reads logits and a log-sum-exp; any lse gives the same subset softmax
    lse = np.array([7.25])
    z = np.array(g["logits"], dtype=np.float64)
    for key, T in (("T=1", 1.0), ("T=2", 2.0)):
        res = opcd.combine(plan, lse, z, temperature=T)[0]
        assert np.allclose(res.prob, g["printed"][key], atol=g["printed_abs_tolerance"])
        assert res.argmax == g["argmax"]
    # exact values of the same example, from exp() written out by hand
    e = math.exp(4.1 - 1.8)
    assert abs(opcd.combine(plan, lse, z, 1.0)[0].prob[0] - e / (1 + e)) < 1e-15


def test_quoted_boolean_path_products():
    """Parallel Constrained Decoding from Scratch, "Small models quote their
    booleans": follow the opening quote, multiply along the path, sum the two
    spellings of each label, renormalise -> True 0.855."""
    g = _golden("quoted_boolean_paths.json")
    Q, BF, BT, T, F = 100, 101, 102, 103, 104
    field = pi.Field([7, 8], [[Q, T], [Q, F], [BF], [BT]])
    plan = oplan.build_plan([(20, [field])], 256)
    # readout 0 is the root, readout 1 the quote node (two candidates below it)
    assert plan.n_readouts == 2
    p_of = {0: {Q: g["root"]["quote"], BF: g["root"]["false"], BT: g["root"]["true"]},
            1: {T: g["after_quote"]["true"], F: g["after_quote"]["false"]}}
    edge = np.empty(plan.n_gather)
    for r in range(plan.n_readouts):
        for gi in range(plan.g_off[r], plan.g_off[r + 1]):
            edge[gi] = math.log(p_of[r][int(plan.g_tok[gi])])
    paths = [plan.s_path[plan.s_path_off[c]:plan.s_path_off[c + 1]] for c in range(4)]
    root = range(plan.g_off[0], plan.g_off[1])
    res = opcd.combine_field(edge, paths, root, 1.0, labels=[0, 1, 1, 0])
    pr = g["printed"]
    tol = g["printed_abs_tolerance"]
    assert abs(math.exp(opcd.combine_field(edge, paths, root).logscore[0]) - pr["quoted_true"]) < tol
    assert abs(math.exp(res.logscore[0]) - pr["True_total"]) < tol
    assert abs(math.exp(res.logscore[1]) - pr["quoted_false_plus_bare"]) < tol
    assert abs(res.prob[0] - pr["True_renormalised"]) < tol
    assert res.argmax == 0


def test_quoted_boolean_spelling_sets():
    """The same worked numbers through the plan of a field whose two labels
    are each a set of spellings (bare, quoted): True 0.812 against 0.137,
    renormalised 0.855; the exact value of the printed rounding is
    0.811424 / 0.948656."""
    g = _golden("quoted_boolean_paths.json")
    Q, BF, BT, T, F = 100, 101, 102, 103, 104
    field = pi.Field([7, 8], [[BT], [BF]], spellings=[[[BT], [Q, T]], [[BF], [Q, F]]])
    plan = oplan.build_plan([(20, [field])], 256)
    assert plan.n_readouts == 2 and list(plan.c_spell_off) == [0, 2, 4]
    p_of = {0: {Q: g["root"]["quote"], BF: g["root"]["false"], BT: g["root"]["true"]},
            1: {T: g["after_quote"]["true"], F: g["after_quote"]["false"]}}
    # logits equal to log p and a zero log-sum-exp make every edge exactly log p
    z = np.array([math.log(p_of[r][int(plan.g_tok[gi])]) for r in range(plan.n_readouts)
                  for gi in range(plan.g_off[r], plan.g_off[r + 1])])
    res = opcd.combine(plan, np.zeros(plan.n_readouts), z)[0]
    pr, tol = g["printed"], g["printed_abs_tolerance"]
    assert abs(math.exp(res.logscore[0]) - pr["True_total"]) < tol
    assert abs(math.exp(res.logscore[1]) - pr["quoted_false_plus_bare"]) < tol
    assert abs(res.prob[0] - pr["True_renormalised"]) < tol
    t = 0.868 * 0.868 + 0.058
    f = 0.073 + 0.868 * 0.074
    assert abs(res.prob[0] - t / (t + f)) < 1e-12 and res.argmax == 0
    assert abs(res.mass - (0.868 + 0.073 + 0.058)) < 1e-12


def test_kv_pile_size():
    """Parallel Constrained Decoding from Scratch, "the KV cache": 1,154
    tokens at the Qwen2.5-1.5B shape is about 32 MiB."""
    g = _golden("kv_pile_size.json")
    b = odec.kv_bytes(pi.SHAPES["qwen2.5-1.5b"], g["tokens"])
    assert b == 1154 * 28 * 2 * 2 * 128 * 2
    assert abs(b / 2 ** 20 - g["printed_mib"]) / g["printed_mib"] < g["printed_rel_tolerance"]


# ---------------------------------------------------------------------------
# the decoder against an independent library implementation
# ---------------------------------------------------------------------------

def _hf_model(w):
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers")
    sh = w.shape
    cfg = tr.Qwen2Config(vocab_size=sh.vocab_size, hidden_size=sh.d_model, intermediate_size=sh.ffn_dim,
                         num_hidden_layers=sh.n_layers, num_attention_heads=sh.n_heads,
                         num_key_value_heads=sh.n_kv_heads, head_dim=sh.head_dim, rope_theta=sh.rope_theta,
                         rms_norm_eps=sh.rms_eps, tie_word_embeddings=sh.tied, max_position_embeddings=sh.max_seq,
                         attn_implementation="eager")
    m = tr.Qwen2ForCausalLM(cfg).double().eval()
    sd = {}
    sd["model.embed_tokens.weight"] = torch.from_numpy(w.values("embed").astype(np.float64))
    if not sh.tied:
        sd["lm_head.weight"] = torch.from_numpy(w.values("lm_head").astype(np.float64))
    names = {"wq": "self_attn.q_proj", "wk": "self_attn.k_proj", "wv": "self_attn.v_proj",
             "wo": "self_attn.o_proj", "w_gate": "mlp.gate_proj", "w_up": "mlp.up_proj", "w_down": "mlp.down_proj"}
    with torch.no_grad():
        for l in range(sh.n_layers):
            for ours, theirs in names.items():
                sd[f"model.layers.{l}.{theirs}.weight"] = torch.from_numpy(w.values(f"l{l}.{ours}").astype(np.float64))
            for b in ("q_proj", "k_proj", "v_proj"):   # these models have no biases
                sd[f"model.layers.{l}.self_attn.{b}.bias"] = torch.zeros(getattr(m.model.layers[l].self_attn, b).out_features,
                                                                       dtype=torch.float64)
        missing, _ = m.load_state_dict(sd, strict=False)
        for k in missing:
            assert "norm" in k or (sh.tied and k == "lm_head.weight"), k
    return m


# the library's float32 rotary tables limit agreement to about 1e-7
LIB_ATOL = 1e-6


def _check_against_library(w, seq_len, atol):
    import torch
    m = _hf_model(w)
    dec = odec.Decoder(w, np.float64)
    rng = np.random.default_rng(7)
    toks = rng.integers(0, w.shape.vocab_size, size=seq_len)
    with torch.no_grad():
        ref = m(torch.from_numpy(toks)[None]).logits[0].numpy()
    x, _ = dec.forward(toks, np.arange(seq_len), odec.causal_mask(seq_len))
    ours = dec.logits(x)
    assert np.max(np.abs(ours - ref)) < atol


def test_decoder_matches_library_tiny():
    """The tiny decoder (RMSNorm, rotate-half RoPE base 1e4, GQA 4/2, SwiGLU,
    tied head) equals the transformers Qwen2 model with zero biases.  The
    library builds its rotary cos/sin tables in float32 even in a float64
    model, which bounds the agreement near 1e-7; the tolerance is 1e-6."""
    _check_against_library(pi.make_weights(pi.SHAPES["tiny"], 1000), 40, LIB_ATOL)


@pytest.mark.slow
def test_decoder_matches_library_qwen_widths():
    """Same check at the 1.5B widths (12 Q / 2 KV heads of 128, RoPE base 1e6,
    FFN 8960), one layer, vocabulary cut to 4096 to keep it small."""
    import dataclasses
    sh = dataclasses.replace(pi.SHAPES["qwen2.5-1.5b"], n_layers=1, vocab_size=4096, name="q15-cut")
    _check_against_library(pi.make_weights(sh, 1001), 24, LIB_ATOL)


# ---------------------------------------------------------------------------
# invariants and brute force
# ---------------------------------------------------------------------------

def test_cached_branch_equals_scratch(tiny, cfg0t):
    """Parallel Constrained Decoding from Scratch, "the KV cache": a cached
    prefix is exact for any continuation.  The batched pass over the cached
    prefix equals a from-scratch run of prefix + scaffold + path per node."""
    reqs = _reqs(cfg0t)
    res = opcd.decide(tiny, reqs)
    plan, edge, lse = opcd.scratch_readouts(tiny, reqs)
    ro_of_g = np.repeat(np.arange(res.plan.n_readouts), np.diff(res.plan.g_off))
    assert np.max(np.abs(res.lse - lse)) < 1e-10
    assert np.max(np.abs((res.z - res.lse[ro_of_g]) - edge)) < 1e-10


def test_cached_branch_equals_scratch_random_tries(tiny):
    """Same equality on random deep tries, two requests with different
    prefixes in one batched pass."""
    V = tiny.sh.vocab_size
    rng = np.random.default_rng(11)
    reqs = []
    for k in range(2):
        prefix = [int(t) for t in rng.integers(0, V, size=17 + 9 * k)]
        reqs.append((prefix, pi.random_trie_fields(300 + k, V, 3, max_cands=7, max_len=3)))
    res = opcd.decide(tiny, reqs)
    plan, edge, lse = opcd.scratch_readouts(tiny, reqs)
    ro_of_g = np.repeat(np.arange(res.plan.n_readouts), np.diff(res.plan.g_off))
    assert np.max(np.abs(res.lse - lse)) < 1e-10
    assert np.max(np.abs((res.z - res.lse[ro_of_g]) - edge)) < 1e-10


def test_argmax_equals_bruteforce_greedy(tiny, cfg0):
    """With single-token candidates, the PCD argmax is the constrained greedy
    choice of each field decided on its own from prefix + scaffold."""
    reqs = _reqs(cfg0)
    res = opcd.decide(tiny, reqs)
    prefix = reqs[0][0]
    for f, fr in zip(reqs[0][1], res.fields):
        assert fr.argmax == opcd.greedy_first_token(tiny, prefix, f)


def test_trie_scores_equal_enumeration(tiny, cfg0t):
    """Multi-token candidates sharing a lead token: each candidate's score is
    the sum of from-scratch conditionals up to where it separates."""
    reqs = _reqs(cfg0t)
    res = opcd.decide(tiny, reqs)
    prefix, fields = reqs[0]
    for f, fr in zip(fields, res.fields):
        ref = opcd.enumerate_scores(tiny, prefix, f)
        assert np.max(np.abs(fr.logscore - ref)) < 1e-10


@pytest.mark.parametrize("mode", ["path", "exact", "level", "mean"])
def test_spelling_scores_equal_enumeration(tiny, mode):
    """Labels with several spellings sharing prefixes, under each scoring
    mode: every label's score equals the brute-force enumeration (from-scratch
    conditionals per spelling, no trie), and the cached pass equals
    from-scratch runs at every readout node of the mode's trie."""
    V = tiny.sh.vocab_size
    prefix = [int(t) for t in np.random.default_rng(5).integers(0, V, size=21)]
    fields = pi.random_spelling_fields(71, V, 4, mode=mode)
    assert any(len(lab) > 1 for f in fields for lab in f.spellings)
    res = opcd.decide(tiny, [(prefix, fields)])
    for f, fr in zip(fields, res.fields):
        assert np.max(np.abs(fr.logscore - opcd.enumerate_scores(tiny, prefix, f))) < 1e-10
        assert abs(fr.prob.sum() - 1.0) < 1e-12 and 0.0 < fr.mass <= 1.0
    plan, edge, lse = opcd.scratch_readouts(tiny, [(prefix, fields)])
    ro_of_g = np.repeat(np.arange(res.plan.n_readouts), np.diff(res.plan.g_off))
    assert np.max(np.abs(res.lse - lse)) < 1e-10
    assert np.max(np.abs((res.z - res.lse[ro_of_g]) - edge)) < 1e-10


def test_level_mode_is_a_distribution(tiny):
    """Per-level probabilities multiplied down a trie: every level's child
    probabilities sum to one, so the label probabilities exp(logscore) sum to
    one before any renormalisation, and q equals them at T = 1."""
    V = tiny.sh.vocab_size
    prefix = [int(t) for t in np.random.default_rng(6).integers(0, V, size=15)]
    fields = pi.random_trie_fields(41, V, 4, max_cands=7, max_len=3)
    for f in fields:
        f.mode = "level"
    res = opcd.decide(tiny, [(prefix, fields)])
    for fr in res.fields:
        assert abs(np.exp(fr.logscore).sum() - 1.0) < 1e-12
        assert np.max(np.abs(fr.prob - np.exp(fr.logscore))) < 1e-12


def test_modes_on_single_token_labels(tiny, cfg0):
    """With one token per label, scoring to the end is the path rule, the mean
    divides by one, and the per-level softmax is the subset softmax: every
    mode gives the same q."""
    prefix, fields = _reqs(cfg0)[0]
    base = opcd.decide(tiny, [(prefix, fields)])
    for mode in ("exact", "mean", "level"):
        fm = [pi.Field(f.scaffold, f.candidates, mode=mode) for f in fields]
        res = opcd.decide(tiny, [(prefix, fm)])
        assert res.plan.n_readouts == base.plan.n_readouts
        for a, b in zip(res.fields, base.fields):
            assert np.max(np.abs(a.prob - b.prob)) < 1e-12 and a.argmax == b.argmax
            if mode != "level":
                assert np.max(np.abs(a.logscore - b.logscore)) < 1e-12


def test_exact_mode_scores_every_token(tiny, cfg0t):
    """Exact scoring reads out at every node a label continues from: the
    tiny-trie field's six 3-token IDs get a readout at the lead token and at
    both second-level nodes (the path rule already does), and each label's
    score sums three conditionals; the mean divides it by three."""
    prefix, fields = _reqs(cfg0t)[0]
    f = fields[-1]
    assert all(len(c) == 3 for c in f.candidates)
    ex = opcd.decide(tiny, [(prefix, [pi.Field(f.scaffold, f.candidates, mode="exact")])])
    mn = opcd.decide(tiny, [(prefix, [pi.Field(f.scaffold, f.candidates, mode="mean")])])
    assert np.all(np.diff(ex.plan.s_path_off) == 3)
    assert np.max(np.abs(ex.fields[0].logscore - 3 * mn.fields[0].logscore)) < 1e-12
    ref = [sum(opcd.next_token_logp(tiny, list(prefix) + list(f.scaffold) + c[:i])[c[i]] for i in range(3))
           for c in f.candidates]
    assert np.max(np.abs(ex.fields[0].logscore - np.array(ref))) < 1e-10


def test_greedy_decode_is_the_sequential_argmax(tiny, cfg0):
    """The token-by-token baseline on single-token labels: each field's label
    is the PCD argmax of that field decided after the prefix plus the earlier
    fields' scaffolds and answers, and it writes one token per scaffold token
    and per label token."""
    prefix, fields = _reqs(cfg0)[0]
    labels, out, n = opcd.greedy_decode(tiny, prefix, fields)
    ext = list(prefix)
    for f, lab in zip(fields, labels):
        assert lab == opcd.decide(tiny, [(ext, [f])]).fields[0].argmax
        ext += list(f.scaffold) + list(f.candidates[lab])
    assert out == ext[len(prefix):]
    assert n == sum(len(f.scaffold) + 1 for f in fields)


def _greedy_by_enumeration(dec, prefix, fields):
    """Brute-force reference for the token-by-token decoder on labels of any
    length: for each field in order, every spelling is tested on its own
    against the definition of a greedy constrained choice (at each of its
    tokens, no other spelling agreeing with it so far continues with a token
    of larger from-scratch log-probability, ties to the continuation that
    appears first in declaration order), with the context written so far.
    No token is generated in a loop; exactly one spelling must pass."""
    text = [int(t) for t in prefix]
    labels, out = [], []
    for f in fields:
        ctx = text + [int(t) for t in f.scaffold]
        spells = [(k, [int(t) for t in s]) for k, lab in enumerate(oplan.field_spellings(f)) for s in lab]
        winners = []
        for k, c in spells:
            ok = True
            for i in range(len(c)):
                rivals = []  # next tokens of the spellings that agree with c[:i], first appearance first
                for _, o in spells:
                    if o[:i] == c[:i] and len(o) > i and o[i] not in rivals:
                        rivals.append(o[i])
                if len(rivals) == 1:
                    continue
                lp = opcd.next_token_logp(dec, ctx + c[:i])
                best = max(lp[t] for t in rivals)
                first_best = next(t for t in rivals if lp[t] == best)
                if c[i] != first_best:
                    ok = False
                    break
            if ok:
                winners.append((k, c))
        assert len(winners) == 1, winners
        k, c = winners[0]
        labels.append(k)
        out += [int(t) for t in f.scaffold] + c
        text = ctx + c
    return labels, out


def test_greedy_decode_multitoken_equals_enumeration(tiny, cfg0t):
    """The token-by-token baseline on multi-token labels (the six 3-token IDs
    of cfg0t, random tries, and labels with several spellings): its labels
    and written tokens equal the enumeration above, and its step count is
    the number of tokens it wrote, one decoder pass each ([Scratch], "The
    problem: most of a JSON answer is not an answer")."""
    prefix, fields = _reqs(cfg0t)[0]
    V = tiny.sh.vocab_size
    cases = [fields, pi.random_trie_fields(71, V, 3, max_cands=6, max_len=3),
             pi.random_spelling_fields(72, V, 3, max_labels=3, max_spellings=2, max_len=3)]
    for flds in cases:
        labels, out, n = opcd.greedy_decode(tiny, prefix[:48], flds)
        ref_labels, ref_out = _greedy_by_enumeration(tiny, prefix[:48], flds)
        assert labels == ref_labels
        assert out == ref_out
        assert n == len(ref_out)
        assert any(len(s) > 1 for f in flds for lab in oplan.field_spellings(f) for s in lab)


def test_token_by_token_steps_count_multitoken(tiny, cfg0t):
    """token_by_token_steps on multi-token labels equals the number of
    tokens the token-by-token decoder actually writes when it picks the same
    labels: every scaffold token plus every token of the chosen label (here
    the 3-token IDs of cfg0t)."""
    prefix, fields = _reqs(cfg0t)[0]
    labels, out, n = opcd.greedy_decode(tiny, prefix, fields)
    picked = [opcd.FieldResult(np.zeros(len(f.candidates)), np.zeros(len(f.candidates)), 1.0, lab, 0.0)
              for f, lab in zip(fields, labels)]
    assert opcd.token_by_token_steps([(len(prefix), fields)], picked) == n == len(out)
    assert n == sum(len(f.scaffold) for f in fields) + sum(len(f.candidates[lab]) for f, lab in zip(fields, labels))
    assert max(len(f.candidates[lab]) for f, lab in zip(fields, labels)) == 3


def test_sequenced_rest_sees_the_answers(tiny, cfg0t):
    """The first-field round: the remaining fields' scores equal from-scratch
    conditionals after prefix + the first field's scaffold and chosen
    candidate, and differ from scores taken against the bare prefix."""
    prefix, fields = _reqs(cfg0t)[0]
    first, rest, ext = opcd.decide_sequenced(tiny, prefix, fields, 1)
    f0 = fields[0]
    assert ext == list(prefix) + list(f0.scaffold) + list(f0.candidates[first.fields[0].argmax])
    for f, fr in zip(fields[1:], rest.fields):
        assert np.max(np.abs(fr.logscore - opcd.enumerate_scores(tiny, ext, f))) < 1e-10
    bare = opcd.decide(tiny, [(prefix, fields[1:])])
    assert max(float(np.max(np.abs(a.logscore - b.logscore))) for a, b in zip(rest.fields, bare.fields)) > 1e-6


def test_subset_softmax_identity(tiny, cfg0):
    """First Principles, "The subset softmax is exact": for single-token
    candidates q = p_S / sum(p_S) = p_S / mass, and the argmax does not depend
    on the temperature."""
    reqs = _reqs(cfg0)
    prefix, fields = reqs[0]
    res = opcd.decide(tiny, reqs)
    for f, fr in zip(fields, res.fields):
        lp = opcd.next_token_logp(tiny, list(prefix) + list(f.scaffold))
        p = np.exp(lp[[c[0] for c in f.candidates]])
        assert np.max(np.abs(fr.prob - p / p.sum())) < 1e-12
        assert abs(fr.mass - p.sum()) < 1e-12
        for T in (0.3, 2.0, 7.0):
            r2 = opcd.combine(res.plan, res.lse, res.z, temperature=T)
            assert all(a.argmax == b.argmax for a, b in zip(r2, res.fields))


def test_probabilities_and_mass_bounds(tiny, cfg0t):
    res = opcd.decide(tiny, _reqs(cfg0t))
    for fr in res.fields:
        assert abs(fr.prob.sum() - 1.0) < 1e-12
        assert 0.0 < fr.mass <= 1.0


def test_zero_lm_head_closed_form(cfg0t):
    """With a zero LM head every logit is 0: lse = log V, every candidate of a
    K-way field gets 1/K (all paths have equal length within a field here) and
    the mass is (distinct first tokens) / V."""
    dec = odec.Decoder(pi.make_weights(pi.SHAPES["tiny"], 1000), np.float64)
    dec.zero_head = True
    reqs = _reqs(cfg0t)
    res = opcd.decide(dec, reqs)
    V = dec.sh.vocab_size
    assert np.max(np.abs(res.lse - math.log(V))) < 1e-12
    for f, fr in zip(reqs[0][1], res.fields):
        K = len(f.candidates)
        assert np.max(np.abs(fr.prob - 1.0 / K)) < 1e-12
        assert abs(fr.mass - len({c[0] for c in f.candidates}) / V) < 1e-12


def test_pass_count_and_token_by_token_steps(tiny, cfg0):
    """One prefill plus one batched pass; the token-by-token equivalent is one
    pass per scaffold token and per label token."""
    reqs = _reqs(cfg0)
    res = opcd.decide(tiny, reqs)
    assert res.passes == {"prefill": 1, "branch": 1}
    fields = reqs[0][1]
    assert res.token_by_token_steps == sum(len(f.scaffold) + 1 for f in fields)


def test_cfg1_step_count():
    """The 28-field workload: 1 + 1 passes against one pass per token, about
    300 (Parallel Constrained Decoding from Scratch counts 276 on its real
    schema)."""
    wl = pi.make_workload("cfg1")
    f = wl.requests[0].fields
    steps = sum(len(x.scaffold) + 1 for x in f)
    assert len(f) == 28 and 224 + 28 <= steps <= 336 + 28


# ---------------------------------------------------------------------------
# the plan
# ---------------------------------------------------------------------------

def test_plan_counts_id_field():
    """255 three-token IDs sharing their lead token: readouts = root + the
    lead-token node + 16 second-level nodes; gathers = 1 + 16 + 255."""
    wl = pi.make_workload("cfg2")
    idf = [f for f in wl.requests[0].fields if f.kind == "id"][0]
    plan = oplan.build_plan([(2048, [idf])], wl.shape.vocab_size)
    assert plan.n_readouts == 18 and plan.n_gather == 272
    assert plan.n_branch == len(idf.scaffold) + 17
    plan_all = oplan.build_plan([(2048, wl.requests[0].fields)], wl.shape.vocab_size)
    assert plan_all.n_readouts == 21 and plan_all.n_gather == 278


def test_plan_positions_and_ancestors_bruteforce():
    """Each readout's branch token sits at the position of the last token of
    prefix + scaffold + path, and sees exactly scaffold + path (checked
    against a direct walk over the candidates)."""
    V = 1000
    fields = pi.random_trie_fields(5, V, 6, max_cands=9, max_len=4)
    P = 33
    plan = oplan.build_plan([(P, fields)], V)
    r = 0
    for fi, f in enumerate(fields):
        prefixes = sorted({tuple(c[:i]) for c in f.candidates for i in range(len(c))}, key=lambda p: (len(p), p))
        nodes = [p for p in prefixes
                 if len(p) == 0 or sum(1 for c in f.candidates if tuple(c[:len(p)]) == p) >= 2]
        seen = set()
        for _ in nodes:
            t = int(plan.ro_tok[r])
            anc = plan.anc[plan.anc_off[t]:plan.anc_off[t + 1]]
            seq = [int(plan.tok[a]) for a in anc]
            path = tuple(seq[len(f.scaffold):])
            assert seq[:len(f.scaffold)] == list(f.scaffold)
            assert path in nodes and path not in seen
            seen.add(path)
            assert plan.pos[t] == P + len(f.scaffold) + len(path) - 1
            kids = sorted({c[len(path)] for c in f.candidates if tuple(c[:len(path)]) == path})
            assert sorted(int(x) for x in plan.g_tok[plan.g_off[r]:plan.g_off[r + 1]]) == kids
            r += 1
        assert seen == set(nodes)
    assert r == plan.n_readouts


@pytest.mark.parametrize("bad,code", [
    (pi.Field([], [[1], [2]]), "EMPTY"),
    (pi.Field([3], [[1]]), "NCAND"),
    (pi.Field([3], [[i] for i in range(256)]), "NCAND"),
    (pi.Field([3], [[1], []]), "EMPTY"),
    (pi.Field([3], [[1], [1]]), "DUP"),
    (pi.Field([3], [[1], [1, 2]]), "PREFIX"),
    (pi.Field([3], [[1], [5000]]), "TOKEN"),
    (pi.Field([-1], [[1], [2]]), "TOKEN"),
    (pi.Field([3], [[1], [2]], mode="greedy"), "ARG"),
    (pi.Field([3], [[1], [2]], spellings=[[[1]], []]), "EMPTY"),
    (pi.Field([3], [[1], [2]], spellings=[[[1], [7, 2]], [[2], [7, 2]]]), "DUP"),
    (pi.Field([3], [[1], [2]], spellings=[[[1], [7]], [[2], [7, 2]]]), "PREFIX"),
    (pi.Field([3], [[1], [2]], spellings=[[[1]], [[2]] + [[9, i] for i in range(1023)]]), "NCAND"),
])
def test_plan_rejects(bad, code):
    with pytest.raises(oplan.PlanError) as e:
        oplan.build_plan([(4, [bad])], 1000)
    assert e.value.code == code


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# ---------------------------------------------------------------------------

def _library_pin_fails(dec_cls_patch, monkeypatch):
    for name, fn in dec_cls_patch.items():
        monkeypatch.setattr(odec.Decoder, name, fn)
    with pytest.raises(AssertionError):
        _check_against_library(pi.make_weights(pi.SHAPES["tiny"], 1000), 24, LIB_ATOL)


def test_planted_rope_sign_is_caught(monkeypatch):
    orig = odec.Decoder.rope

    def bad(self, x, positions):
        return orig(self, x, -np.asarray(positions))
    _library_pin_fails({"rope": bad}, monkeypatch)


def test_planted_gqa_mapping_is_caught(monkeypatch):
    def bad(self, q, k_ctx, v_ctx, k_new, v_new, mask):
        # query head h uses KV head h % Hkv instead of h // group
        Hq, Hkv = q.shape[0], k_new.shape[0]
        perm = [(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)]
        out = orig(self, q[perm], k_ctx, v_ctx, k_new, v_new, mask)
        inv = np.argsort(perm)
        return out[inv]
    orig = odec.Decoder.attention
    _library_pin_fails({"attention": bad}, monkeypatch)


def test_planted_rmsnorm_eps_is_caught(monkeypatch):
    def bad(self, x):
        return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-2)
    _library_pin_fails({"rmsnorm": bad}, monkeypatch)


def test_planted_branch_position_is_caught(monkeypatch, tiny, cfg0):
    orig = oplan.build_plan

    def bad(requests, V):
        p = orig(requests, V)
        p.pos = p.pos + 1
        return p
    monkeypatch.setattr(opcd, "build_plan", bad)
    reqs = _reqs(cfg0)
    res = opcd.decide(tiny, reqs)
    monkeypatch.setattr(opcd, "build_plan", orig)
    _, edge, lse = opcd.scratch_readouts(tiny, reqs)
    assert np.max(np.abs(res.lse - lse)) > 1e-6


def test_planted_separation_point_is_caught(monkeypatch, tiny, cfg0t):
    """Scoring one edge too few on multi-token candidates breaks the
    brute-force enumeration pin."""
    orig = opcd.combine_field

    def bad(edge_logp, paths, root_edges, temperature=1.0, labels=None, mean=False):
        return orig(edge_logp, [p[:max(1, len(p) - 1)] for p in paths], root_edges, temperature, labels, mean)
    monkeypatch.setattr(opcd, "combine_field", bad)
    reqs = _reqs(cfg0t)
    res = opcd.decide(tiny, reqs)
    prefix, fields = reqs[0]
    f, fr = fields[-1], res.fields[-1]
    assert np.max(np.abs(fr.logscore - opcd.enumerate_scores(tiny, prefix, f))) > 1e-6


def test_planted_spelling_max_is_caught(monkeypatch):
    """Taking a label's best spelling instead of the sum of its spellings
    breaks the quoted-boolean worked numbers."""
    orig = opcd.combine_field

    def bad(edge_logp, paths, root_edges, temperature=1.0, labels=None, mean=False):
        if labels is None:
            return orig(edge_logp, paths, root_edges, temperature, None, mean)
        best = {}
        for c, k in enumerate(labels):
            sc = sum(edge_logp[g] for g in paths[c])
            if k not in best or sc > best[k][0]:
                best[k] = (sc, c)
        keep = sorted(c for _, c in best.values())
        return orig(edge_logp, [paths[c] for c in keep], root_edges, temperature, None, mean)
    monkeypatch.setattr(opcd, "combine_field", bad)
    with pytest.raises(AssertionError):
        test_quoted_boolean_spelling_sets()


def test_planted_level_normaliser_is_caught(monkeypatch, tiny):
    """Normalising a level over the full vocabulary instead of its child
    tokens breaks the level-mode distribution pin."""
    orig = opcd.combine

    def bad(plan, lse, z, temperature=1.0):
        plan.f_mode = np.zeros_like(plan.f_mode)
        return orig(plan, lse, z, temperature)
    monkeypatch.setattr(opcd, "combine", bad)
    with pytest.raises(AssertionError):
        test_level_mode_is_a_distribution(tiny)

