"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case runs the same seeded inputs through the library (libpcd.so on
cuda:0) and through the fp64 oracle, and compares readout log-sum-exps,
gathered candidate logits, candidate log-scores and probabilities, candidate
mass and argmax.  Integer work (the plan) is checked bit-exactly on the CPU
(test_host.py); here the plan's effect is checked through the outputs.

Tolerances (GPU minus fp64 oracle on the same weights), from
tests/tolerances.py:
  fp32 model:  lse, z, logscore <= 1e-4 abs;  prob <= 1e-5 abs;  mass <= 1e-4 rel
  bf16 models at 2 layers: lse, z <= 2.5e-2 abs; logscore <= 2.6e-2 x path
               length; prob <= 1.3e-2 abs; mass <= 2.6e-2 rel
  argmax equal unless the oracle's top-2 margin is under the waiver: 2 z for
  single-token fields (0.05 nats in bf16: two logits each off by 2.5e-2 can
  swap at most that margin), 2 ls per token of the field's deepest path.
The bf16 bounds come from rounding the GEMM inputs (normalised activations,
attention probabilities and outputs, SwiGLU outputs) and the KV cache to
bf16, a relative error of 2^-9 per element; test_bf16_bound.py relates them
to a model of those rounding points.
"""
import dataclasses

import numpy as np
import pytest

import pcd_inputs as pi
from oracle import decoder as odec
from oracle import pcd as opcd
import tolerances as tl

cpd = pytest.importorskip("constrained_decoding_pcd_amd")
torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = {"f32": tl.F32, "bf16": tl.BF16_L2}


def _model(shape, weights, requests, max_prefill=0):
    dev = cpd.upload_weights(weights.mats, shape.n_layers, shape.d_model, "cuda:0")
    lens = [len(p) for p, _ in requests]
    lim = cpd.limits_for(shape.vocab_size, shape.max_seq, lens, [f for _, f in requests], max_prefill)
    return cpd.PcdModel(cpd.config_of(shape), dev, lim)


def cand_depth(plan) -> np.ndarray:
    """Per candidate, the longest scored path over its spellings."""
    slen = np.diff(plan.s_path_off)
    return np.array([slen[plan.c_spell_off[c]:plan.c_spell_off[c + 1]].max()
                     for c in range(len(plan.c_spell_off) - 1)])


def field_depth(plan) -> np.ndarray:
    """Per field, the longest scored path of its candidates."""
    cd = cand_depth(plan)
    return np.array([cd[plan.f_cand_off[f]:plan.f_cand_off[f + 1]].max() for f in range(len(plan.f_cand_off) - 1)])


def check_argmax(arg, ref_fields, plan, bounds, name=""):
    """The argmax must equal the oracle's wherever the oracle's top-2 margin
    is at least the field's waiver."""
    for i, (a, f, dep) in enumerate(zip(arg, ref_fields, field_depth(plan))):
        if f.margin >= tl.margin_waiver(bounds, int(dep)):
            assert int(a) == f.argmax, (name, i, f.margin)


def _compare(name, got, ref, plan, dtype, label=""):
    """got: list of per-request dicts from the library; ref: oracle result;
    plan: the oracle's plan (for the candidates' path lengths)."""
    tol = TOL[dtype]
    lse = np.concatenate([g["lse"] for g in got])
    z = np.concatenate([g["z"] for g in got])
    prob = np.concatenate([g["prob"] for g in got])
    ls = np.concatenate([g["logscore"] for g in got])
    mass = np.concatenate([g["mass"] for g in got])
    arg = np.concatenate([g["argmax"] for g in got])
    rprob = np.concatenate([f.prob for f in ref.fields])
    rls = np.concatenate([f.logscore for f in ref.fields])
    rmass = np.array([f.mass for f in ref.fields])
    plen = cand_depth(plan)
    d = {
        "lse": float(np.max(np.abs(lse - ref.lse))),
        "z": float(np.max(np.abs(z - ref.z))),
        "ls/len": float(np.max(np.abs(ls - rls) / plen)),
        "prob": float(np.max(np.abs(prob - rprob))),
        "mass_rel": float(np.max(np.abs(mass - rmass) / rmass)),
    }
    print(f"[{name}{label}] max errors: " + ", ".join(f"{k} {v:.3e}" for k, v in d.items()), flush=True)
    assert d["lse"] <= tol.get("lse", tol["z"]) and d["z"] <= tol["z"]
    assert d["ls/len"] <= tol["ls"]
    assert d["prob"] <= tol["prob"]
    assert d["mass_rel"] <= tol["mass"]
    check_argmax(arg, ref.fields, plan, tol, name)
    # invariants of every field
    off = 0
    for g in got:
        assert np.all(g["mass"] <= 1.0 + 1e-6) and np.all(g["mass"] > 0)
    for f in ref.fields:
        k = len(f.prob)
        assert abs(float(prob[off:off + k].sum()) - 1.0) <= 1e-6
        off += k


def _run_case(name, shape, weights, requests, temperature=1.0, dec=None):
    print(f"case {name}: {len(requests)} request(s), prefixes {[len(p) for p, _ in requests]}", flush=True)
    m = _model(shape, weights, requests)
    states = [m.prefill(p) for p, _ in requests]
    got = m.decide_many(states, [f for _, f in requests], temperature, debug=True)
    dec = dec or odec.Decoder(weights, np.float64)
    ref = opcd.decide(dec, requests, temperature)
    _compare(name, got, ref, ref.plan, shape.dtype)
    for s in states:
        s.close()
    m.close()
    return got, ref


@pytest.fixture(scope="module")
def tiny_w():
    return pi.make_weights(pi.SHAPES["tiny"], 1000)


@pytest.fixture(scope="module")
def tiny_dec(tiny_w):
    return odec.Decoder(tiny_w, np.float64)


def _reqs(wl):
    return [(r.prefix, r.fields) for r in wl.requests]


def test_tiny_cfg0(tiny_w, tiny_dec):
    wl = pi.make_workload("cfg0")
    _run_case("cfg0", wl.shape, tiny_w, _reqs(wl), dec=tiny_dec)


def test_tiny_cfg0_trie(tiny_w, tiny_dec):
    wl = pi.make_workload("cfg0t")
    _run_case("cfg0t", wl.shape, tiny_w, _reqs(wl), dec=tiny_dec)


@pytest.mark.parametrize("temperature", [0.5, 2.0])
def test_tiny_temperature(tiny_w, tiny_dec, temperature):
    wl = pi.make_workload("cfg0t")
    _run_case(f"cfg0t-T{temperature}", wl.shape, tiny_w, _reqs(wl), temperature, dec=tiny_dec)


def test_tiny_ragged_multi_request_deep_tries(tiny_w, tiny_dec):
    """Three requests in one branch pass, prefixes of 1, 65 and 130 tokens
    (below, above and across the 64-key tile), deep random tries."""
    V = pi.SHAPES["tiny"].vocab_size
    rng = np.random.default_rng(5)
    reqs = []
    for k, P in enumerate((1, 65, 130)):
        prefix = [int(t) for t in rng.integers(0, V, size=P)]
        reqs.append((prefix, pi.random_trie_fields(700 + k, V, 4, max_cands=12, max_len=4)))
    _run_case("tiny-multi", pi.SHAPES["tiny"], tiny_w, reqs, dec=tiny_dec)


def _deep_chain_fields(seed, V):
    """Two fields whose candidates share long lead runs, so trie tokens sit 11
    and 15 levels below the scaffold: their visibility chains run past the 8
    links held in registers and continue through the parent links."""
    rng = np.random.default_rng(seed)
    tok = lambda n: [int(t) for t in rng.choice(V, size=n, replace=False)]
    b, x = tok(10), tok(8)
    a = pi.Field(tok(4), [b + [x[0]], b + [x[1], x[2]], b + [x[3], x[4], x[5]], [x[6]]], kind="trie")
    d, z = tok(14), tok(3)
    f = pi.Field(tok(3), [d + [z[0]], d + [z[1]], d[:6] + [z[2]]], kind="trie")
    return [a, f]


def test_tiny_deep_chains(tiny_w, tiny_dec):
    """Trie chains deeper than 8 links, three requests (prefixes 3, 64, 100)."""
    V = pi.SHAPES["tiny"].vocab_size
    rng = np.random.default_rng(9)
    reqs = []
    for k, P in enumerate((3, 64, 100)):
        prefix = [int(t) for t in rng.integers(0, V, size=P)]
        reqs.append((prefix, _deep_chain_fields(900 + k, V) + pi.random_trie_fields(910 + k, V, 2)))
    _run_case("tiny-deep", pi.SHAPES["tiny"], tiny_w, reqs, dec=tiny_dec)


@pytest.mark.parametrize("mode", ["path", "exact", "level", "mean"])
def test_tiny_spellings_and_modes(tiny_w, tiny_dec, mode):
    """Labels with up to four spellings sharing prefixes, plus deep tries,
    under each scoring mode; two requests (prefixes 9 and 70) in one pass."""
    V = pi.SHAPES["tiny"].vocab_size
    rng = np.random.default_rng(13)
    reqs = []
    for k, P in enumerate((9, 70)):
        prefix = [int(t) for t in rng.integers(0, V, size=P)]
        fields = pi.random_spelling_fields(1300 + k, V, 4, max_labels=6, max_spellings=4, max_len=4, mode=mode)
        fields += pi.random_trie_fields(1400 + k, V, 2, max_cands=9, max_len=4)
        for f in fields[-2:]:
            f.mode = mode
        reqs.append((prefix, fields))
    _run_case(f"tiny-spell-{mode}", pi.SHAPES["tiny"], tiny_w, reqs, dec=tiny_dec)


def test_tiny_mixed_modes_one_request(tiny_w, tiny_dec):
    """Fields of one request each in its own mode, labels with spellings,
    at temperature 0.7."""
    V = pi.SHAPES["tiny"].vocab_size
    prefix = [int(t) for t in np.random.default_rng(14).integers(0, V, size=40)]
    fields = []
    for i, mode in enumerate(("path", "exact", "level", "mean", "exact", "level")):
        fields += pi.random_spelling_fields(1500 + i, V, 1, max_labels=5, max_spellings=3, max_len=3, mode=mode)
    _run_case("tiny-mixed-modes", pi.SHAPES["tiny"], tiny_w, [(prefix, fields)], 0.7, dec=tiny_dec)


def test_tiny_prefill_many(tiny_w, tiny_dec):
    """Three prompts (1, 64 and 130 tokens: below, at and across the 64-key
    tile) prefilled in one pass: each state's KV equals the oracle's prefill
    of that prompt alone, and one branch pass over the three states decides
    as the oracle does."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(17)
    reqs = []
    for k, P in enumerate((1, 64, 130)):
        prefix = [int(t) for t in rng.integers(0, sh.vocab_size, size=P)]
        reqs.append((prefix, pi.random_trie_fields(1100 + k, sh.vocab_size, 3)))
    m = _model(sh, tiny_w, reqs, max_prefill=sum(len(p) for p, _ in reqs))
    states = m.prefill_many([p for p, _ in reqs])
    for st, (prefix, _) in zip(states, reqs):
        assert st.n_tokens == len(prefix)
        kv = st.kv.view(torch.float32).cpu().numpy().reshape(sh.n_layers, 2, sh.n_kv_heads, len(prefix), sh.head_dim)
        ref = opcd.prefill(tiny_dec, prefix)
        err = max(float(np.max(np.abs(kv[l, i] - ref[l][i]))) for l in range(sh.n_layers) for i in range(2))
        print(f"[prefill-many] P={len(prefix)} KV max abs error {err:.3e}", flush=True)
        assert err < 1e-4
    got = m.decide_many(states, [f for _, f in reqs], debug=True)
    ref = opcd.decide(tiny_dec, reqs)
    _compare("tiny-prefill-many", got, ref, ref.plan, "f32")
    assert m.stats()["prefill_passes"] == 1
    for st in states:
        st.close()
    m.close()


def test_tiny_prefill_many_errors(tiny_w):
    """Rejected before any device work: shared buffer memory, too many tokens,
    a token outside the vocabulary, an empty sequence."""
    sh = pi.SHAPES["tiny"]
    fields = pi.make_workload("cfg0").requests[0].fields
    m = _model(sh, tiny_w, [([1] * 10, fields), ([2] * 10, fields)], max_prefill=20)
    one = torch.empty(m.state_bytes(20), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(cpd.PcdError) as e:
        m.prefill_many([[1] * 10, [2] * 10], kvs=[one, one])
    assert e.value.name == "ARG"
    with pytest.raises(cpd.PcdError) as e:
        m.prefill_many([[1] * 12, [2] * 10])
    assert e.value.name == "CAP"
    with pytest.raises(cpd.PcdError) as e:
        m.prefill_many([[1] * 10, [2, sh.vocab_size]])
    assert e.value.name == "TOKEN"
    with pytest.raises(cpd.PcdError) as e:
        m.prefill_many([[1] * 10, []])
    assert e.value.name == "ARG"
    sts = m.prefill_many([[1] * 10, [2] * 10])
    assert [s.n_tokens for s in sts] == [10, 10]
    for s in sts:
        s.close()
    m.close()


def test_tiny_prefill_kv(tiny_w, tiny_dec):
    """The state's KV buffer holds every layer's K (after RoPE) and V of the
    prefix, [layer][K|V][kv head][token][head_dim]."""
    sh = pi.SHAPES["tiny"]
    wl = pi.make_workload("cfg0")
    prefix = wl.requests[0].prefix
    m = _model(sh, tiny_w, _reqs(wl))
    st = m.prefill(prefix)
    kv = st.kv.view(torch.float32).cpu().numpy().reshape(sh.n_layers, 2, sh.n_kv_heads, len(prefix), sh.head_dim)
    ref = opcd.prefill(tiny_dec, prefix)
    err = max(float(np.max(np.abs(kv[l, i] - ref[l][i]))) for l in range(sh.n_layers) for i in range(2))
    print(f"[prefill-kv] max abs error {err:.3e}", flush=True)
    assert err < 1e-4
    st.close()
    m.close()


def test_tiny_invariants(tiny_w):
    """One prefill + one branch pass per request; decide never writes the
    state's KV; results are bit-identical from run to run."""
    wl = pi.make_workload("cfg0t")
    reqs = _reqs(wl)
    m = _model(wl.shape, tiny_w, reqs)
    st = m.prefill(reqs[0][0])
    kv0 = st.kv.clone()
    a = m.decide(st, reqs[0][1], debug=True)
    b = m.decide(st, reqs[0][1], debug=True)
    assert torch.equal(kv0, st.kv)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    s = m.stats()
    assert s["prefill_passes"] == 1 and s["branch_passes"] == 2
    plan = cpd.debug_plan(wl.shape.vocab_size, wl.shape.max_seq, [len(reqs[0][0])], [reqs[0][1]])
    assert s["last_branch_tokens"] == len(plan["tok"]) and s["last_readouts"] == len(plan["ro_tok"])
    st.close()
    m.close()


def test_tiny_errors_before_device_work(tiny_w):
    wl = pi.make_workload("cfg0")
    reqs = _reqs(wl)
    m = _model(wl.shape, tiny_w, reqs)
    st = m.prefill(reqs[0][0])
    bad = [pi.Field([1, 2], [[3], [3]])]
    with pytest.raises(cpd.PcdError) as e:
        m.decide(st, bad)
    assert e.value.name == "DUP"
    with pytest.raises(cpd.PcdError) as e:
        m.prefill([0, 1, 99999])
    assert e.value.name == "TOKEN"
    with pytest.raises(cpd.PcdError) as e:
        m.decide(st, reqs[0][1], temperature=0.0)
    assert e.value.name == "ARG"
    # the model still works after rejected calls
    got = m.decide(st, reqs[0][1])
    assert np.all(np.isfinite(got["prob"]))
    st.close()
    m.close()


# ---------------------------------------------------------------------------
# bf16 at head dims 32 and 64 (the bf16 workloads all use 128)
# ---------------------------------------------------------------------------

def _small_bf16_shape(hd):
    """The tiny widths (d 128, FFN 384, vocabulary 2048) in bf16 with 32- or
    64-wide heads (4 query / 2 KV heads, or 2 / 1), room for 8,448 tokens."""
    heads = {32: (4, 2), 64: (2, 1)}[hd]
    return dataclasses.replace(pi.SHAPES["tiny"], name=f"tiny-bf16-hd{hd}", dtype="bf16", head_dim=hd,
                               n_heads=heads[0], n_kv_heads=heads[1], max_seq=8448)


@pytest.mark.parametrize("hd", [32, 64])
def test_bf16_small_head_dims(hd):
    """The attention kernel's 32- and 64-wide instances and the GEMM tiles at
    width 128 in bf16.  Three ragged requests with deep tries in one branch
    pass (launches of a few blocks: two key chains per workgroup), then one
    long prefix whose prefill launch has more than 256 row blocks (4-wave
    blocks) and whose branch rows split their keys over workgroups."""
    sh = _small_bf16_shape(hd)
    w = pi.make_weights(sh, 1003)
    dec = odec.Decoder(w, np.float64)
    V = sh.vocab_size
    rng = np.random.default_rng(40 + hd)
    reqs = []
    for k, P in enumerate((1, 65, 130)):
        prefix = [int(t) for t in rng.integers(0, V, size=P)]
        reqs.append((prefix, pi.random_trie_fields(4000 + k, V, 3, max_cands=8, max_len=3)))
    _run_case(f"bf16-hd{hd}-multi", sh, w, reqs, dec=dec)
    # row blocks of the prefill: tokens x (query heads per KV head) / 64 x KV heads > 256
    P = {32: 4200, 64: 8300}[hd]
    assert P * (sh.n_heads // sh.n_kv_heads) // 64 * sh.n_kv_heads > 256
    prefix = [int(t) for t in rng.integers(0, V, size=P)]
    _run_case(f"bf16-hd{hd}-long", sh, w, [(prefix, pi.random_trie_fields(4100, V, 3, max_cands=6, max_len=3))],
              dec=dec)


def _wide_bf16_shape(hd):
    """The tiny widths in bf16 with many heads in pairs (32 query / 16 KV
    heads of 32, or 16 / 8 of 64): causal prefill launches reach 512 row
    blocks of 128 rows at a few thousand tokens."""
    heads = {32: (32, 16), 64: (16, 8)}[hd]
    return dataclasses.replace(pi.SHAPES["tiny"], name=f"tiny-bf16-wide-hd{hd}", dtype="bf16", head_dim=hd,
                               n_heads=heads[0], n_kv_heads=heads[1], max_seq=4608)


@pytest.mark.parametrize("hd", [32, 64])
def test_bf16_wide_prefill_attention_blocks(hd):
    """Causal prefill whose launch has at least 512 blocks of 128 query rows:
    those blocks give each wave two 16-row groups, the query rows wait in
    the key ring's second slot, and the last block of each KV head is
    ragged.  One long prompt (pcd_prefill), then two prompts in one
    pcd_prefill_many pass, each decided against the oracle."""
    sh = _wide_bf16_shape(hd)
    grp, hkv = sh.n_heads // sh.n_kv_heads, sh.n_kv_heads
    w = pi.make_weights(sh, 1005)
    dec = odec.Decoder(w, np.float64)
    V = sh.vocab_size
    rng = np.random.default_rng(70 + hd)
    P = {32: 2100, 64: 4100}[hd]
    assert hkv * -(-P * grp // 128) >= 512 and (P * grp) % 128 != 0
    prefix = [int(t) for t in rng.integers(0, V, size=P)]
    _run_case(f"bf16-wide-hd{hd}-one", sh, w, [(prefix, pi.random_trie_fields(4200, V, 3, max_cands=6, max_len=3))],
              dec=dec)
    lens = {32: (1100, 1061), 64: (2050, 2029)}[hd]
    assert hkv * sum(-(-n * grp // 128) for n in lens) >= 512
    reqs = [([int(t) for t in rng.integers(0, V, size=n)], pi.random_trie_fields(4300 + k, V, 2, max_cands=5, max_len=2))
            for k, n in enumerate(lens)]
    m = _model(sh, w, reqs, max_prefill=sum(lens))
    states = m.prefill_many([p for p, _ in reqs])
    got = m.decide_many(states, [f for _, f in reqs], debug=True)
    ref = opcd.decide(dec, reqs)
    _compare(f"bf16-wide-hd{hd}-many", got, ref, ref.plan, "bf16")
    for st in states:
        st.close()
    m.close()


# ---------------------------------------------------------------------------
# Qwen2.5-1.5B widths in bf16
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def q15_l2():
    sh = pi.SHAPES["qwen2.5-1.5b"]
    w = pi.make_weights(sh, 1001, n_layers=2)
    return w.shape, w, odec.Decoder(w, np.float64)


def test_bf16_two_layer_cfg1(q15_l2):
    """The 28-field workload (512-token prefix) on the first 2 layers of the
    1.5B-shaped model: every output of every field."""
    sh, w, dec = q15_l2
    _run_case("q15-L2-cfg1", sh, w, _reqs(pi.make_workload("cfg1")), dec=dec)


def test_bf16_two_layer_spellings_and_modes(q15_l2):
    """The 1.5B widths in bf16: the cfg1 prefix with fields whose labels have
    several spellings, one field group per scoring mode, in one pass."""
    sh, w, dec = q15_l2
    wl = pi.make_workload("cfg1")
    prefix = wl.requests[0].prefix
    fields = []
    for i, mode in enumerate(("path", "exact", "level", "mean")):
        fields += pi.random_spelling_fields(1600 + i, sh.vocab_size, 3, max_labels=8, max_spellings=3,
                                            max_len=3, mode=mode)
    _run_case("q15-L2-spell", sh, w, [(prefix, fields)], dec=dec)


def test_bf16_two_layer_prefill_many(q15_l2):
    """Four prompts of the throughput workload (1024 tokens each) prefilled in
    one pass at the 1.5B widths, then one branch pass over the four states."""
    sh, w, dec = q15_l2
    reqs = _reqs(pi.make_workload("cfg3"))[:4]
    m = _model(sh, w, reqs, max_prefill=sum(len(p) for p, _ in reqs))
    states = m.prefill_many([p for p, _ in reqs])
    got = m.decide_many(states, [f for _, f in reqs], debug=True)
    ref = opcd.decide(dec, reqs)
    _compare("q15-L2-prefill-many", got, ref, ref.plan, "bf16")
    for st in states:
        st.close()
    m.close()


def test_bf16_two_layer_large_prefill_tiles(q15_l2):
    """Ten prompts of the throughput workload, the last one token longer
    (10,241 rows), in one prefill pass: at this row count the residual GEMMs
    take 256x256 tiles and gate/up 256-row tiles, the last row tile holding
    one row.  The first, a middle and the last prompt's states are then
    decided against the oracle (rows at the start, middle and end of the
    pass)."""
    sh, w, dec = q15_l2
    reqs = _reqs(pi.make_workload("cfg3"))[:10]
    reqs[9] = (list(reqs[9][0]) + [7], reqs[9][1])
    m = _model(sh, w, reqs, max_prefill=sum(len(p) for p, _ in reqs))
    states = m.prefill_many([p for p, _ in reqs])
    pick = [0, 5, 9]
    got = m.decide_many([states[i] for i in pick], [reqs[i][1] for i in pick], debug=True)
    ref = opcd.decide(dec, [reqs[i] for i in pick])
    _compare("q15-L2-prefill-10241", got, ref, ref.plan, "bf16")
    for st in states:
        st.close()
    m.close()


def test_bf16_two_layer_prefill_past_tile_switch(q15_l2):
    """A 1,025-token prompt: one row past the count where the GEMMs switch
    to their large-row tiles, so the last 128- and 256-row tiles hold a
    single row; then the 28-field decide."""
    sh, w, dec = q15_l2
    wl = pi.make_workload("cfg3")
    prefix = list(wl.requests[1].prefix) + [11]
    _run_case("q15-L2-prefill-1025", sh, w, [(prefix, wl.requests[1].fields)], dec=dec)


def test_bf16_two_layer_wide_readout_tiles(q15_l2):
    """1,100 fields with one-token labels after a 32-token prefix: 1,100
    readout rows, above which the LM-head GEMM takes 128x256 tiles, the last
    one ragged at the 151,936-token vocabulary."""
    sh, w, dec = q15_l2
    prefix = [int(t) for t in np.random.default_rng(12).integers(0, sh.vocab_size, size=32)]
    fields = pi.random_trie_fields(1700, sh.vocab_size, 1100, max_cands=3, max_len=1, scaffold_len=(1, 2))
    got, ref = _run_case("q15-L2-readout-1100", sh, w, [(prefix, fields)], dec=dec)
    assert len(ref.plan.ro_tok) > 1024


def test_bf16_two_layer_cfg2_id_field(q15_l2):
    """2048-token prefix; 3 booleans and one 255-option 3-token ID field whose
    options share their lead token (18 trie readouts)."""
    sh, w, dec = q15_l2
    _run_case("q15-L2-cfg2", sh, w, _reqs(pi.make_workload("cfg2")), dec=dec)


def test_bf16_two_layer_batched_requests(q15_l2):
    """Four requests of the throughput workload (1024-token prefixes, 28
    fields each) in one branch pass."""
    sh, w, dec = q15_l2
    wl = pi.make_workload("cfg3")
    _run_case("q15-L2-cfg3x4", sh, w, [(r.prefix, r.fields) for r in wl.requests[:4]], dec=dec)


def test_bf16_two_layer_deep_chains(q15_l2):
    """Trie chains deeper than 8 links at the 1.5B widths (head_dim 128),
    three requests with prefixes of 1, 65 and 130 tokens in one branch pass."""
    sh, w, dec = q15_l2
    rng = np.random.default_rng(11)
    reqs = []
    for k, P in enumerate((1, 65, 130)):
        prefix = [int(t) for t in rng.integers(0, sh.vocab_size, size=P)]
        reqs.append((prefix, _deep_chain_fields(920 + k, sh.vocab_size) +
                     pi.random_trie_fields(930 + k, sh.vocab_size, 2, max_len=6)))
    _run_case("q15-L2-deep", sh, w, reqs, dec=dec)


def test_tiny_compiled_fields_match_lists(tiny_w):
    """Every decide path gives bit-identical results whether it is handed the
    field list or the same schema marshalled once."""
    V = pi.SHAPES["tiny"].vocab_size
    rng = np.random.default_rng(77)
    prefix = [int(t) for t in rng.integers(0, V, size=50)]
    fields = pi.random_spelling_fields(7700, V, 3, max_labels=5, max_spellings=3, max_len=3, mode="exact")
    fields += pi.random_trie_fields(7701, V, 2, max_cands=8, max_len=3)
    print("case tiny-compiled: prefix 50", flush=True)
    sh = pi.SHAPES["tiny"]
    cap = len(prefix) + len(fields[0].scaffold) + max(len(c) for c in fields[0].candidates)
    dev = cpd.upload_weights(tiny_w.mats, sh.n_layers, sh.d_model, "cuda:0")
    lim = cpd.limits_for(sh.vocab_size, sh.max_seq, [cap, cap], [fields, fields], cap + 64)
    m = cpd.PcdModel(cpd.config_of(sh), dev, lim)
    comp = m.compile_fields(fields)
    keys = ("prob", "logscore", "mass", "margin", "argmax")

    def same(a, b):
        for k in keys:
            assert np.array_equal(a[k], b[k]), k

    st = m.prefill(prefix)
    same(m.decide(st, fields), m.decide(st, comp))
    same(m.decide_many([st, st], [fields, fields])[1], m.decide_many([st, st], [comp, fields])[0])
    outs = []
    for f in (fields, comp):
        s2 = st.fork(capacity=cap)
        outs.append(m.decide_sequenced(s2, f, 1))
        s2.close()
    same(*outs)
    outs = []
    for f in (fields, comp):
        s3 = m.new_state(len(prefix))
        outs.append(m.extend_decide(s3, prefix, f))
        s3.close()
    same(*outs)
    st.close()
    m.close()
