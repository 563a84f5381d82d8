"""GPU parity of growing a state through the C ABI against the fp64 oracle:
pcd_extend (a causal pass over new tokens after the cached ones), pcd_fork
(one cached prompt head, many requests) and pcd_decide_sequenced (the
first-field round: decide the first field, write its answer in, decide the
rest).  An extended state must equal a prefill of the concatenated tokens;
tolerances as in test_gpu_parity.py.
"""
import numpy as np
import pytest

import pcd_inputs as pi
from oracle import decoder as odec
from oracle import pcd as opcd
import tolerances as tl
from test_gpu_parity import TOL, _compare

cpd = pytest.importorskip("constrained_decoding_pcd_amd")
torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny_w():
    return pi.make_weights(pi.SHAPES["tiny"], 1000)


@pytest.fixture(scope="module")
def tiny_dec(tiny_w):
    return odec.Decoder(tiny_w, np.float64)


def _model(shape, weights, lens, requests, max_prefill):
    dev = cpd.upload_weights(weights.mats, shape.n_layers, shape.d_model, "cuda:0")
    lim = cpd.limits_for(shape.vocab_size, shape.max_seq, lens, requests, max_prefill)
    return cpd.PcdModel(cpd.config_of(shape), dev, lim)


def _kv(state, shape, cap, np_dtype):
    a = state.kv.view(torch.float32 if np_dtype == np.float32 else torch.int16).cpu().numpy()
    return a.reshape(shape.n_layers, 2, shape.n_kv_heads, cap, shape.head_dim)[:, :, :, :state.n_tokens]


def _tokens(rng, V, n):
    return [int(t) for t in rng.integers(0, V, size=n)]


def _compare_fields(name, got, ref_fields, dtype, fields):
    """Per-candidate probabilities and log-scores, per-field mass and argmax
    (fields: the request's fields, for each one's longest spelling)."""
    tol = TOL[dtype]
    prob = np.concatenate([f.prob for f in ref_fields])
    ls = np.concatenate([f.logscore for f in ref_fields])
    mass = np.array([f.mass for f in ref_fields])
    d = {"prob": float(np.max(np.abs(got["prob"] - prob))), "ls": float(np.max(np.abs(got["logscore"] - ls))),
         "mass_rel": float(np.max(np.abs(got["mass"] - mass) / mass))}
    print(f"[{name}] max errors: " + ", ".join(f"{k} {v:.3e}" for k, v in d.items()), flush=True)
    # log-scores sum at most 4 conditionals here (trie depth of the workloads)
    assert d["prob"] <= tol["prob"] and d["mass_rel"] <= tol["mass"] and d["ls"] <= tol["ls"] * 4
    for i, (f, fd) in enumerate(zip(ref_fields, fields)):
        depth = max(len(s) for lab in (fd.spellings or [[c] for c in fd.candidates]) for s in lab)
        if f.margin >= tl.margin_waiver(tol, depth):
            assert int(got["argmax"][i]) == f.argmax, (name, i, f.margin)


def test_tiny_extend_kv_matches_prefill(tiny_w, tiny_dec):
    """prefill(A) + extend(B) + extend(C) leaves the KV of prefill(A+B+C);
    the pieces (50, 30, 70 tokens) straddle the 64-key tiles."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(21)
    A, B, C = _tokens(rng, sh.vocab_size, 50), _tokens(rng, sh.vocab_size, 30), _tokens(rng, sh.vocab_size, 70)
    fields = pi.make_workload("cfg0").requests[0].fields
    m = _model(sh, tiny_w, [150], [fields], 70)
    st = m.prefill(A, capacity=150)
    st.extend(B)
    st.extend(C)
    assert st.n_tokens == 150
    kv = _kv(st, sh, 150, np.float32)
    ref = opcd.prefill(tiny_dec, A + B + C)
    err = max(float(np.max(np.abs(kv[l, i] - ref[l][i]))) for l in range(sh.n_layers) for i in range(2))
    print(f"[extend-kv] max abs error {err:.3e}", flush=True)
    assert err < 1e-4
    assert m.stats()["prefill_passes"] == 3
    # decide against the grown state equals decide against the concatenation
    got = [m.decide(st, fields, debug=True)]
    ref = opcd.decide(tiny_dec, [(A + B + C, fields)])
    _compare("tiny-extend", got, ref, ref.plan, "f32")
    st.close()
    m.close()


def test_tiny_fork_serves_two_requests(tiny_w, tiny_dec):
    """One cached head (60 tokens) forked twice and extended by two different
    inputs (20 and 45 tokens): each equals its own concatenation, and the
    head's KV is untouched."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(22)
    head = _tokens(rng, sh.vocab_size, 60)
    inputs = [_tokens(rng, sh.vocab_size, 20), _tokens(rng, sh.vocab_size, 45)]
    fields = pi.make_workload("cfg0t").requests[0].fields
    m = _model(sh, tiny_w, [105], [fields], 60)
    hs = m.prefill(head)
    kv0 = hs.kv.clone()
    for k, inp in enumerate(inputs):
        st = hs.fork(capacity=len(head) + len(inp))
        st.extend(inp)
        got = [m.decide(st, fields, debug=True)]
        ref = opcd.decide(tiny_dec, [(head + inp, fields)])
        _compare(f"tiny-fork{k}", got, ref, ref.plan, "f32")
        st.close()
    assert torch.equal(kv0, hs.kv) and hs.n_tokens == len(head)
    hs.close()
    m.close()


def test_tiny_first_field_round(tiny_w, tiny_dec):
    """pcd_decide_sequenced: field 0 decided, its scaffold and chosen
    candidate appended, the other fields decided against that."""
    sh = pi.SHAPES["tiny"]
    wl = pi.make_workload("cfg0t")
    prefix, fields = wl.requests[0].prefix, wl.requests[0].fields
    ans_max = len(fields[0].scaffold) + max(len(c) for c in fields[0].candidates)
    m = _model(sh, tiny_w, [len(prefix) + ans_max], [fields], len(prefix) + ans_max)
    st = m.prefill(prefix, capacity=len(prefix) + ans_max)
    got = m.decide_sequenced(st, fields, 1)
    first, rest, ext = opcd.decide_sequenced(tiny_dec, prefix, fields, 1)
    assert st.n_tokens == len(ext)
    _compare_fields("tiny-sequenced", got, first.fields + rest.fields, "f32", fields)
    s = m.stats()
    assert s["prefill_passes"] == 2 and s["branch_passes"] == 2
    st.close()
    m.close()


def test_tiny_first_field_round_spellings(tiny_w, tiny_dec):
    """The first-field round on labels with spellings: the answer written in
    is the chosen label's first spelling."""
    sh = pi.SHAPES["tiny"]
    prefix = _tokens(np.random.default_rng(24), sh.vocab_size, 50)
    fields = pi.random_spelling_fields(1800, sh.vocab_size, 4, max_labels=5, max_spellings=3, max_len=3)
    fields[2].mode = "exact"
    ans_max = len(fields[0].scaffold) + max(len(c) for c in fields[0].candidates)
    m = _model(sh, tiny_w, [len(prefix) + ans_max], [fields], len(prefix) + ans_max)
    st = m.prefill(prefix, capacity=len(prefix) + ans_max)
    got = m.decide_sequenced(st, fields, 1)
    first, rest, ext = opcd.decide_sequenced(tiny_dec, prefix, fields, 1)
    assert st.n_tokens == len(ext)
    _compare_fields("tiny-sequenced-spell", got, first.fields + rest.fields, "f32", fields)
    st.close()
    m.close()


def test_tiny_extend_errors_leave_state(tiny_w):
    """Past the buffer's capacity or outside the vocabulary: the call fails
    before any device work and the state keeps its tokens."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(23)
    fields = pi.make_workload("cfg0").requests[0].fields
    m = _model(sh, tiny_w, [40], [fields], 40)
    st = m.prefill(_tokens(rng, sh.vocab_size, 30), capacity=40)
    with pytest.raises(cpd.PcdError) as e:
        st.extend(_tokens(rng, sh.vocab_size, 11))
    assert e.value.name == "CAP" and st.n_tokens == 30
    with pytest.raises(cpd.PcdError) as e:
        st.extend([1, 2, sh.vocab_size])
    assert e.value.name == "TOKEN" and st.n_tokens == 30
    st.extend(_tokens(rng, sh.vocab_size, 10))
    assert st.n_tokens == 40
    st.close()
    m.close()


@pytest.fixture(scope="module")
def q15_l2():
    sh = pi.SHAPES["qwen2.5-1.5b"]
    w = pi.make_weights(sh, 1001, n_layers=2)
    return w.shape, w, odec.Decoder(w, np.float64)


def test_bf16_two_layer_warm_head_and_first_field_round(q15_l2):
    """The 28-field workload at the 1.5B widths (2 layers): its 512-token
    prefix as a cached 400-token head plus a 112-token request input (fork +
    extend), then the first-field round on the grown state."""
    sh, w, dec = q15_l2
    wl = pi.make_workload("cfg1")
    prefix, fields = wl.requests[0].prefix, wl.requests[0].fields
    ans_max = len(fields[0].scaffold) + max(len(c) for c in fields[0].candidates)
    cap = len(prefix) + ans_max
    m = _model(sh, w, [cap], [fields], cap)
    hs = m.prefill(prefix[:400])
    st = hs.fork(capacity=cap)
    st.extend(prefix[400:])
    got = [m.decide(st, fields, debug=True)]
    ref = opcd.decide(dec, [(list(prefix), fields)])
    _compare("q15-L2-warm", got, ref, ref.plan, "bf16")
    seq = m.decide_sequenced(st, fields, 1)
    first, rest, ext = opcd.decide_sequenced(dec, prefix, fields, 1)
    assert st.n_tokens == len(ext)
    _compare_fields("q15-L2-sequenced", seq, first.fields + rest.fields, "bf16", fields)
    st.close()
    hs.close()
    m.close()


# ---------------------------------------------------------------------------
# single-pass mode: new tokens and branch tokens in one decoder pass
# ---------------------------------------------------------------------------

def _fused_model(shape, weights, prefix_len, fields):
    """Limits with room for the prefix rows and the branch rows in one pass."""
    plan = cpd.debug_plan(shape.vocab_size, shape.max_seq, [prefix_len], [fields])
    return _model(shape, weights, [prefix_len], [fields], prefix_len + len(plan["tok"]))


def test_tiny_fused_cold_request(tiny_w, tiny_dec):
    """An empty state + extend_decide(prefix, fields): the decisions of
    prefill + decide, and the state's KV that prefill would leave, from one
    pass (150-token prefix across three 64-key tiles, trie fields)."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(31)
    prefix = _tokens(rng, sh.vocab_size, 150)
    fields = pi.make_workload("cfg0t").requests[0].fields
    m = _fused_model(sh, tiny_w, len(prefix), fields)
    st = m.new_state(len(prefix))
    got = [m.extend_decide(st, prefix, fields, debug=True)]
    assert st.n_tokens == len(prefix)
    ref = opcd.decide(tiny_dec, [(prefix, fields)])
    _compare("tiny-fused-cold", got, ref, ref.plan, "f32")
    kv = _kv(st, sh, len(prefix), np.float32)
    rkv = opcd.prefill(tiny_dec, prefix)
    err = max(float(np.max(np.abs(kv[l, i] - rkv[l][i]))) for l in range(sh.n_layers) for i in range(2))
    assert err < 1e-4
    s = m.stats()
    assert s["branch_passes"] == 1 and s["prefill_passes"] == 0
    # the state serves later decides as a prefilled one would
    again = [m.decide(st, fields, debug=True)]
    _compare("tiny-fused-then-decide", again, ref, ref.plan, "f32")
    st.close()
    m.close()


def test_tiny_fused_warm_request(tiny_w, tiny_dec):
    """A cached head (70 tokens) forked, then extend_decide(input of 40
    tokens, fields); and extend_decide with no new tokens is decide."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(32)
    head, inp = _tokens(rng, sh.vocab_size, 70), _tokens(rng, sh.vocab_size, 40)
    fields = pi.random_trie_fields(940, sh.vocab_size, 3)
    m = _fused_model(sh, tiny_w, len(head) + len(inp), fields)
    hs = m.prefill(head)
    st = hs.fork(capacity=len(head) + len(inp))
    got = [m.extend_decide(st, inp, fields, debug=True)]
    ref = opcd.decide(tiny_dec, [(head + inp, fields)])
    _compare("tiny-fused-warm", got, ref, ref.plan, "f32")
    got0 = [m.extend_decide(st, [], fields, debug=True)]
    _compare("tiny-fused-none", got0, ref, ref.plan, "f32")
    st.close()
    hs.close()
    m.close()


def test_tiny_fused_spellings_and_modes(tiny_w, tiny_dec):
    """Single-pass mode with labels that have spellings, one field pair per
    scoring mode (90-token prefix)."""
    sh = pi.SHAPES["tiny"]
    prefix = _tokens(np.random.default_rng(34), sh.vocab_size, 90)
    fields = []
    for i, mode in enumerate(("path", "exact", "level", "mean")):
        fields += pi.random_spelling_fields(1900 + i, sh.vocab_size, 2, max_spellings=4, max_len=4, mode=mode)
    m = _fused_model(sh, tiny_w, len(prefix), fields)
    st = m.new_state(len(prefix))
    got = [m.extend_decide(st, prefix, fields, debug=True)]
    ref = opcd.decide(tiny_dec, [(prefix, fields)])
    _compare("tiny-fused-spell", got, ref, ref.plan, "f32")
    st.close()
    m.close()


def test_bf16_two_layer_fused_cold(q15_l2):
    """The 28-field workload (512-token prefix) and the 255-option ID
    workload (2048-token prefix) at the 1.5B widths, 2 layers, each as one
    fused pass on an empty state."""
    sh, w, dec = q15_l2
    for name in ("cfg1", "cfg2"):
        wl = pi.make_workload(name)
        prefix, fields = wl.requests[0].prefix, wl.requests[0].fields
        m = _fused_model(sh, w, len(prefix), fields)
        st = m.new_state(len(prefix))
        got = [m.extend_decide(st, prefix, fields, debug=True)]
        ref = opcd.decide(dec, [(list(prefix), fields)])
        _compare(f"q15-L2-fused-{name}", got, ref, ref.plan, "bf16")
        st.close()
        m.close()


@pytest.mark.parametrize("hd", [32, 64])
def test_bf16_wide_fused_request(hd):
    """Single-pass requests whose new tokens fill at least 512 attention
    blocks of 128 rows: those causal rows run in a launch of their own,
    after the branch rows' launch, whose keys are then split as in a pass
    of branch rows only.  Head dim 32: an empty state and a 2,100-token
    prompt; head dim 64: a 300-token head, forked, and 4,100 new tokens
    (causal rows from position 300 on); then a decide on the state the pass
    left."""
    from test_gpu_parity import _wide_bf16_shape
    sh = _wide_bf16_shape(hd)
    w = pi.make_weights(sh, 1006)
    dec = odec.Decoder(w, np.float64)
    rng = np.random.default_rng(90 + hd)
    V = sh.vocab_size
    fields = pi.random_trie_fields(4400 + hd, V, 3, max_cands=6, max_len=3)
    head = _tokens(rng, V, {32: 0, 64: 300}[hd])
    inp = _tokens(rng, V, {32: 2100, 64: 4100}[hd])
    grp = sh.n_heads // sh.n_kv_heads
    assert sh.n_kv_heads * -(-len(inp) * grp // 128) >= 512
    m = _fused_model(sh, w, len(head) + len(inp), fields)
    if head:
        hs = m.prefill(head)
        st = hs.fork(capacity=len(head) + len(inp))
    else:
        hs, st = None, m.new_state(len(inp))
    got = [m.extend_decide(st, inp, fields, debug=True)]
    ref = opcd.decide(dec, [(head + inp, fields)])
    _compare(f"bf16-wide-fused-hd{hd}", got, ref, ref.plan, "bf16")
    # the state's KV, written by the pass, serves a later decide as prefill's would
    again = [m.decide(st, fields, debug=True)]
    _compare(f"bf16-wide-fused-hd{hd}-then-decide", again, ref, ref.plan, "bf16")
    if hs is not None:
        hs.close()
    st.close()
    m.close()


def test_tiny_started_calls_match_extend_decide(tiny_w):
    """extend_decide_start + finish returns what extend_decide does, bit for
    bit, with MAX_PENDING calls in flight on as many states and finished in
    reverse order; one more start while they are pending is refused (CAP)
    and leaves its state as it was."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(35)
    n = cpd.MAX_PENDING + 1
    prefixes = [_tokens(rng, sh.vocab_size, 40 + 9 * i) for i in range(n)]
    reqs = [pi.random_trie_fields(960 + i, sh.vocab_size, 2 + i % 2) for i in range(n)]
    p_all = cpd.debug_plan(sh.vocab_size, sh.max_seq, [len(p) for p in prefixes], reqs)
    m = _model(sh, tiny_w, [len(p) for p in prefixes], reqs, max(map(len, prefixes)) + len(p_all["tok"]))
    want = []
    for p, f in zip(prefixes, reqs):
        st = m.new_state(len(p))
        want.append(m.extend_decide(st, p, f))
        st.close()
    states = [m.new_state(len(p)) for p in prefixes]
    pend = [m.extend_decide_start(states[i], prefixes[i], reqs[i]) for i in range(n - 1)]
    with pytest.raises(cpd.PcdError) as e:
        m.extend_decide_start(states[-1], prefixes[-1], reqs[-1])
    assert e.value.name == "CAP"
    assert int(m.lib.pcd_state_tokens(states[-1].handle)) == 0
    got = [None] * n
    for i in reversed(range(n - 1)):
        got[i] = pend[i].finish()
    with pytest.raises(RuntimeError):
        pend[0].finish()
    # the refused call goes through once a slot is free
    got[-1] = m.extend_decide_start(states[-1], prefixes[-1], reqs[-1]).finish()
    for i in range(n):
        assert states[i].n_tokens == len(prefixes[i])
        for k in ("prob", "logscore", "mass", "margin", "argmax"):
            assert np.array_equal(got[i][k], want[i][k]), (i, k)
    assert m.stats()["branch_passes"] == 2 * n
    # a prefill enqueued between started calls (the workspace is shared; the
    # stream orders the passes): the same results as the calls one by one
    hs = m.prefill(prefixes[1])
    want_b = m.extend_decide(hs, [], reqs[1])
    hs.close()
    sa = m.new_state(len(prefixes[0]))
    pa = m.extend_decide_start(sa, prefixes[0], reqs[0])
    hb = m.prefill(prefixes[1])
    pb = m.extend_decide_start(hb, [], reqs[1])
    got_b, got_a = pb.finish(), pa.finish()
    for k in ("prob", "logscore", "mass", "margin", "argmax"):
        assert np.array_equal(got_a[k], want[0][k]) and np.array_equal(got_b[k], want_b[k]), k
    sa.close()
    hb.close()
    # a call still pending when the model is closed is finished first
    # and the states still open are freed before the model
    late = m.extend_decide_start(states[0], [], reqs[0])
    m.close()
    assert late.handle is None and all(st.handle is None for st in states)


def test_misaligned_buffers_are_refused(tiny_w):
    """Device buffers are accessed in 16-byte vectors: a KV buffer off that
    alignment is refused before any device work (PCD_E_ARG)."""
    sh = pi.SHAPES["tiny"]
    fields = pi.random_trie_fields(970, sh.vocab_size, 2)
    m = _model(sh, tiny_w, [16], [fields], 16)
    kv = torch.empty(m.state_bytes(16) + 16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(cpd.PcdError) as e:
        m.new_state(16, kv[8:])
    assert e.value.name == "ARG"
    st = m.new_state(16, kv[16:])
    assert st.n_tokens == 0
    m.close()


def test_tiny_models_on_two_streams_share_weights(tiny_w):
    """Two models over the same device weights, each with its own workspace,
    run started calls on two streams at once: every result equals the one
    the first model gives one call at a time."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(36)
    prefixes = [_tokens(rng, sh.vocab_size, 60 + 7 * i) for i in range(6)]
    reqs = [pi.random_trie_fields(980 + i, sh.vocab_size, 3) for i in range(6)]
    p_all = cpd.debug_plan(sh.vocab_size, sh.max_seq, [len(p) for p in prefixes], reqs)
    lim = cpd.limits_for(sh.vocab_size, sh.max_seq, [len(p) for p in prefixes], reqs,
                         max(map(len, prefixes)) + len(p_all["tok"]))
    dev = cpd.upload_weights(tiny_w.mats, sh.n_layers, sh.d_model, "cuda:0")
    models = [cpd.PcdModel(cpd.config_of(sh), dev, lim) for _ in range(2)]
    want = []
    for p, f in zip(prefixes, reqs):
        st = models[0].new_state(len(p))
        want.append(models[0].extend_decide(st, p, f))
        st.close()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    pend = []
    for i, (p, f) in enumerate(zip(prefixes, reqs)):
        k = i % 2
        with torch.cuda.stream(streams[k]):
            st = models[k].new_state(len(p))
            pend.append((models[k].extend_decide_start(st, p, f), st))
    for i, (pd, st) in enumerate(pend):
        got = pd.finish()
        st.close()
        for key in ("prob", "logscore", "mass", "margin", "argmax"):
            assert np.array_equal(got[key], want[i][key]), (i, key)
    for m in models:
        m.close()


def test_tiny_started_calls_with_kernel_timing(tiny_w):
    """With per-kernel timing on, two started calls finished in reverse
    order give the untimed results, and every launch of both passes is
    counted."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(37)
    prefixes = [_tokens(rng, sh.vocab_size, 50 + 20 * i) for i in range(2)]
    reqs = [pi.random_trie_fields(990 + i, sh.vocab_size, 2) for i in range(2)]
    p_all = cpd.debug_plan(sh.vocab_size, sh.max_seq, [len(p) for p in prefixes], reqs)
    m = _model(sh, tiny_w, [len(p) for p in prefixes], reqs, max(map(len, prefixes)) + len(p_all["tok"]))
    want, counts = [], []
    for p, f in zip(prefixes, reqs):
        st = m.new_state(len(p))
        m.set_kernel_timing(True)
        want.append(m.extend_decide(st, p, f))
        counts.append(sum(n for _, n in m.kernel_times().values()))
        m.set_kernel_timing(False)
        st.close()
    m.set_kernel_timing(True)
    states = [m.new_state(len(p)) for p in prefixes]
    pend = [m.extend_decide_start(states[i], prefixes[i], reqs[i]) for i in range(2)]
    got = [None, pend[1].finish(), None]
    got[0] = pend[0].finish()
    kt = m.kernel_times()
    assert sum(n for _, n in kt.values()) == sum(counts)
    assert all(ms >= 0 for ms, _ in kt.values())
    for i in range(2):
        for k in ("prob", "logscore", "mass", "margin", "argmax"):
            assert np.array_equal(got[i][k], want[i][k]), (i, k)
    m.close()


def test_call_on_another_stream_is_refused_while_a_call_runs(tiny_w, q15_l2):
    """A model's passes share its workspace, so while one of its calls is
    still on the device another call of the same model on a different stream
    is refused (PCD_E_ARG, before any device work); on the same stream, or
    once the call has left the device, it runs.  A started decide call is
    kept on the device by a bounded spin kernel (torch.cuda._sleep) ahead of
    it; a prefill is kept there by its own length (4,000 tokens at the 1.5B
    widths, 2 layers: milliseconds, against the microseconds the host takes
    to make the next call)."""
    sh = pi.SHAPES["tiny"]
    rng = np.random.default_rng(37)
    prefix = _tokens(rng, sh.vocab_size, 70)
    fields = pi.random_trie_fields(990, sh.vocab_size, 3)
    p = cpd.debug_plan(sh.vocab_size, sh.max_seq, [len(prefix)], [fields])
    m = _model(sh, tiny_w, [len(prefix)], [fields], len(prefix) + len(p["tok"]))
    st = m.prefill(prefix)
    want = m.decide(st, fields)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    # a started decide call on s1
    sa = m.new_state(len(prefix))
    with torch.cuda.stream(s1):
        torch.cuda._sleep(50_000_000)
        pa = m.extend_decide_start(sa, prefix, fields)
    with torch.cuda.stream(s2):
        with pytest.raises(cpd.PcdError) as e:
            m.decide(st, fields)
        assert e.value.name == "ARG"
        with pytest.raises(cpd.PcdError) as e:
            m.prefill(prefix)
        assert e.value.name == "ARG"
    with torch.cuda.stream(s1):  # same stream: ordered after it
        same = m.decide(st, fields)
    got_a = pa.finish()
    with torch.cuda.stream(s2):  # the call has left the device
        other = m.decide(st, fields)
    for got in (got_a, same, other):
        for k in ("prob", "logscore", "mass", "margin", "argmax"):
            assert np.array_equal(got[k], want[k]), k
    torch.cuda.synchronize()
    m.close()
    # a prefill pass still running on s1
    sh2, w2, _ = q15_l2
    wl = pi.make_workload("cfg1")
    f2 = wl.requests[0].fields
    long_prefix = _tokens(rng, sh2.vocab_size, 4000)
    m2 = _model(sh2, w2, [len(long_prefix)], [f2], len(long_prefix))
    with torch.cuda.stream(s1):
        hb = m2.prefill(long_prefix)
    with torch.cuda.stream(s2):
        with pytest.raises(cpd.PcdError) as e:
            m2.decide(hb, f2)
        assert e.value.name == "ARG"
    s1.synchronize()
    with torch.cuda.stream(s2):
        after = m2.decide(hb, f2)
    with torch.cuda.stream(s1):
        again = m2.decide(hb, f2)
    for k in ("prob", "logscore", "mass", "margin", "argmax"):
        assert np.array_equal(after[k], again[k]), k
    torch.cuda.synchronize()
    m2.close()
