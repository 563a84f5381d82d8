"""GPU parity at full model depth and full workload sizes.

The bench request (28 layers, 512-token prefix, 28 fields) and the
255-option ID workload run whole through the library and through the fp64
oracle.  The 64-request throughput batch runs in one branch pass on the GPU;
two of its requests are re-computed by the oracle and compared one by one.
The 7B shape runs with 2 layers against the oracle (on the first 2,048
prefix tokens live, and on the whole 16,384-token prefix against the
oracle's stored values), and at full depth with its 16,384-token prefix
against properties that hold at any size.

Full-depth bf16 tolerances (tests/tolerances.py): the 2-layer bounds scaled
by the growth of the logit error with depth in a model of the device's bf16
rounding points (test_bf16_bound.py derives the factor, sigma_28 / sigma_2 =
2.65, on the 28-field request): 6.6e-2 on logits, 2.7e-3 on log-sum-exps,
6.9e-2 on per-token log-scores, 3.5e-2 on probabilities, 7.1e-2 relative on
mass; the argmax must match wherever the oracle's top-2 margin is at least
2 z (0.13 nats) for single-token fields, 2 ls per token on deeper paths.
"""
import importlib.util
import json
import os

import numpy as np
import pytest

import pcd_inputs as pi
from oracle import decoder as odec
from oracle import pcd as opcd
from test_gpu_parity import cand_depth, check_argmax
import tolerances as tl

cpd = pytest.importorskip("constrained_decoding_pcd_amd")
torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEEP = tl.BF16_L28


def _errors(got, ref_fields, ref_lse, ref_z, plan):
    prob = np.concatenate([g["prob"] for g in got])
    ls = np.concatenate([g["logscore"] for g in got])
    mass = np.concatenate([g["mass"] for g in got])
    rprob = np.concatenate([f.prob for f in ref_fields])
    rls = np.concatenate([f.logscore for f in ref_fields])
    rmass = np.array([f.mass for f in ref_fields])
    d = {
        "lse": float(np.max(np.abs(np.concatenate([g["lse"] for g in got]) - ref_lse))),
        "z": float(np.max(np.abs(np.concatenate([g["z"] for g in got]) - ref_z))),
        "ls/len": float(np.max(np.abs(ls - rls) / cand_depth(plan))),
        "prob": float(np.max(np.abs(prob - rprob))),
        "mass_rel": float(np.max(np.abs(mass - rmass) / rmass)),
    }
    return d


def _check(name, got, ref, tol=DEEP):
    d = _errors(got, ref.fields, ref.lse, ref.z, ref.plan)
    arg = np.concatenate([g["argmax"] for g in got])
    agree = sum(int(a == f.argmax) for a, f in zip(arg, ref.fields))
    print(f"[{name}] max errors: " + ", ".join(f"{k} {v:.3e}" for k, v in d.items()) +
          f"; argmax {agree}/{len(ref.fields)}, min margin {min(f.margin for f in ref.fields):.3f}", flush=True)
    assert d["lse"] <= tol["lse"] and d["z"] <= tol["z"]
    assert d["ls/len"] <= tol["ls"]
    assert d["prob"] <= tol["prob"]
    assert d["mass_rel"] <= tol["mass"]
    check_argmax(arg, ref.fields, ref.plan, tol, name)
    _invariants(got)


def _invariants(got):
    for g in got:
        assert np.all(np.isfinite(g["prob"])) and np.all(np.isfinite(g["logscore"]))
        assert np.all(g["mass"] > 0) and np.all(g["mass"] <= 1.0 + 1e-6)


def _field_sums_to_one(got, requests):
    for g, fields in zip(got, requests):
        off = 0
        for i, f in enumerate(fields):
            k = len(f.candidates)
            p = g["prob"][off:off + k]
            assert abs(float(p.sum()) - 1.0) <= 1e-6
            # the argmax is the candidate with the largest log-score (first on ties)
            assert int(g["argmax"][i]) == int(np.argmax(g["logscore"][off:off + k]))
            off += k


def _model(shape, weights, prefixes, requests):
    dev = cpd.upload_weights(weights.mats, shape.n_layers, shape.d_model, "cuda:0")
    lim = cpd.limits_for(shape.vocab_size, shape.max_seq, [len(p) for p in prefixes], requests)
    return cpd.PcdModel(cpd.config_of(shape), dev, lim), dev


@pytest.fixture(scope="module")
def q15_full():
    sh = pi.SHAPES["qwen2.5-1.5b"]
    w = pi.make_weights(sh, 1001)
    return sh, w


def _full_case(name, shape, w, wl_name):
    wl = pi.make_workload(wl_name)
    reqs = [(r.prefix, r.fields) for r in wl.requests]
    print(f"case {name}: {shape.n_layers} layers, prefix {len(reqs[0][0])}, {len(reqs[0][1])} fields", flush=True)
    m, dev = _model(shape, w, [p for p, _ in reqs], [f for _, f in reqs])
    st = m.prefill(reqs[0][0])
    got = [m.decide(st, reqs[0][1], debug=True)]
    ref = opcd.decide(odec.Decoder(w, np.float64), reqs)
    _check(name, got, ref)
    _field_sums_to_one(got, [reqs[0][1]])
    st.close()
    m.close()


def test_bench_request_full_depth(q15_full):
    """The bench's request, in the bench's launch configuration: every
    readout, gather and field of the 28-layer model."""
    sh, w = q15_full
    _full_case("cfg1-full", sh, w, "cfg1")


def test_bench_request_full_depth_fused(q15_full):
    """The bench's request in single-pass mode (empty state, the 512 prefix
    tokens and the 287 branch tokens in one 28-layer pass)."""
    sh, w = q15_full
    wl = pi.make_workload("cfg1")
    prefix, fields = wl.requests[0].prefix, wl.requests[0].fields
    plan = cpd.debug_plan(sh.vocab_size, sh.max_seq, [len(prefix)], [fields])
    dev = cpd.upload_weights(w.mats, sh.n_layers, sh.d_model, "cuda:0")
    lim = cpd.limits_for(sh.vocab_size, sh.max_seq, [len(prefix)], [fields], len(prefix) + len(plan["tok"]))
    m = cpd.PcdModel(cpd.config_of(sh), dev, lim)
    st = m.new_state(len(prefix))
    got = [m.extend_decide(st, prefix, fields, debug=True)]
    ref = opcd.decide(odec.Decoder(w, np.float64), [(list(prefix), fields)])
    _check("cfg1-full-fused", got, ref)
    _field_sums_to_one(got, [fields])
    st.close()
    m.close()


def test_id_field_full_depth(q15_full):
    """2048-token prefix; one 255-option ID field resolved by trie
    continuation rows, plus 3 booleans; 28 layers."""
    sh, w = q15_full
    _full_case("cfg2-full", sh, w, "cfg2")


def test_throughput_batch_sampled(q15_full):
    """64 requests (1024-token prefixes, 28 fields each: 1792 fields) in ONE
    branch pass; requests 0 and 63 re-computed by the oracle one by one."""
    sh, w = q15_full
    wl = pi.make_workload("cfg3")
    reqs = [(r.prefix, r.fields) for r in wl.requests]
    m, dev = _model(sh, w, [p for p, _ in reqs], [f for _, f in reqs])
    states = [m.prefill(p) for p, _ in reqs]
    got = m.decide_many(states, [f for _, f in reqs], debug=True)
    s = m.stats()
    assert s["branch_passes"] == 1 and s["last_requests"] == 64
    print(f"[cfg3] one branch pass: {s['last_branch_tokens']} branch tokens, {s['last_readouts']} readouts", flush=True)
    _field_sums_to_one(got, [f for _, f in reqs])
    _invariants(got)
    dec = odec.Decoder(w, np.float64)
    for r in (0, 63):
        ref = opcd.decide(dec, [reqs[r]])
        _check(f"cfg3-req{r}", [got[r]], ref)
    for st in states:
        st.close()
    m.close()


@pytest.fixture(scope="module")
def q7_two_layer():
    sh = pi.SHAPES["qwen2.5-7b"]
    w = pi.make_weights(sh, 1002, n_layers=2)
    return w.shape, w


def test_7b_two_layer_parity(q7_two_layer):
    """The 7B shape (28 Q / 4 KV heads, FFN 18944, untied head) with its
    64-field schema (one 200-option ID field) on the first 2 layers and the
    first 2048 tokens of its prefix: every output against the oracle."""
    sh, w = q7_two_layer
    wl = pi.make_workload("cfg4")
    req = (wl.requests[0].prefix[:2048], wl.requests[0].fields)
    m, dev = _model(sh, w, [req[0]], [req[1]])
    st = m.prefill(req[0])
    got = [m.decide(st, req[1], debug=True)]
    ref = opcd.decide(odec.Decoder(w, np.float64), [req])
    _check("cfg4-L2-P2048", got, ref, tl.BF16_7B_L2)
    st.close()
    m.close()


def test_7b_full_depth_long_prefix_invariants():
    """The 7B shape at full depth with the 16384-token prefix and 64 fields:
    properties that hold at any size (probabilities sum to 1, 0 < mass <= 1,
    argmax = largest log-score, one prefill + one branch pass, bit-identical
    reruns, the prefix KV untouched by decide)."""
    sh = pi.SHAPES["qwen2.5-7b"]
    wl = pi.make_workload("cfg4")
    w = pi.make_weights(sh, wl.weight_seed)
    req = wl.requests[0]
    m, dev = _model(sh, w, [req.prefix], [req.fields])
    del w
    st = m.prefill(req.prefix)
    kv_sum = float(st.kv.view(torch.int16)[:: 4096].float().sum())
    a = m.decide(st, req.fields, debug=True)
    b = m.decide(st, req.fields, debug=True)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert float(st.kv.view(torch.int16)[:: 4096].float().sum()) == kv_sum
    _field_sums_to_one([a], [req.fields])
    _invariants([a])
    s = m.stats()
    assert s["prefill_passes"] == 1 and s["branch_passes"] == 2
    print(f"[cfg4-full] prefill {s['last_prefill_ms']:.1f} ms, branch {s['last_branch_ms']:.2f} ms, "
          f"readout {s['last_readout_ms']:.2f} ms, {s['last_branch_tokens']} branch tokens", flush=True)
    st.close()
    m.close()


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_7b_two_layer_full_prefix_against_stored_oracle():
    """The 7B shape on its first 2 layers with the WHOLE 16,384-token
    prefix and all 64 fields (one 200-option 3-token ID field): every
    readout's log-sum-exp and gathered logits, every candidate's log-score
    and probability, every field's mass and argmax against the fp64
    oracle's values, stored by tests/golden/make_cfg4_l2_golden.py (which
    calls only the oracle; it needs about 12 minutes of CPU).  The long-key
    path (256 key tiles of the prefix per attention row block) is compared
    element by element here.  A cached prefix gives the exact result for
    any continuation ("Parallel Constrained Decoding from Scratch", "The
    piece of plumbing you need: the KV cache")."""
    with open(os.path.join(GOLDEN, "cfg4_l2_full_prefix.json")) as fh:
        g = json.load(fh)
    spec = importlib.util.spec_from_file_location("mk", os.path.join(GOLDEN, "make_cfg4_l2_golden.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    wl = pi.make_workload("cfg4")
    req = wl.requests[0]
    assert mk.tokens_sha(req.prefix, req.fields) == g["tokens_sha256"], "the input generators changed"
    w = pi.make_weights(pi.SHAPES["qwen2.5-7b"], g["weight_seed"], n_layers=g["n_layers"])
    sh = w.shape
    m, dev = _model(sh, w, [req.prefix], [req.fields])
    del w
    st = m.prefill(req.prefix)
    got = m.decide(st, req.fields, debug=True)
    tol = tl.BF16_7B_L2
    depth = np.array(g["cand_depth"])
    d = {"lse": float(np.max(np.abs(got["lse"] - np.array(g["lse"])))),
         "z": float(np.max(np.abs(got["z"] - np.array(g["z"])))),
         "ls/len": float(np.max(np.abs(got["logscore"] - np.array(g["logscore"])) / depth)),
         "prob": float(np.max(np.abs(got["prob"] - np.array(g["prob"])))),
         "mass_rel": float(np.max(np.abs(got["mass"] - np.array(g["mass"])) / np.array(g["mass"])))}
    agree = sum(int(a == b) for a, b in zip(got["argmax"], g["argmax"]))
    print("[cfg4-L2-P16384] max errors: " + ", ".join(f"{k} {v:.3e}" for k, v in d.items()) +
          f"; argmax {agree}/{len(g['argmax'])}, min margin {min(g['margin']):.3f}", flush=True)
    assert len(got["lse"]) == len(g["lse"]) and len(got["z"]) == len(g["z"])
    assert d["lse"] <= tol["lse"] and d["z"] <= tol["z"]
    assert d["ls/len"] <= tol["ls"] and d["prob"] <= tol["prob"] and d["mass_rel"] <= tol["mass"]
    off = g["field_cand_off"]
    for f in range(len(g["argmax"])):
        fd = int(depth[off[f]:off[f + 1]].max())
        if g["margin"][f] >= tl.margin_waiver(tol, fd):
            assert int(got["argmax"][f]) == g["argmax"][f], (f, g["margin"][f])
    _invariants([got])
    _field_sums_to_one([got], [req.fields])
    st.close()
    m.close()
