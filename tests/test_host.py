"""Host-side checks of the C-ABI library (no device work).

The library's plan builder (C++) must equal the oracle's plan element by
element, and reject the same invalid inputs with the same error codes.
"""
import ctypes
import re
import os

import numpy as np
import pytest

import pcd_inputs as pi
from oracle import plan as oplan

cpd = pytest.importorskip("constrained_decoding_pcd_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return cpd.load_library()


def test_library_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "pcd.h")).read()
    declared = set(re.findall(r"\b(pcd_[a-z_]+)\s*\(", hdr))
    assert declared == set(cpd.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_binding_constants_match_the_header():
    hdr = open(os.path.join(ROOT, "include", "pcd.h")).read()
    assert int(re.search(r"#define PCD_MAX_PENDING (\d+)", hdr).group(1)) == cpd.MAX_PENDING


def _compare_plans(requests, V, max_seq=1 << 20):
    lens = [len(p) for p, _ in requests]
    ours = cpd.debug_plan(V, max_seq, lens, [f for _, f in requests])
    ref = oplan.build_plan([(len(p), f) for p, f in requests], V)
    names = {"field": "tfield"}
    for k, v in ours.items():
        r = getattr(ref, names.get(k, k))
        assert v.dtype == np.int32
        assert np.array_equal(v, r), k


@pytest.mark.parametrize("name", ["cfg0", "cfg0t", "cfg1", "cfg2"])
def test_plan_equals_oracle_on_workloads(name):
    wl = pi.make_workload(name)
    _compare_plans([(r.prefix, r.fields) for r in wl.requests], wl.shape.vocab_size)


def test_plan_equals_oracle_multi_request():
    wl = pi.make_workload("cfg3")
    reqs = [(r.prefix, r.fields) for r in wl.requests[:5]]
    _compare_plans(reqs, wl.shape.vocab_size)


@pytest.mark.parametrize("seed", range(6))
def test_plan_equals_oracle_random_tries(seed):
    V = 5000
    rng = np.random.default_rng(seed)
    reqs = []
    for r in range(1 + seed % 3):
        prefix = [int(t) for t in rng.integers(0, V, size=int(rng.integers(1, 50)))]
        reqs.append((prefix, pi.random_trie_fields(100 * seed + r, V, 5, max_cands=20, max_len=5)))
    _compare_plans(reqs, V)


@pytest.mark.parametrize("mode", ["path", "exact", "level", "mean"])
@pytest.mark.parametrize("seed", range(3))
def test_plan_equals_oracle_spellings_and_modes(seed, mode):
    """Labels with several spellings, and every scoring mode (EXACT and MEAN
    read out at every node a spelling continues from)."""
    V = 3000
    rng = np.random.default_rng(50 + seed)
    reqs = []
    for r in range(1 + seed % 2):
        prefix = [int(t) for t in rng.integers(0, V, size=int(rng.integers(1, 40)))]
        fields = pi.random_spelling_fields(700 + 10 * seed + r, V, 4, max_labels=6, max_spellings=4, max_len=4,
                                           mode=mode)
        fields += pi.random_trie_fields(900 + 10 * seed + r, V, 2, max_cands=9, max_len=4)
        for f in fields[-2:]:
            f.mode = mode
        reqs.append((prefix, fields))
    _compare_plans(reqs, V)


def test_plan_id_field_with_255_options():
    wl = pi.make_workload("cfg2")
    r = wl.requests[0]
    plan = cpd.debug_plan(wl.shape.vocab_size, 1 << 20, [len(r.prefix)], [r.fields])
    assert len(plan["ro_tok"]) == 21 and len(plan["g_tok"]) == 278


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
    (pi.Field([3], [[1], [2]], spellings=[[[1], [7, 9999]], [[2]]]), "TOKEN"),
    (pi.Field([3], [[1], [2]], spellings=[[[1]], [[2]] + [[9, i] for i in range(1023)]]), "NCAND"),
])
def test_plan_rejects_like_the_oracle(bad, code):
    with pytest.raises(oplan.PlanError) as e:
        oplan.build_plan([(4, [bad])], 1000)
    assert e.value.code == code
    with pytest.raises(cpd.PcdError) as e2:
        cpd.debug_plan(1000, 1 << 20, [4], [[bad]])
    assert e2.value.name == code


def test_positions_beyond_max_seq_are_rejected():
    f = pi.Field([1, 2, 3], [[4, 5], [4, 6]])
    cpd.debug_plan(1000, 10, [5], [[f]])         # last position 5 + 3 + 1 - 1 = 8 < 10
    with pytest.raises(cpd.PcdError) as e:
        cpd.debug_plan(1000, 8, [5], [[f]])
    assert e.value.name == "CAP"


def test_workspace_bytes_rejects_bad_configs(lib):
    good = dict(n_layers=2, d_model=128, n_heads=4, n_kv_heads=2, head_dim=32, ffn_dim=384, vocab_size=2048,
                max_seq=512, rope_theta=1e4, rms_eps=1e-6, tied_lm_head=1, dtype=0)
    lim = cpd.binding.pcd_limits(256, 64, 16, 64, 8, 32, 2, 0)
    assert lib.pcd_workspace_bytes(ctypes.byref(cpd.binding.pcd_config(**good)), ctypes.byref(lim)) > 0
    for k, v in (("head_dim", 48), ("n_kv_heads", 3), ("d_model", 100), ("dtype", 7), ("vocab_size", 2000)):
        bad = dict(good, **{k: v})
        assert lib.pcd_workspace_bytes(ctypes.byref(cpd.binding.pcd_config(**bad)), ctypes.byref(lim)) == 0


def test_pass_rows_may_exceed_max_seq_but_are_bounded(lib):
    """max_prefill_tokens counts the rows of one pass (all sequences of a
    batched prefill), so it may exceed max_seq; the row count of a pass is
    bounded (2^18) and every limit must be positive."""
    cfg = cpd.binding.pcd_config(n_layers=2, d_model=128, n_heads=4, n_kv_heads=2, head_dim=32, ffn_dim=384,
                                 vocab_size=2048, max_seq=512, rope_theta=1e4, rms_eps=1e-6, tied_lm_head=1,
                                 dtype=0)
    ws = lambda *a: lib.pcd_workspace_bytes(ctypes.byref(cfg), ctypes.byref(cpd.binding.pcd_limits(*a)))
    small = ws(256, 64, 16, 64, 8, 32, 2, 0)
    big = ws(64 * 512, 64, 16, 64, 8, 32, 64, 0)
    assert 0 < small < big
    assert ws(1 << 18, 64, 16, 64, 8, 32, 2, 0) > 0
    assert ws((1 << 18) + 1, 64, 16, 64, 8, 32, 2, 0) == 0
    assert ws(256, (1 << 18) + 1, 16, 64, 8, 32, 2, 0) == 0
    assert ws(0, 64, 16, 64, 8, 32, 2, 0) == 0


def test_null_arguments_are_rejected(lib):
    assert lib.pcd_decide_many(None, None, 0, 1.0, None, None) == -1
    assert lib.pcd_prefill(None, None, 0, None, 0, None, None) == -1
    assert b"null" in lib.pcd_last_error()
    lib.pcd_free_state(None)
    lib.pcd_free_model(None)


def test_compiled_fields_give_the_same_plan():
    """A schema marshalled once (CompiledFields) hands the library the same
    C arrays as the field lists: the plans are identical, also mixed with
    plain lists in one multi-request call."""
    V = 3000
    wl = pi.make_workload("cfg1")
    r = wl.requests[0]
    sp = pi.random_spelling_fields(4242, V, 3, max_labels=5, max_spellings=3, max_len=3, mode="level")
    for fields, P, vocab in ((r.fields, len(r.prefix), wl.shape.vocab_size), (sp, 17, V)):
        comp = cpd.PcdModel.compile_fields(fields)
        a = cpd.debug_plan(vocab, 1 << 20, [P, P + 5], [fields, fields])
        b = cpd.debug_plan(vocab, 1 << 20, [P, P + 5], [comp, fields])
        c = cpd.debug_plan(vocab, 1 << 20, [P, P + 5], [comp, comp])
        for k in a:
            assert np.array_equal(a[k], b[k]) and np.array_equal(a[k], c[k]), k
    assert len(comp) == len(sp) and comp[0] is sp[0]
