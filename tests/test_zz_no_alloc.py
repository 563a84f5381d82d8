"""pcd_load_weights_noalloc: a model whose workspace is the library's static
device array, for callers that cannot allocate device memory.

Its calls run the same kernels on the same inputs as a model created by
pcd_load_weights over a torch-allocated workspace, so every output must be
bit-identical to that model's: prefill + decide and the single pass, for
the tiny fp32 model and the 1.5B widths at 2 layers.  Each model runs a
request and then a smaller one (the static array keeps the first call's
contents), and a second no-allocation model with smaller limits is created
after the first is freed and runs the smaller request again.  Limits that
need more than the array holds are refused (PCD_E_CAP), and so is a second
live no-allocation model on the same device (PCD_E_ARG).
"""
import numpy as np
import pytest

import pcd_inputs as pi

cpd = pytest.importorskip("constrained_decoding_pcd_amd")
torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

KEYS = ("prob", "logscore", "mass", "margin", "argmax", "lse", "z")


def _lim(sh, prefix, fields):
    p = cpd.debug_plan(sh.vocab_size, sh.max_seq, [len(prefix)], [fields])
    return cpd.limits_for(sh.vocab_size, sh.max_seq, [len(prefix)], [fields], len(prefix) + len(p["tok"]))


def _both_modes(m, prefix, fields):
    st = m.prefill(prefix)
    two = m.decide(st, fields, debug=True)
    st.close()
    st = m.new_state(len(prefix))
    one = m.extend_decide(st, prefix, fields, debug=True)
    st.close()
    return two, one


def _same(a, b, what):
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), (what, k)


CASES = {
    "tiny": ("tiny", 1000, None, "cfg0t", 40, 2),
    "bf16-L2": ("qwen2.5-1.5b", 1001, 2, "cfg1", 200, 9),
}


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_model_matches_the_allocating_model(case):
    shape_name, seed, n_layers, wl_name, small_prefix, small_fields = CASES[case]
    w = pi.make_weights(pi.SHAPES[shape_name], seed, n_layers=n_layers)
    sh = w.shape
    req = pi.make_workload(wl_name).requests[0]
    big = (req.prefix, req.fields)
    small = (req.prefix[:small_prefix], req.fields[:small_fields])
    print(f"case {case}: {sh.n_layers} layers, requests of {len(big[0])} and {len(small[0])} tokens", flush=True)
    dev = cpd.upload_weights(w.mats, sh.n_layers, sh.d_model, "cuda:0")
    lim = _lim(sh, *big)
    ref = cpd.PcdModel(cpd.config_of(sh), dev, lim)
    want = {k: _both_modes(ref, *r) for k, r in (("big", big), ("small", small))}
    ref.close()
    na = cpd.PcdModel(cpd.config_of(sh), dev, lim, noalloc=True)
    try:
        # a second model on the same device while the first holds the array
        with pytest.raises(cpd.PcdError) as e:
            cpd.PcdModel(cpd.config_of(sh), dev, lim, noalloc=True)
        assert e.value.name == "ARG"
        for k in ("big", "small"):  # two calls in a row, the second smaller
            got = _both_modes(na, *(big if k == "big" else small))
            _same(got[0], want[k][0], (k, "two-pass"))
            _same(got[1], want[k][1], (k, "single-pass"))
    finally:
        na.close()
    # freed: the array serves a new model, here with smaller limits
    na2 = cpd.PcdModel(cpd.config_of(sh), dev, _lim(sh, *small), noalloc=True)
    try:
        got = _both_modes(na2, *small)
        _same(got[0], want["small"][0], ("second model", "two-pass"))
        _same(got[1], want["small"][1], ("second model", "single-pass"))
    finally:
        na2.close()
    torch.cuda.synchronize()


def test_noalloc_limits_beyond_the_array_are_refused():
    """The 64-request batch needs far more workspace than the static array
    holds: refused before anything is created."""
    sh = pi.SHAPES["qwen2.5-1.5b"].with_layers(1)
    w = pi.make_weights(pi.SHAPES["qwen2.5-1.5b"], 1001, n_layers=1)
    dev = cpd.upload_weights(w.mats, sh.n_layers, sh.d_model, "cuda:0")
    lim = dict(max_prefill_tokens=65536, max_branch_tokens=18000, max_readouts=1792, max_gathers=6000,
               max_fields=1792, max_candidates=6000, max_requests=64, max_spellings=0)
    with pytest.raises(cpd.PcdError) as e:
        cpd.PcdModel(cpd.config_of(sh), dev, lim, noalloc=True)
    assert e.value.name == "CAP"
    # nothing was claimed: a model that fits is still accepted
    small = pi.make_workload("cfg1").requests[0]
    m = cpd.PcdModel(cpd.config_of(sh), dev, _lim(sh, small.prefix[:64], small.fields[:3]), noalloc=True)
    m.close()
