"""GPU checks against a closed form and the tie rule.

With an all-zero LM head every logit is exactly 0, whatever the decoder
computes before it.  Then, for every readout row, the log-sum-exp over the
vocabulary is log V; every candidate of a field whose paths have equal
length gets the same log-score, so its probability is 1/K at any
temperature; the argmax falls to the lowest declaration index ("Parallel
Constrained Decoding: A Technical Reference", "Notes on the softmax" leaves
ties open, its FAQ suggests first in declaration order); the top-2 margin
is 0; and the candidate mass is (distinct first tokens) / V ("Parallel
Constrained Decoding from Scratch", "And you get confidence for free").

The untied zero head goes through the library's ordinary untied-head path
(pcd_weights.lm_head).  Each case also runs the fp64 oracle with its zero
head switched on and checks that both sides give these values.
"""
import math

import numpy as np
import pytest

import pcd_inputs as pi
from oracle import decoder as odec
from oracle import pcd as opcd

cpd = pytest.importorskip("constrained_decoding_pcd_amd")
torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _zero_head_model(shape, weights, prefix, fields):
    dev = cpd.upload_weights(weights.mats, shape.n_layers, shape.d_model, "cuda:0")
    dt = torch.float32 if shape.dtype == "f32" else torch.int16  # bf16 zeros are all-zero 16-bit patterns
    dev["lm_head"] = torch.zeros(shape.vocab_size, shape.d_model, dtype=dt, device="cuda:0")
    cfg = cpd.config_of(shape)
    cfg["tied_lm_head"] = 0
    lim = cpd.limits_for(shape.vocab_size, shape.max_seq, [len(prefix)], [fields])
    return cpd.PcdModel(cfg, dev, lim)


CASES = {
    # tiny fp32 model: 4 single-token fields and one field of six 3-token IDs
    "tiny-cfg0t": ("tiny", 1000, None, "cfg0t"),
    # the 1.5B widths at 2 layers: 10 booleans (one shared token pair) and 18 four-way enums
    "bf16-L2-cfg1": ("qwen2.5-1.5b", 1001, 2, "cfg1"),
    # the 1.5B widths at 2 layers: 3 booleans and a 255-option 3-token ID field (18 trie readouts)
    "bf16-L2-cfg2": ("qwen2.5-1.5b", 1001, 2, "cfg2"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_zero_lm_head_closed_form_and_tie_rule(case):
    shape_name, seed, n_layers, wl_name = CASES[case]
    w = pi.make_weights(pi.SHAPES[shape_name], seed, n_layers=n_layers)
    sh = w.shape
    wl = pi.make_workload(wl_name)
    prefix, fields = wl.requests[0].prefix, wl.requests[0].fields
    print(f"case {case}: {sh.n_layers} layers, prefix {len(prefix)}, {len(fields)} fields", flush=True)
    m = _zero_head_model(sh, w, prefix, fields)
    st = m.prefill(prefix)
    V = sh.vocab_size
    logV = math.log(V)
    dec = odec.Decoder(w, np.float64)
    dec.zero_head = True
    ref = opcd.decide(dec, [(prefix, fields)])
    for T in (1.0, 0.5):
        got = m.decide(st, fields, temperature=T, debug=True)
        # every readout: all V logits are 0
        assert np.all(got["z"] == 0.0)
        assert np.max(np.abs(got["lse"].astype(np.float64) - logV)) <= 2e-6
        assert np.max(np.abs(ref.lse - logV)) <= 1e-12
        off = 0
        for i, (f, fr) in enumerate(zip(fields, ref.fields)):
            k = len(f.candidates)
            q = got["prob"][off:off + k].astype(np.float64)
            ls = got["logscore"][off:off + k]
            # equal path lengths within each field: one log-score for all candidates, bit for bit
            assert np.all(ls == ls[0]), (i, ls)
            assert np.max(np.abs(q - 1.0 / k)) <= 1e-6, (i, q)
            # the tie rule: the lowest declaration index, margin exactly 0
            assert int(got["argmax"][i]) == 0 and fr.argmax == 0, i
            assert float(got["margin"][i]) == 0.0 and fr.margin == 0.0, i
            distinct = len({c[0] for c in f.candidates})
            assert abs(float(got["mass"][i]) - distinct / V) <= 1e-5 * distinct / V, (i, got["mass"][i])
            assert abs(fr.mass - distinct / V) <= 1e-12
            # the oracle (T = 1) against the library: identical closed-form values
            if T == 1.0:
                assert np.max(np.abs(q - fr.prob)) <= 1e-6
                assert np.max(np.abs(ls.astype(np.float64) - fr.logscore)) <= 1e-5 * max(1.0, abs(fr.logscore[0]))
            off += k
    st.close()
    m.close()
