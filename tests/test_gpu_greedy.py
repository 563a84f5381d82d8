"""The token-by-token baseline on the library's kernels against the oracle's
from-scratch greedy decoder: same labels, same output tokens, one decoder
pass per output token."""
import numpy as np
import pytest

import pcd_inputs as pi
from oracle import decoder as odec
from oracle import pcd as opcd

cpd = pytest.importorskip("constrained_decoding_pcd_amd")
torch = pytest.importorskip("torch")
from constrained_decoding_pcd_amd import greedy  # noqa: E402

pytestmark = pytest.mark.gpu


def test_tiny_token_by_token():
    sh = pi.SHAPES["tiny"]
    w = pi.make_weights(sh, 1000)
    dec = odec.Decoder(w, np.float64)
    wl = pi.make_workload("cfg0t")
    prefix, fields = wl.requests[0].prefix, list(wl.requests[0].fields)
    fields += pi.random_spelling_fields(2100, sh.vocab_size, 3, max_labels=4, max_spellings=3, max_len=3)
    print(f"case tiny-greedy: prefix {len(prefix)}, {len(fields)} fields", flush=True)
    lim = cpd.limits_for(sh.vocab_size, sh.max_seq, [len(prefix)], [fields])
    dev = cpd.upload_weights(w.mats, sh.n_layers, sh.d_model, "cuda:0")
    m = cpd.PcdModel(cpd.config_of(sh), dev, lim)
    got = greedy.decode(m, prefix, fields)
    labels, out, n = opcd.greedy_decode(dec, prefix, fields)
    print(f"[tiny-greedy] labels {got.labels} (oracle {labels}), {got.passes} passes", flush=True)
    assert got.labels == labels and got.tokens == out
    assert got.passes == n == len(out)
    m.close()
