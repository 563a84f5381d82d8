"""Writes cfg4_l2_full_prefix.json: the fp64 oracle's outputs for the
7B-shaped workload (16,384-token prefix, 64 fields, one of them a
200-option 3-token ID field) on the first 2 layers of its seeded weights.

The GPU test that reads it (tests/test_gpu_fullsize.py) runs the same
2-layer model over the whole prefix on the device and compares every
readout log-sum-exp, gathered logit, candidate log-score and probability,
field mass and argmax.  The oracle needs several minutes for this case, too
long for a GPU test's time limit, hence the stored values.  Only oracle/ and
the seeded input generators (pcd_inputs) are used here.

Run from the repository root:  python tests/golden/make_cfg4_l2_golden.py
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import pcd_inputs as pi  # noqa: E402
from oracle import decoder as odec  # noqa: E402
from oracle import pcd as opcd  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cfg4_l2_full_prefix.json")
N_LAYERS = 2


def tokens_sha(prefix, fields) -> str:
    """Digest of the workload's token ids, so the test can tell that the
    input generators still produce what these values were computed on."""
    h = hashlib.sha256(np.asarray(prefix, np.int64).tobytes())
    for f in fields:
        h.update(np.asarray(f.scaffold, np.int64).tobytes())
        for c in f.candidates:
            h.update(np.asarray(c, np.int64).tobytes())
    return h.hexdigest()


def main():
    wl = pi.make_workload("cfg4")
    req = wl.requests[0]
    t = time.time()
    w = pi.make_weights(wl.shape, wl.weight_seed, n_layers=N_LAYERS)
    print(f"weights {time.time() - t:.0f} s", flush=True)
    t = time.time()
    res = opcd.decide(odec.Decoder(w, np.float64), [(list(req.prefix), req.fields)])
    print(f"oracle {time.time() - t:.0f} s", flush=True)
    doc = {
        "what": "fp64 oracle, cfg4 workload (7B shape) on its first 2 layers, whole 16384-token prefix",
        "generator": "tests/golden/make_cfg4_l2_golden.py",
        "weight_seed": wl.weight_seed, "input_seed": wl.input_seed, "n_layers": N_LAYERS,
        "prefix_tokens": len(req.prefix), "fields": len(req.fields),
        "tokens_sha256": tokens_sha(req.prefix, req.fields),
        "lse": [float(v) for v in res.lse],
        "z": [float(v) for v in res.z],
        "prob": [float(v) for f in res.fields for v in f.prob],
        "logscore": [float(v) for f in res.fields for v in f.logscore],
        "mass": [float(f.mass) for f in res.fields],
        "argmax": [int(f.argmax) for f in res.fields],
        "margin": [float(f.margin) for f in res.fields],
        "cand_depth": [int(max(np.diff(res.plan.s_path_off)[res.plan.c_spell_off[c]:res.plan.c_spell_off[c + 1]]))
                       for c in range(len(res.plan.c_spell_off) - 1)],
        "field_cand_off": [int(v) for v in res.plan.f_cand_off],
    }
    with open(OUT, "w") as fh:
        json.dump(doc, fh)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
