"""Derivation of the bf16 parity tolerances (CPU, no GPU needed).

The device rounds to bf16 at seven points per layer (tests/bf16_emulation.py
lists them).  Running that model of its arithmetic against the fp64 oracle
on the 28-field request of the 1.5B-shaped model gives the RMS error of the
gathered logits at 2 and at 28 layers, sigma_2 and sigma_28.  The bounds in
tests/tolerances.py scale the 2-layer anchor (2.5e-2 per logit, the 0.05-nat
argmax waiver) by sigma_L / sigma_2; this test re-derives that ratio and
checks the committed constants against it, and checks that the anchor sits
at least 4 sigma_2 above zero, so that a device whose rounding behaves as
modelled passes with high probability at every depth.
"""
import os

import numpy as np
import pytest

import pcd_inputs as pi
from bf16_emulation import Bf16Emulation
from oracle import decoder as odec
from oracle import pcd as opcd
import tolerances as tol


@pytest.mark.slow
def test_bf16_tolerances_follow_the_rounding_model():
    wl = pi.make_workload("cfg1")
    w = pi.make_weights(wl.shape, wl.weight_seed)  # 28 layers; the 2-layer run uses the first two
    reqs = [(r.prefix, r.fields) for r in wl.requests]
    ref_dec, emu_dec = odec.Decoder(w, np.float64), Bf16Emulation(w)
    sig, worst = {}, {}
    for L in (2, 28):
        ref = opcd.decide(ref_dec, reqs, n_layers=L)
        emu = opcd.decide(emu_dec, reqs, n_layers=L)
        ez, el = emu.z - ref.z, emu.lse - ref.lse
        sig[L] = float(np.sqrt(np.mean(ez ** 2)))
        worst[L] = (float(np.max(np.abs(ez))), float(np.max(np.abs(el))))
        print(f"L={L}: logit error rms {sig[L]:.3e}, max {worst[L][0]:.3e}; lse max {worst[L][1]:.3e}", flush=True)
    ratio = sig[28] / sig[2]
    # the anchor is well clear of the modelled 2-layer error
    assert tol.Z_L2 / sig[2] >= 4.0
    # the committed depth ratio is the derived one (to 3%)
    assert abs(tol.SIGMA_RATIO_28 - ratio) <= 0.03 * ratio, ratio
    # the model of the device passes the bounds derived from it
    assert worst[2][0] <= tol.BF16_L2["z"] and worst[2][1] <= tol.BF16_L2["lse"]
    assert worst[28][0] <= tol.BF16_L28["z"] and worst[28][1] <= tol.BF16_L28["lse"]


@pytest.mark.slow
@pytest.mark.skipif(os.environ.get("PCD_SLOW_DERIVATION") != "1",
                    reason="about 5 minutes of CPU (the fp64 oracle casts the 7B shape's embedding and head); "
                           "run with PCD_SLOW_DERIVATION=1")
@pytest.mark.parametrize("prefix_tokens", [512, 2048])
def test_bf16_tolerance_of_the_7b_shape(prefix_tokens):
    """The 7B shape at 2 layers with its 64-field schema: the ratio of its
    emulated logit error to the 1.5B shape's 2-layer one, against the
    committed SIGMA_RATIO_7B_L2 (which takes the larger of the two prefix
    lengths' ratios)."""
    wl1 = pi.make_workload("cfg1")
    w1 = pi.make_weights(wl1.shape, wl1.weight_seed, n_layers=2)
    reqs1 = [(r.prefix, r.fields) for r in wl1.requests]
    e1 = opcd.decide(Bf16Emulation(w1), reqs1).z - opcd.decide(odec.Decoder(w1, np.float64), reqs1).z
    del w1
    wl = pi.make_workload("cfg4")
    w = pi.make_weights(wl.shape, wl.weight_seed, n_layers=2)
    reqs = [(wl.requests[0].prefix[:prefix_tokens], wl.requests[0].fields)]
    ref = opcd.decide(odec.Decoder(w, np.float64), reqs)
    emu = opcd.decide(Bf16Emulation(w), reqs)
    ez = emu.z - ref.z
    ratio = float(np.sqrt(np.mean(ez ** 2)) / np.sqrt(np.mean(e1 ** 2)))
    print(f"7B L=2 P={prefix_tokens}: sigma ratio {ratio:.3f}, logit error max {np.max(np.abs(ez)):.3e}", flush=True)
    assert ratio <= tol.SIGMA_RATIO_7B_L2 * 1.03
    assert np.max(np.abs(ez)) <= tol.BF16_7B_L2["z"]
    assert np.max(np.abs(emu.lse - ref.lse)) <= tol.BF16_7B_L2["lse"]
