"""Parity tolerances of the device path against the fp64 oracle.

fp32 model (the tiny decoder): fixed bounds, measured errors are about 1e-6.

bf16 models.  The anchor is the bound the 1.5B-shaped bf16 model is held to
at 2 layers: 2.5e-2 on each logit and log-sum-exp, and the argmax compared
wherever the oracle's top-2 margin is at least 0.05 nats (two logits each
off by 2.5e-2 can swap at most that margin).  The device's error grows
with depth.  test_bf16_bound.py runs an fp32 model of the device's seven
bf16 rounding points per layer (tests/bf16_emulation.py) on the 28-field
request at 2 and at 28 layers and measures the RMS logit error against the
oracle, sigma_2 and sigma_28.  At 2 layers the anchor is about 4.3 sigma_2,
so a request of ~120 compared values exceeds it with probability about 2e-3
if the errors are normal.  At depth L the bound is the same multiple of
sigma_L:

    z_L = 2.5e-2 * sigma_L / sigma_2.

The rest follows from z (first order, for single-readout comparisons):
  - per-token log-score = z - lse: the z bound plus the lse bound;
  - probability q = softmax(logscore / T): |dq| <= q(1-q) * 2 ls <= ls / 2;
  - mass = sum exp(z - lse): relative error <= exp(z + lse) - 1;
  - argmax waiver: single-token candidates share one readout, whose
    log-sum-exp cancels, so two of them move at most 2 z apart (0.05 nats at
    2 layers); deeper paths cross several readouts and move at most 2 ls per
    scored token.
"""
import math

F32 = dict(z=1e-4, ls=1e-4, prob=1e-5, mass=1e-4)

Z_L2 = 2.5e-2        # logits and log-sum-exps, 2 layers
LSE_L2 = 1e-3        # log-sum-exp alone (the emulation's is about 1e-4)
# sigma_28 / sigma_2 of the emulation on the 28-field request; test_bf16_bound
# re-derives it and checks this value (and the bound below) against it
SIGMA_RATIO_28 = 2.65
# sigma of the 7B-shaped model (d 3584, FFN 18944) at 2 layers over sigma_2:
# the emulation gives 2.31 with the workload's first 512 prefix tokens and
# 2.18 with its first 2048 (test_bf16_bound, the 7B case); the larger is used
SIGMA_RATIO_7B_L2 = 2.31


def bf16_bounds(sigma_ratio: float = 1.0) -> dict:
    z = Z_L2 * sigma_ratio
    lse = LSE_L2 * sigma_ratio
    ls = z + lse
    return dict(z=z, lse=lse, ls=ls, prob=ls / 2, mass=math.expm1(z + lse))


BF16_L2 = bf16_bounds(1.0)
BF16_L28 = bf16_bounds(SIGMA_RATIO_28)
BF16_7B_L2 = bf16_bounds(SIGMA_RATIO_7B_L2)


def margin_waiver(bounds: dict, depth: int = 1) -> float:
    """Top-2 margin (nats) below which the argmax is not compared, for a
    field whose deepest scored path has `depth` tokens.  Single-token
    candidates of a field share one readout row, whose log-sum-exp cancels
    in the margin: 2 z.  Deeper paths cross several readouts: 2 ls per
    token."""
    return 2 * bounds["z"] if depth <= 1 else 2 * bounds["ls"] * depth
