#!/usr/bin/env python
"""Benchmark of the PCD hot path on one MI355X.

One step = one whole request through the C ABI: pcd_prefill of the shared
prefix, then pcd_decide of every field in one batched branch pass + readout.
Default workload: the Qwen2.5-1.5B-shaped random-init bf16 decoder, a
512-token prefix and a 28-field schema (10 booleans, 18 four-way enums).
Prints one JSON line: fields decided per second (value: independent
single-pass requests on three streams at once, one in flight per stream)
and p50 request latency (one request at a time), the roofline position of
the dominant kernel (timed live with hipEvents on the library's stream) and
the CPU oracle timed on a bounded sample.
"""
import argparse
import collections
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3


def algorithmic_work(sh, P, Tb, R):
    """Per-launch algorithmic (flops, bytes) of each kernel class: every
    operand read once and every output written once."""
    d, F, V, hd = sh.d_model, sh.ffn_dim, sh.vocab_size, sh.head_dim
    nq, nk = sh.n_heads * hd, sh.n_kv_heads * hd
    e = 2 if sh.dtype == "bf16" else 4
    kv_tok = 2 * nk * e  # K and V of one token in one layer

    def gemm(M, N, K, out_b):
        return 2.0 * M * N * K, float(N * K * e + M * K * e + M * N * out_b)

    w = {}
    w["prefill_qkv"] = gemm(P, nq + 2 * nk, d, e)
    w["prefill_o"] = gemm(P, d, nq, 4)
    w["prefill_gateup"] = gemm(P, 2 * F, d, 0)
    w["prefill_gateup"] = (w["prefill_gateup"][0], w["prefill_gateup"][1] + P * F * e)
    w["prefill_down"] = gemm(P, d, F, 4)
    w["prefill_attn"] = (4.0 * sh.n_heads * hd * P * (P + 1) / 2, float(2 * P * nq * e + P * kv_tok))
    w["branch_qkv"] = gemm(Tb, nq + 2 * nk, d, e)
    w["branch_o"] = gemm(Tb, d, nq, 4)
    w["branch_gateup"] = gemm(Tb, 2 * F, d, 0)
    w["branch_gateup"] = (w["branch_gateup"][0], w["branch_gateup"][1] + Tb * F * e)
    w["branch_down"] = gemm(Tb, d, F, 4)
    # prefix part of the shared-prefix attention: the prefix K/V of a layer read once
    w["branch_attn"] = (4.0 * sh.n_heads * hd * Tb * P, float(P * kv_tok + Tb * nq * e))
    w["readout_lmhead"] = gemm(R, V, d, 0)
    # single-pass mode: the prefix rows and the branch rows in one pass
    Mf = P + Tb
    w["fused_qkv"] = gemm(Mf, nq + 2 * nk, d, e)
    w["fused_o"] = gemm(Mf, d, nq, 4)
    w["fused_gateup"] = gemm(Mf, 2 * F, d, 0)
    w["fused_gateup"] = (w["fused_gateup"][0], w["fused_gateup"][1] + Mf * F * e)
    w["fused_down"] = gemm(Mf, d, F, 4)
    w["fused_attn"] = (w["prefill_attn"][0] + w["branch_attn"][0], w["prefill_attn"][1] + Tb * nq * e)
    return w


BOUND = {"prefill_qkv": "mfma", "prefill_o": "mfma", "prefill_gateup": "mfma", "prefill_down": "mfma",
         "prefill_attn": "mfma", "branch_qkv": "hbm", "branch_o": "hbm", "branch_gateup": "hbm",
         "branch_down": "hbm", "branch_attn": "hbm", "readout_lmhead": "hbm", "fused_qkv": "mfma",
         "fused_o": "mfma", "fused_gateup": "mfma", "fused_down": "mfma", "fused_attn": "mfma"}


def roofline_entry(cls, total_ms, launches, work, peak_mfma):
    flops, nbytes = work[cls]
    avg_s = total_ms / launches / 1e3
    if BOUND[cls] == "mfma":
        a = flops / avg_s / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": peak_mfma, "unit": "TFLOP/s",
                "frac": round(a / peak_mfma, 4), "traffic": None, "kernel": cls,
                "avg_launch_us": round(avg_s * 1e6, 2), "launches": launches,
                "per_launch": {"flops": flops, "bytes": nbytes}}
    a = nbytes / avg_s / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None, "kernel": cls,
            "avg_launch_us": round(avg_s * 1e6, 2), "launches": launches,
            "per_launch": {"flops": flops, "bytes": nbytes}}


def cpu_baseline(weights, wl, n_layers, reps=3):
    """The fp32 oracle, as it stands, on the same request: prefill, branch
    pass, full-vocabulary readout and combine.  With n_layers below the model
    depth, the prefill and branch time is scaled to the full depth."""
    import numpy as np
    from oracle import decoder as odec
    from oracle import pcd as opcd
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    req = wl.requests[0]
    dec = odec.Decoder(weights, np.float32)
    k = n_layers
    L = wl.shape.n_layers
    # cast the used layers and the head to fp32 once, outside the timed part
    for l in range(k):
        for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            dec.mat(f"l{l}.{n}")
    dec.mat(weights.lm_head_name())
    dec.mat("embed")
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        kv = opcd.prefill(dec, req.prefix, n_layers=k)
        plan = opcd.build_plan([(len(req.prefix), req.fields)], wl.shape.vocab_size)
        x = opcd.branch(dec, plan, [kv], n_layers=k)
        t2 = time.perf_counter()
        lse, z = opcd.readout(dec, plan, x)
        opcd.combine(plan, lse, z)
        t3 = time.perf_counter()
        times.append((t2 - t0) * L / k + (t3 - t2))
    est = float(np.median(times))
    nf = len(req.fields)
    what = "all" if k == L else f"the first {k} (prefill and branch time scaled by {L}/{k})"
    return {"value": round(nf / est, 3), "unit": "fields/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp32 NumPy oracle on the bench request (P={len(req.prefix)}, {nf} fields), {what} of {L} "
                       f"layers plus the full readout and combine; p50 of {reps} runs: {est:.2f} s per request"),
            "request_s": round(est, 3)}


def kernel_source_sha():
    import hashlib
    src = os.path.join(ROOT, "constrained_decoding_pcd_amd", "csrc", "pcd_kernels.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()


def measured_traffic(cls):
    """HBM bytes per launch of kernel class `cls` from the committed rocprofv3
    counter summary, or None when there is none for it or the kernel source
    has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{cls}_cfg1_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_class") != cls or kv.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return float(kv["traffic_bytes_per_launch"])


def copy_calibration(nbytes):
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 5}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cfg1", help="cfg0 (tiny) or cfg1 (1.5B, 512-token prefix, 28 fields)")
    ap.add_argument("--cpu-layers", type=int, default=28, help="layers of the CPU-oracle sample (0: skip)")
    ap.add_argument("--warm-input", type=int, default=100,
                    help="warm request: the prefix minus this many tokens is a cached head (0: skip)")
    ap.add_argument("--mode", choices=("both", "single-pass", "two-pass"), default="both",
                    help="request modes to time; the faster timed mode is the headline")
    ap.add_argument("--no-token-by-token", action="store_true", help="skip the token-by-token baseline")
    ap.add_argument("--concurrent-streams", type=int, default=3,
                    help="streams of the throughput loop (0: skip it; value is then one request at a time). "
                         "Profiles of kernel durations use 0, so that no two kernels overlap")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the path is single-GPU by design (requests are independent and "
              "would shard over GPUs with no communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import constrained_decoding_pcd_amd as cpd
    import pcd_inputs as pi
    from constrained_decoding_pcd_amd import greedy

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = pi.make_workload(args.workload)
    sh = wl.shape
    req = wl.requests[0]
    t = time.time()
    weights = pi.make_weights(sh, wl.weight_seed)
    print(f"# weights drawn in {time.time() - t:.1f} s", file=sys.stderr, flush=True)
    dev = cpd.upload_weights(weights.mats, sh.n_layers, sh.d_model, "cuda:0")
    plan = cpd.debug_plan(sh.vocab_size, sh.max_seq, [len(req.prefix)], [req.fields])
    Tb, R = len(plan["tok"]), len(plan["ro_tok"])
    # room for the single-pass mode: the prefix rows and the branch rows in one pass
    lim = cpd.limits_for(sh.vocab_size, sh.max_seq, [len(req.prefix)], [req.fields], len(req.prefix) + Tb)
    model = cpd.PcdModel(cpd.config_of(sh), dev, lim)
    kv = torch.empty(model.state_bytes(len(req.prefix)), dtype=torch.uint8, device="cuda:0")
    # the schema's Python lists are turned into C arrays once, as a server does
    # for a schema it serves many times; the library validates it and builds
    # the plan on every request
    schema = model.compile_fields(req.fields)
    prompt = np.asarray(req.prefix, dtype=np.int32)  # token ids as a tokenizer hands them over

    def step_two_pass():  # prefill pass, then the branch pass
        st = model.prefill(prompt, kv)
        out = model.decide(st, schema)
        st.close()
        return out

    def step_single_pass():  # an empty state; the prefix rows and the branch rows in one pass
        st = model.new_state(len(req.prefix), kv)
        out = model.extend_decide(st, prompt, schema)
        st.close()
        return out

    def timed(step, fused):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        lat = []
        gc.collect()
        gc.disable()  # no collector pause inside the timed steps
        t0 = time.perf_counter()
        for _ in range(args.steps):
            s0 = time.perf_counter()
            out = step()
            lat.append(time.perf_counter() - s0)
        torch.cuda.synchronize()
        gc.enable()
        r = {"ms_per_step": (time.perf_counter() - t0) / args.steps * 1e3,
             "p50_request_ms": float(np.percentile(np.array(lat) * 1e3, 50)),
             "p90_request_ms": float(np.percentile(np.array(lat) * 1e3, 90)), "out": out,
             "max_request_ms": float(np.max(lat) * 1e3), "slowest_step": int(np.argmax(lat))}
        st = model.stats()
        # the single-pass mode runs no prefill pass: its one pass is the branch pass
        r["phases_ms"] = {k: round(st[f"last_{k}_ms"], 4) for k in ("prefill", "branch", "readout")}
        if fused:
            r["phases_ms"] = {"fused": r["phases_ms"]["branch"], "readout": r["phases_ms"]["readout"]}
        return r

    nf = len(req.fields)
    modes = {}
    if args.mode in ("both", "two-pass"):
        modes["two-pass"] = timed(step_two_pass, False)
    if args.mode in ("both", "single-pass"):
        modes["single-pass"] = timed(step_single_pass, True)
    # the headline mode: the lower p50 (a single slow step must not decide it)
    mode = min(modes, key=lambda k: modes[k]["p50_request_ms"])
    head = modes[mode]
    step, out = (step_single_pass if mode == "single-pass" else step_two_pass), head["out"]
    ms_per_step, p50, p90 = head["ms_per_step"], head["p50_request_ms"], head["p90_request_ms"]
    for k, r in modes.items():
        print(f"# {k}: {args.steps} steps: {r['ms_per_step']:.3f} ms/step, p50 {r['p50_request_ms']:.3f} ms, "
              f"p90 {r['p90_request_ms']:.3f} ms", file=sys.stderr, flush=True)
    phases = dict(head["phases_ms"])
    dev_ms = sum(phases.values())

    # Pipelined throughput: the next request is started (validated, planned,
    # its plan uploaded and its pass enqueued) before the previous one is
    # finished, so the host's per-request work runs while the device works.
    # Each in-flight request has its own KV buffer; every request does the
    # whole single pass and its readout.
    pipelined = None
    if "single-pass" in modes:
        depth = 2
        kvs = [kv] + [torch.empty_like(kv) for _ in range(depth - 1)]

        def run_pipelined(n):
            pend, outs = collections.deque(), []
            for i in range(n):
                st = model.new_state(len(req.prefix), kvs[i % depth])
                pend.append((model.extend_decide_start(st, prompt, schema), st))
                if len(pend) == depth:
                    p_, s_ = pend.popleft()
                    outs.append(p_.finish())
                    s_.close()
            while pend:
                p_, s_ = pend.popleft()
                outs.append(p_.finish())
                s_.close()
            return outs

        run_pipelined(args.warmup)
        torch.cuda.synchronize()
        gc.collect()
        gc.disable()
        t0 = time.perf_counter()
        pouts = run_pipelined(args.steps)
        torch.cuda.synchronize()
        pl_ms = (time.perf_counter() - t0) / args.steps * 1e3
        gc.enable()
        ref_out = modes["single-pass"]["out"]
        same = all(np.array_equal(o[k], ref_out[k]) for o in pouts for k in ("prob", "mass", "argmax"))
        pipelined = {"depth": depth, "ms_per_request": round(pl_ms, 4), "fields_per_s": round(nf / (pl_ms / 1e3), 2),
                     "same_results_as_one_at_a_time": bool(same)}
        print(f"# pipelined (depth {depth}): {pl_ms:.3f} ms/request", file=sys.stderr, flush=True)

    # Concurrent throughput: independent requests on three streams at once,
    # each stream with its own model (its own workspace and start/finish
    # slots) over the same device weights, one request in flight per stream.
    # The kernels of one request fill the compute units that another's leave
    # idle (launch ramps, the tails of partial last rounds, latency-bound
    # attention).  Each request still does its whole single pass and readout.
    concurrent = None
    if "single-pass" in modes and args.concurrent_streams > 0:
        # 3 by default: a fourth stream gained 1% on one box and lost 6% on another
        n_conc = args.concurrent_streams
        cmodels = [model] + [cpd.PcdModel(cpd.config_of(sh), dev, lim) for _ in range(n_conc - 1)]
        cschemas = [schema] + [m_.compile_fields(req.fields) for m_ in cmodels[1:]]
        cstreams = [torch.cuda.Stream() for _ in range(n_conc)]
        ckvs = kvs + [torch.empty_like(kv) for _ in range(n_conc - len(kvs))]

        def run_concurrent(n):
            pend, outs = collections.deque(), []
            for i in range(n):
                k = i % n_conc
                with torch.cuda.stream(cstreams[k]):
                    st = cmodels[k].new_state(len(req.prefix), ckvs[k])
                    pend.append((cmodels[k].extend_decide_start(st, prompt, cschemas[k]), st))
                if len(pend) == n_conc:
                    p_, s_ = pend.popleft()
                    outs.append(p_.finish())
                    s_.close()
            while pend:
                p_, s_ = pend.popleft()
                outs.append(p_.finish())
                s_.close()
            return outs

        run_concurrent(max(args.warmup, n_conc))
        torch.cuda.synchronize()
        gc.collect()
        gc.disable()
        t0 = time.perf_counter()
        couts = run_concurrent(args.steps)
        torch.cuda.synchronize()
        cc_ms = (time.perf_counter() - t0) / args.steps * 1e3
        gc.enable()
        same = all(np.array_equal(o[k], ref_out[k]) for o in couts for k in ("prob", "mass", "argmax"))
        concurrent = {"streams": n_conc, "ms_per_request": round(cc_ms, 4),
                      "fields_per_s": round(nf / (cc_ms / 1e3), 2), "same_results_as_one_at_a_time": bool(same)}
        print(f"# concurrent ({n_conc} streams): {cc_ms:.3f} ms/request", file=sys.stderr, flush=True)
        for m_ in cmodels[1:]:
            m_.close()

    # Warm requests: the prefix's first tokens are a cached head; each request
    # forks it, appends its own input tokens and decides (one extend + one
    # branch pass), or runs the first-field round on top (decide field 0,
    # append its answer, decide the rest: two extends + two branch passes).
    warm = None
    if 0 < args.warm_input < len(req.prefix):
        head_n = len(req.prefix) - args.warm_input
        f0 = req.fields[0]
        cap = len(req.prefix) + len(f0.scaffold) + max(len(c) for c in f0.candidates)
        head_st = model.prefill(req.prefix[:head_n])
        kv_w = torch.empty(model.state_bytes(cap), dtype=torch.uint8, device="cuda:0")

        def warm_step(kind):
            st = head_st.fork(kv=kv_w)
            if kind == "single_pass_p50_ms":
                model.extend_decide(st, prompt[head_n:], schema)
            else:
                st.extend(prompt[head_n:])
                if kind == "first_field_round_p50_ms":
                    model.decide_sequenced(st, schema, 1)
                else:
                    model.decide(st, schema)
            st.close()

        warm = {"head_tokens": head_n, "input_tokens": args.warm_input}
        for key in ("single_pass_p50_ms", "two_pass_p50_ms", "first_field_round_p50_ms"):
            for _ in range(args.warmup):
                warm_step(key)
            torch.cuda.synchronize()
            lw = []
            gc.collect()
            gc.disable()
            for _ in range(args.steps):
                s0 = time.perf_counter()
                warm_step(key)
                lw.append(time.perf_counter() - s0)
            gc.enable()
            warm[key] = round(float(np.percentile(np.array(lw) * 1e3, 50)), 4)
        head_st.close()

    # The token-by-token baseline on the same kernels: the prefill, then one
    # decoder pass per output token (every scaffold token and label token of
    # the 28 fields, each field written after the earlier answers).
    token_by_token = None
    if not args.no_token_by_token:
        greedy.decode(model, req.prefix, req.fields[:2])
        torch.cuda.synchronize()
        gc.collect()
        gc.disable()
        t0 = time.perf_counter()
        gd = greedy.decode(model, req.prefix, req.fields)
        torch.cuda.synchronize()
        tbt_ms = (time.perf_counter() - t0) * 1e3
        gc.enable()
        token_by_token = {"request_ms": round(tbt_ms, 3), "passes": gd.passes,
                          "ms_per_pass": round(tbt_ms / gd.passes, 4), "pcd_speedup": round(tbt_ms / p50, 1),
                          "same_answers": int(sum(int(a == b) for a, b in zip(gd.labels, out["argmax"])))}
        print(f"# token-by-token: {gd.passes} passes, {tbt_ms:.1f} ms", file=sys.stderr, flush=True)

    # the same steps again with every kernel launch bracketed by hipEvents on the library's stream
    model.set_kernel_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = model.kernel_times()
    model.set_kernel_timing(False)
    work = algorithmic_work(sh, len(req.prefix), Tb, R)
    peak_mfma = BF16_PEAK_TFLOPS if sh.dtype == "bf16" else FP32_PEAK_TFLOPS
    kernels = {c: roofline_entry(c, ms, n, work, peak_mfma) for c, (ms, n) in kt.items() if n > 0 and c in work}
    dominant = max(kernels, key=lambda c: kt[c][0])
    traffic = measured_traffic(dominant)
    if traffic is not None:
        kernels[dominant]["traffic"] = traffic
    timed_ms_per_step = sum(ms for ms, _ in kt.values()) / args.steps
    # Phase rooflines (hipEvent phase times of the timed steps): the branch
    # pass against HBM (every weight matrix, the prefix K/V read once, the
    # branch K/V and activations), prefill and the single pass against
    # MFMA, the readout against HBM (the LM head).
    def phase_roofline():
        out = {}
        e = 2 if sh.dtype == "bf16" else 4
        P = len(req.prefix)
        w_bytes = float(sum(work[c][1] for c in ("branch_qkv", "branch_o", "branch_gateup", "branch_down")))
        kv_tok = sh.n_layers * 2 * sh.n_kv_heads * sh.head_dim * e
        br_bytes = w_bytes * sh.n_layers + P * kv_tok + Tb * kv_tok
        # The last layer of a pass does only the work later steps read: QKV of
        # every row (the K/V), then, in a pass with readouts, the branch rows'
        # attention and the readout rows' O projection and MLP.
        d, F, nq = sh.d_model, sh.ffn_dim, sh.n_heads * sh.head_dim
        last_r = 2.0 * R * (d * nq + 2 * F * d + d * F)
        pf_flops = sum(work[c][0] for c in ("prefill_qkv", "prefill_o", "prefill_gateup", "prefill_down",
                                            "prefill_attn")) * (sh.n_layers - 1) + work["prefill_qkv"][0]
        fu_flops = (sum(work[c][0] for c in ("fused_qkv", "fused_o", "fused_gateup", "fused_down",
                                             "fused_attn")) * (sh.n_layers - 1)
                    + work["fused_qkv"][0] + work["branch_attn"][0] + last_r)
        ro_bytes = float(work["readout_lmhead"][1])
        if "two-pass" in modes:
            ph = modes["two-pass"]["phases_ms"]
            out["branch_pass"] = {"ms": ph["branch"], "bytes": br_bytes,
                                  "GB/s": round(br_bytes / ph["branch"] / 1e6, 1),
                                  "hbm_frac": round(br_bytes / ph["branch"] / 1e6 / HBM_PEAK_GBS, 4)}
            out["prefill"] = {"ms": ph["prefill"], "flops": pf_flops,
                              "TFLOP/s": round(pf_flops / ph["prefill"] / 1e9, 1),
                              "mfma_frac": round(pf_flops / ph["prefill"] / 1e9 / peak_mfma, 4)}
        if "single-pass" in modes:
            ph = modes["single-pass"]["phases_ms"]
            out["single_pass"] = {"ms": ph["fused"], "flops": fu_flops,
                                  "TFLOP/s": round(fu_flops / ph["fused"] / 1e9, 1),
                                  "mfma_frac": round(fu_flops / ph["fused"] / 1e9 / peak_mfma, 4)}
        ro = head["phases_ms"]["readout"]
        out["readout"] = {"ms": ro, "bytes": ro_bytes, "GB/s": round(ro_bytes / ro / 1e6, 1),
                          "hbm_frac": round(ro_bytes / ro / 1e6 / HBM_PEAK_GBS, 4)}
        return out
    # whole-job throughput: the concurrent loop where it ran (every request
    # still does all of its work), else the headline mode's steps
    thr_ms = concurrent["ms_per_request"] if concurrent else ms_per_step
    res = {
        "metric": "schema fields decided/sec + p50 28-field request ms, 1.5B-shaped bf16",
        "value": round(nf / (thr_ms / 1e3), 2),
        "unit": "fields/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(thr_ms, 4),
        "p50_request_ms": round(p50, 4),
        "p90_request_ms": round(p90, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sh.dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {sh.name} random-init {sh.dtype}, {len(req.prefix)}-token "
                               f"prefix, {nf} fields, {Tb} branch tokens, {R} readouts, batch 1",
                   "layers": sh.n_layers, "prefix_tokens": len(req.prefix), "fields": nf,
                   "branch_tokens": Tb, "readouts": R, "mode": mode,
                   "schema": "marshalled to C arrays once; validated and planned on every request",
                   "throughput": (f"single-pass requests on {concurrent['streams']} streams at once, one in "
                                  f"flight per stream (start/finish calls)" if concurrent
                                  else f"{mode} requests one at a time"),
                   "latency": f"{mode} requests one at a time"},
        "phases_ms": phases,
        "device_fields_per_s": round(nf / (dev_ms / 1e3), 2),
        "passes": dict({"fused": 1} if mode == "single-pass" else {"prefill": 1, "branch": 1},
                       token_by_token_equivalent=int(sum(len(f.scaffold) + len(f.candidates[int(a)])
                                                         for f, a in zip(req.fields, out["argmax"])))),
        "modes": {k: {"ms_per_step": round(r["ms_per_step"], 4), "p50_request_ms": round(r["p50_request_ms"], 4),
                      "max_request_ms": round(r["max_request_ms"], 4), "slowest_step": r["slowest_step"],
                      "phases_ms": r["phases_ms"]} for k, r in modes.items()},
        "roofline": kernels[dominant],
        "phase_roofline": phase_roofline(),
        "kernels": {c: {k: v for k, v in e.items() if k in ("achieved", "unit", "frac", "avg_launch_us",
                                                            "launches", "bound")} for c, e in kernels.items()},
        "kernel_timed_ms_per_step": round(timed_ms_per_step, 4),
    }
    if concurrent is not None:
        res["concurrent"] = concurrent
    if pipelined is not None:
        res["pipelined"] = pipelined
        res["one_at_a_time_fields_per_s"] = round(nf / (ms_per_step / 1e3), 2)
    if token_by_token is not None:
        res["token_by_token"] = token_by_token
    if warm is not None:
        res["warm"] = warm
    if args.cpu_layers > 0:
        print("# timing the CPU oracle sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(weights, wl, min(args.cpu_layers, sh.n_layers))
        res["cpu_baseline"]["gpu_speedup"] = round(res["value"] / res["cpu_baseline"]["value"], 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
