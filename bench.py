#!/usr/bin/env python3
"""Benchmark of the looped transformer's hot path on one MI355X.

Step: one forward scoring pass of the 2048-wide model with an INT4 shared loop
block (vocab 50304, 16 heads x 128, SwiGLU 5632, 1 pre block, 1 x 128 tokens,
L = 8, no logits) with inputs resident in HBM.  Reported value: token-loop
iterations per second (128 tokens x 8 iterations per step); ms_per_step is the
milliseconds per seq-128 L = 8 forward.  Secondary fields: greedy cached decode
tok/s at L = 8 on the FP16-body model (32 lanes, 32-token prompts), the FP16-body
32 x 128 forward at L = 2, 8 and 32, L-aware INT4 decode (64 lanes), the
Infinity-Cache residency control, shared-prefix reuse, self-speculative and
store-h decoding, the 5280-wide continuous-depth workload (prefill, continuous
depth and lockstep decode), and the CPU oracle timed on the host.

Prints one JSON line.  Synthetic seeded weights and token ids (no checkpoint).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0
PAGES_H100_INT4_MS = 30.48     # the pages' H100 INT4 forward at seq 128, loops 8 (context)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefix", action="store_true", help="skip the shared-prefix measurement")
    ap.add_argument("--no-spec", action="store_true", help="skip the self-speculative measurement")
    ap.add_argument("--no-store-h", action="store_true", help="skip the store-h cache-mode measurement")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the FP16-body 32 x 128 forwards, the L-aware 64-lane INT4 decode and the MALL control")
    ap.add_argument("--no-cfg5", action="store_true", help="skip the 5280-wide continuous-depth workload")
    ap.add_argument("--profile-only", action="store_true", help="run the timed steps only (for rocprofv3)")
    ap.add_argument("--profile-decode", action="store_true",
                    help="run batch-1 INT4 decode steps only (32-token prompt, 63 steps at L=8; for rocprofv3)")
    ap.add_argument("--profile-decode-fp16", action="store_true",
                    help="run 32-lane FP16-body decode steps only (32-token prompts, 31 steps at L=8; for rocprofv3)")
    ap.add_argument("--profile-lane-aware", action="store_true",
                    help="run the 64-lane L-aware INT4 decode steps only (for rocprofv3)")
    ap.add_argument("--eager", action="store_true", help="launch kernels one by one (no graph replay)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the steps, copy 256 MiB once with a plain device copy (counter calibration)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def gemm_source_sha256() -> str:
    """Hash of the sources the GEMM kernels are compiled from (counters go stale when they change)."""
    h = hashlib.sha256()
    for name in ("gemm.hip", "epilogue.h", "device_common.h"):
        h.update(open(os.path.join(ROOT, "looped_transformer_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def traffic_for(kernel_class: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel source is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % kernel_class)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("gemm_source_sha256") != gemm_source_sha256():
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds: float):
    """The fp64 numpy oracle on the host: the same cfg-2 forward (1 x 128 tokens,
    L = 8), with every BLAS thread for about `seconds`, then one forward on one
    thread."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_info, threadpool_limits
    spec = synth.SPECS[2]
    w = synth.make_weights(spec, 0)
    m = oracle.OracleModel.from_weights(w)
    toks = synth.tokens(0, synth.STREAM_TOKENS, 128, spec.vocab)
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill(m, toks, 8, want_logits="none")
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds or runs >= 50:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        oracle.prefill(m, toks, 8, want_logits="none")
        el1 = time.perf_counter() - t1
    return {"value": round(1024 * runs / el, 1), "unit": "token-loop iterations/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "%d full forwards of the same workload (1x128 tokens, L=8) by the fp64 numpy oracle, %.1f s"
                      % (runs, el),
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "one_thread": {"value": round(1024 / el1, 1), "unit": "token-loop iterations/s", "cores": 1,
                           "sample": "one forward of the same workload on one BLAS thread, %.1f s" % el1}}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (lanes would be sharded across "
              "GPUs with replicated weights). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import looped_transformer_amd as tl
    import synth
    from tests.harness import ensure_built, kv_bytes, load_model

    ensure_built()
    if args.profile_decode:
        profile_decode(tl, torch, np, synth, kv_bytes, load_model)
        return
    if args.profile_lane_aware:
        lane_aware_bench(tl, torch, np, synth, kv_bytes, load_model)
        return
    if args.profile_decode_fp16:
        profile_decode_fp16(tl, torch, np, synth, kv_bytes, load_model)
        return
    spec = synth.SPECS[2]
    log("generating weights")
    w = synth.make_weights(spec, 0)
    model = load_model(w, max_pos=256)
    toks = torch.tensor(synth.tokens(0, synth.STREAM_TOKENS, 128, spec.vocab), dtype=torch.int32, device="cuda")
    cu = np.array([0, 128], np.int32)
    hid = torch.empty(128, spec.d_model, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    # a dedicated stream: repeated identical scoring calls replay a captured HIP graph
    stream = 0 if args.eager else torch.cuda.Stream()

    def step():
        tl.tl_forward(model, cu, toks, L=8, out_hidden=hid, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timed region: %d steps" % args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = el / args.steps * 1e3
    value = 128 * 8 / (ms / 1e3)
    if args.profile_only:
        log("ms/step %.4f" % ms)
        if args.calibrate_copy:
            src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
            log("copied %d bytes" % (src.numel() * 4))
        return

    # per-kernel-class HIP-event timing over a second timed region of the same steps,
    # eager launches on the forward's stream: a pair recorded around each launch
    # group (dispatch and event overhead included), and for every kernel a pair the
    # runtime stamps with the kernel's own start and end (used below)
    tl.tl_timing_enable(model, True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    cls = tl.tl_timing_read(model)
    kcls = tl.tl_timing_read_kernels(model)
    tl.tl_timing_enable(model, False)
    M, d, F = 128, spec.d_model, spec.ffn
    flops = {"gemm_qkv_loop": 2 * M * 3 * d * d, "gemm_o_loop": 2 * M * d * d,
             "gemm_gu_loop": 2 * M * 2 * F * d, "gemm_down_loop": 2 * M * d * F}
    dom = max(flops, key=lambda k: kcls[k][0])
    k_ms, nk = kcls[dom]
    tot_ms, n = cls[dom]
    avg_s = k_ms / n / 1e3          # kernel time per launch group (one kernel per group here)
    achieved = flops[dom] / avg_s / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": traffic_for(dom),
                "avg_launch_us": round(avg_s * 1e6, 2), "launches": n, "kernels": nk,
                "timing": "kernel start/end stamped by the runtime (hipExtLaunchKernel event pairs)",
                "event_pair_us": round(tot_ms / n * 1e3, 2),
                "algorithmic_flops_per_launch": flops[dom]}
    breakdown = {k: round(v[0] / args.steps * 1e3, 2) for k, v in kcls.items() if v[1]}
    tl.tl_free(model)
    del model

    out = {"metric": "token-loop iterations/sec + ms per seq128 L=8 forward; decode tok/s at L=8",
           "value": round(value, 1), "unit": "token-loop iterations/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": round(PAGES_H100_INT4_MS / ms, 2), "dtype": "f16", "data": "synthetic",
           "config": {"workload": "forward scoring, INT4 (W4G128) shared loop block, d_model 2048, 16x128 heads, "
                                  "SwiGLU 5632, vocab 50304, 1 pre block, batch 1, seq_len 128, L=8, no logits",
                      "batch": 1, "seq_len": 128, "L": 8, "parallelism": "single GPU"},
           "roofline": roofline, "us_per_step_by_kernel_class": breakdown,
           "baseline_note": "vs_baseline = the pages' H100 INT4 forward (30.48 ms, same workload) / ms_per_step; "
                            "another machine's number, context only"}

    if not args.no_decode:
        out["decode_L8"] = decode_bench(tl, torch, np, synth, kv_bytes, load_model)
    if not args.no_extra_configs:
        w3 = synth.make_weights(synth.SPECS[3], 0)
        for L in (2, 8, 32):
            out["forward_fp16_L%d" % L] = forward_fp16_bench(tl, torch, np, synth, load_model, w3, L)
        del w3
        out["decode_lane_aware"] = lane_aware_bench(tl, torch, np, synth, kv_bytes, load_model)
        out["mall_control"] = mall_bench(tl, torch, np, synth, load_model)
    if not args.no_prefix:
        out["shared_prefix"] = prefix_bench(tl, torch, np, synth, kv_bytes, load_model)
    if not args.no_spec:
        out["speculative_B1"] = spec_bench(tl, torch, np, synth, kv_bytes, load_model)
    if not args.no_store_h:
        out["store_h_B1"] = store_h_bench(tl, torch, np, synth, kv_bytes, load_model)
    if not args.no_cfg5:
        torch.cuda.empty_cache()
        out["cfg5_continuous_depth"] = cfg5_bench(tl, torch, np, synth, kv_bytes, load_model)
    if not args.no_cpu_baseline:
        log("cpu baseline")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


def profile_decode(tl, torch, np, synth, kv_bytes, load_model):
    """Batch-1 greedy decode on the INT4 model (32-token prompt, 63 steps at L = 8),
    nothing else: the workload of the batch-1 kernel statistics."""
    spec = synth.SPECS[2]
    w = synth.make_weights(spec, 0)
    model = load_model(w, max_lanes=1, max_pos=128, max_L=8, kv_arena_bytes=kv_bytes(spec, [8], [128]))
    prompt = torch.tensor(synth.tokens(0, synth.STREAM_PROMPT_TOKENS, 32, spec.vocab), dtype=torch.int32,
                          device="cuda")
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    tl.tl_forward(model, np.array([0, 32], np.int32), prompt, L=8, lanes=[0], max_new_tokens=64)
    for _ in range(63):
        tl.tl_decode_step(model, [0], [8], out)
    torch.cuda.synchronize()
    log("decoded 63 tokens")
    tl.tl_free(model)


def profile_decode_fp16(tl, torch, np, synth, kv_bytes, load_model):
    """The decode workload of decode_bench without early exit: FP16-body model, 32
    lanes, 32-token prompts, 31 greedy steps at L = 8."""
    spec = synth.SPECS[3]
    w = synth.make_weights(spec, 0)
    n, plen, new = 32, 32, 32
    model = load_model(w, max_lanes=n, max_pos=plen + new, kv_arena_bytes=kv_bytes(spec, [8] * n, [plen + new] * n))
    toks = torch.tensor(synth.tokens(0, synth.STREAM_PROMPT_TOKENS, n * plen, spec.vocab), dtype=torch.int32,
                        device="cuda")
    cu = np.arange(0, n * plen + 1, plen, dtype=np.int32)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    tl.tl_forward(model, cu, toks, L=8, lanes=list(range(n)), max_new_tokens=new)
    for _ in range(new - 1):
        tl.tl_decode_step(model, list(range(n)), [8] * n, out)
    torch.cuda.synchronize()
    log("decoded %d steps on %d lanes" % (new - 1, n))
    tl.tl_free(model)


HBM_PEAK_GBPS = 8000.0


def block_weight_bytes(spec, w4):
    """Bytes of one block's weights: fp16, or W4G128 nibbles plus one fp16 scale per
    128-wide group."""
    params = 4 * spec.d_model * spec.d_model + 3 * spec.d_model * spec.ffn
    return params // 2 + params // 128 * 2 if w4 else 2 * params


def decode_step_bytes(spec, loop_w4, lane_L, ctx):
    """Algorithmic HBM bytes of one cached decode step: the pre/post blocks (fp16), the
    loop stack once per iteration up to the deepest lane, the head (fp16), and each
    lane's K/V (fp16) of every slot it attends over ctx positions."""
    d = spec.d_model
    weights = ((spec.n_pre + spec.n_post) * block_weight_bytes(spec, False)
               + int(max(lane_L)) * spec.n_loop * block_weight_bytes(spec, loop_w4) + spec.vocab * d * 2)
    kv = sum((spec.n_pre + int(L) * spec.n_loop + spec.n_post) * ctx * 2 * d * 2 for L in lane_L)
    return weights + kv


def hbm_rate(nbytes, seconds):
    gbps = nbytes / seconds / 1e9
    return {"algorithmic_bytes_per_step": int(nbytes), "achieved_GBps": round(gbps, 1),
            "peak_GBps": HBM_PEAK_GBPS, "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def forward_fp16_bench(tl, torch, np, synth, load_model, w, L):
    """Scoring forward of 32 x 128 tokens at depth L on the FP16-body model (4096 rows
    per pass), graph-replayed like the main forward; best of 3 timed runs of 5 calls."""
    spec = synth.SPECS[3]
    log("forward: FP16-body model, 32 x 128 tokens, L=%d" % L)
    n, T = 32, 128
    model = load_model(w, max_pos=256)
    toks = torch.tensor(synth.tokens(0, synth.STREAM_TOKENS, n * T, spec.vocab), dtype=torch.int32, device="cuda")
    cu = np.arange(0, n * T + 1, T, dtype=np.int32)
    hid = torch.empty(n * T, spec.d_model, dtype=torch.float32, device="cuda")
    ds = torch.cuda.Stream()
    for _ in range(3):
        tl.tl_forward(model, cu, toks, L=L, out_hidden=hid, stream=ds)
    torch.cuda.synchronize()
    best = 1e9
    for _ in range(3):
        t0 = time.perf_counter()
        for _ in range(5):
            tl.tl_forward(model, cu, toks, L=L, out_hidden=hid, stream=ds)
        torch.cuda.synchronize()
        best = min(best, (time.perf_counter() - t0) / 5)
    tl.tl_free(model)
    d = spec.d_model
    per_token_block = 2 * (4 * d * d + 3 * d * spec.ffn)
    flops = n * T * (spec.n_pre + L * spec.n_loop + spec.n_post) * per_token_block \
        + n * (spec.n_pre + L * spec.n_loop + spec.n_post) * 4 * (T * T // 2) * d
    tf = flops / best / 1e12
    return {"config": "FP16-body loop block (2048-wide), 32 sequences x 128 tokens, L=%d, no logits" % L,
            "ms": round(best * 1e3, 3), "token_iterations_per_s": round(n * T * L / best, 1),
            "mfma": {"algorithmic_flops": int(flops), "achieved_TFLOPs": round(tf, 1), "peak_TFLOPs": PEAK_F16_TFLOPS,
                     "frac": round(tf / PEAK_F16_TFLOPS, 4)}}


def lane_aware_bench(tl, torch, np, synth, kv_bytes, load_model):
    """L-aware batched decode on the INT4 model: 64 lanes, per-lane depth drawn from
    {2, 4, 8, 16, 32}, 32-token prompts, 31 cached greedy steps; best of 2 runs."""
    ds = torch.cuda.Stream()
    spec = synth.SPECS[4]
    log("decode: L-aware lanes, INT4 model")
    w = synth.make_weights(spec, 0)
    n, plen, new = 64, 32, 32
    lane_L = synth.lane_loops(0, n)
    model = load_model(w, max_lanes=n, max_pos=plen + new, max_L=int(lane_L.max()),
                       kv_arena_bytes=kv_bytes(spec, lane_L, [plen + new] * n))
    toks = torch.tensor(synth.tokens(0, synth.STREAM_PROMPT_TOKENS, n * plen, spec.vocab), dtype=torch.int32,
                        device="cuda")
    cu = np.arange(0, n * plen + 1, plen, dtype=np.int32)
    lanes = np.arange(n, dtype=np.int32)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    best = 1e9
    for _ in range(2):
        tl.tl_forward(model, cu, toks, seq_L=lane_L, lanes=lanes, max_new_tokens=new, stream=ds)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(new - 1):
            tl.tl_decode_step(model, lanes, lane_L, out, stream=ds)
        torch.cuda.synchronize()
        best = min(best, time.perf_counter() - t0)
    tl.tl_free(model)
    step_s = best / (new - 1)
    ctx = plen + new / 2
    return {"config": "INT4 loop block (2048-wide), 64 lanes, per-lane L from {2, 4, 8, 16, 32} (seed 0), "
                      "32-token prompts, 31 cached greedy steps",
            "lane_L_sum": int(lane_L.sum()), "ms_per_step": round(step_s * 1e3, 4),
            "token_iterations_per_s": round(int(lane_L.sum()) / step_s, 1), "tok_per_s": round(n / step_s, 1),
            "hbm": hbm_rate(decode_step_bytes(spec, True, lane_L, ctx), step_s)}


def decode_bench(tl, torch, np, synth, kv_bytes, load_model):
    """32 lanes, 32-token prompts, greedy cached decode at L = 8 on the FP16-body model;
    the same run with the device-side early-exit rule at three settings."""
    ds = torch.cuda.Stream()
    spec = synth.SPECS[3]
    log("decode: FP16-body model")
    w = synth.make_weights(spec, 0)
    n, plen, new = 32, 32, 32
    model = load_model(w, max_lanes=n, max_pos=plen + new, kv_arena_bytes=kv_bytes(spec, [8] * n, [plen + new] * n))
    prompts = synth.tokens(0, synth.STREAM_PROMPT_TOKENS, n * plen, spec.vocab)
    toks = torch.tensor(prompts, dtype=torch.int32, device="cuda")
    cu = np.arange(0, n * plen + 1, plen, dtype=np.int32)
    lanes = np.arange(n, dtype=np.int32)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    Ls = np.full(n, 8, np.int32)

    def run(step):
        times, depth = [], 0
        for rep in range(3):
            tl.tl_forward(model, cu, toks, L=8, lanes=lanes, max_new_tokens=new, stream=ds)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            tot = 0
            for _ in range(new - 1):
                tot += int(np.sum(step()))
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
            depth = tot / (n * (new - 1))
        best = min(times)
        return {"tok_per_s": round(n * (new - 1) / best, 1), "ms_per_step": round(best / (new - 1) * 1e3, 4),
                "mean_depth": round(depth, 3)}

    res = run(lambda: tl.tl_decode_step(model, lanes, Ls, out, stream=ds))
    res["config"] = ("FP16-body loop block, 32 lanes, 32-token prompts, 31 cached greedy steps at L=8 "
                     "(first token comes from the prefill)")
    res["hbm"] = hbm_rate(decode_step_bytes(spec, False, Ls, plen + new / 2), res["ms_per_step"] / 1e3)
    ee = {
        # relative-L2 rule that never fires: the cost of probing every iteration from 2 on
        "hidden_rule_never_fires": dict(patience=1, min_L=2, tau=0.0),
        # the pages' logit-margin setting (margin 3, patience 1, peek every 2, min L 4)
        "margin3_patience1_peek2_minL4": dict(patience=1, min_L=4, peek_every=2, logit_margin=3.0),
        # every token finishes at iteration 4: iterations 5..8 run gated kernels only
        "all_finish_at_4": dict(patience=1, min_L=4, tau=1e30),
    }
    res["early_exit"] = {k: run(lambda kw=kw: tl.tl_decode_step_ee(model, lanes, Ls, out, **kw, stream=ds))
                         for k, kw in ee.items()}
    tl.tl_free(model)
    return res


def prefix_bench(tl, torch, np, synth, kv_bytes, load_model):
    """Requests that share a prompt prefix, on the INT4 model at L = 8: each request
    is the prefix plus 16 tokens of its own, then 32 greedy tokens (the first from
    the prompt pass, 31 cached steps).  NO_CACHE prefills every full prompt (one
    batched pass); SHARED prefills the prefix once, forks it into every request's
    lane and appends the suffixes (one batched pass).  Wall time of the whole job,
    best of two runs."""
    ds = torch.cuda.Stream()
    spec = synth.SPECS[2]
    log("shared prefix: INT4 model")
    w = synth.make_weights(spec, 0)
    suffix, new, L = 16, 32, 8
    cases = [(500, 10), (1024, 10), (1024, 50)]
    n_max = max(n for _, n in cases)
    P_max = max(p for p, _ in cases)
    cap = P_max + suffix + new
    model = load_model(w, max_lanes=n_max + 1, max_pos=cap, max_L=L,
                       kv_arena_bytes=kv_bytes(spec, [L] * (n_max + 1), [cap] * (n_max + 1)) * 3 // 2)
    out_tok = torch.empty(n_max, dtype=torch.int32, device="cuda")
    res = {"config": "INT4 loop block (2048-wide, vocab 50304), L=8; each request = shared prefix + 16 own tokens, "
                     "then 32 greedy tokens; wall time of all requests, best of 2"}
    for P, n in cases:
        prefix = synth.tokens(0, synth.STREAM_PROMPT_TOKENS, P, spec.vocab)
        sufs = synth.tokens(0, synth.STREAM_PROMPT_TOKENS + 1, n * suffix, spec.vocab).reshape(n, suffix)
        full = torch.tensor(np.concatenate([np.concatenate([prefix, sufs[i]]) for i in range(n)]),
                            dtype=torch.int32, device="cuda")
        pre = torch.tensor(prefix, dtype=torch.int32, device="cuda")
        suf = torch.tensor(sufs.reshape(-1), dtype=torch.int32, device="cuda")
        lanes = np.arange(n, dtype=np.int32)
        Ls = np.full(n, L, np.int32)
        out = out_tok[:n]

        def decode():
            for _ in range(new - 1):
                tl.tl_decode_step(model, lanes, Ls, out, stream=ds)

        def no_cache():
            cu = np.arange(0, n * (P + suffix) + 1, P + suffix, dtype=np.int32)
            tl.tl_forward(model, cu, full, L=L, lanes=lanes, max_new_tokens=new, stream=ds)
            decode()

        def shared():
            tl.tl_forward(model, np.array([0, P], np.int32), pre, L=L, lanes=[n_max], max_new_tokens=0, stream=ds)
            for i in range(n):
                tl.tl_lane_fork(model, n_max, i, P, max_new_tokens=suffix + new, stream=ds)
            tl.tl_append(model, np.arange(0, n * suffix + 1, suffix, dtype=np.int32), suf, lanes, Ls, stream=ds)
            decode()

        row = {}
        for name, fn in (("no_cache_ms", no_cache), ("shared_ms", shared)):
            best = None
            for _ in range(2):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                el = (time.perf_counter() - t0) * 1e3
                best = el if best is None else min(best, el)
            row[name] = round(best, 2)
        row["speedup"] = round(row["no_cache_ms"] / row["shared_ms"], 2)
        res["prefix%d_requests%d" % (P, n)] = row
        log("prefix %d, %d requests: %s" % (P, n, row))
    tl.tl_free(model)
    return res


def spec_bench(tl, torch, np, synth, kv_bytes, load_model):
    """Batch-1 greedy decode on the INT4 model, 32-token prompt, 64 new tokens:
    plain steps at L = 8 against self-speculative decoding (drafts at L = 2, 4
    ahead, verify at L = 8).  Random weights make the acceptance rate meaningless,
    so the pieces of a round are timed as well: one draft step at L = 2, one
    5-token verify pass at L = 8, one plain step at L = 8; with a drafts accepted
    per round a round yields a + 1 tokens, which gives the acceptance at which
    speculation breaks even."""
    ds = torch.cuda.Stream()
    spec = synth.SPECS[2]
    log("speculative: INT4 model, batch 1")
    w = synth.make_weights(spec, 0)
    plen, new, k = 32, 64, 4
    cap = plen + new + k + 8
    model = load_model(w, max_lanes=4, max_pos=cap, max_L=8, kv_arena_bytes=kv_bytes(spec, [8] * 4, [cap] * 4))
    prompt = torch.tensor(synth.tokens(0, synth.STREAM_PROMPT_TOKENS, plen, spec.vocab), dtype=torch.int32,
                          device="cuda")
    cu = np.array([0, plen], np.int32)
    out1 = torch.empty(1, dtype=torch.int32, device="cuda")
    outs = torch.empty(1, new, dtype=torch.int32, device="cuda")

    def timed(fn, reps=3):
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            best = el if best is None else min(best, el)
        return best

    def prefill(lane, L):
        tl.tl_forward(model, cu, prompt, L=L, lanes=[lane], max_new_tokens=cap - plen, stream=ds)
        torch.cuda.synchronize()

    res = {"config": "INT4 model (2048-wide), batch 1, 32-token prompt, 64 greedy tokens; drafts at L=2, "
                     "4 ahead, verify at L=8"}
    acc_log = []

    def plain():
        prefill(0, 8)
        for _ in range(new - 1):
            tl.tl_decode_step(model, [0], [8], out1, stream=ds)

    def specd():
        prefill(1, 8)
        acc_log.append(tl.tl_speculate(model, [1], 2, 8, k, new - 1, outs, stream=ds))

    t_plain = timed(plain)
    t_spec = timed(specd)
    acc = [int(a) for a in acc_log[-1][0] if a >= 0]
    res["plain_tok_per_s"] = round((new - 1) / t_plain, 1)
    res["speculative_tok_per_s"] = round((new - 1) / t_spec, 1)
    res["rounds"] = len(acc)
    res["mean_accepted_per_round"] = round(float(np.mean(acc)), 3)

    # pieces of a round (prefill excluded: each piece is timed over 20 repetitions)
    def rep20(fn):
        fn()   # the first call of a shape captures its graph
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / 20

    prefill(2, 2)
    t_draft = rep20(lambda: tl.tl_decode_step(model, [2], [2], out1, in_tokens=out1, stream=ds))
    prefill(2, 8)
    t_step = rep20(lambda: tl.tl_decode_step(model, [2], [8], out1, in_tokens=out1, stream=ds))
    five = torch.zeros(k + 1, dtype=torch.int32, device="cuda")
    prefill(3, 8)
    t_verify = rep20(lambda: (tl.tl_lane_fork(model, 3, 2, plen, max_new_tokens=k + 1, stream=ds),
                              tl.tl_append(model, [0, k + 1], five, [2], [8], stream=ds)))
    res["draft_step_L2_ms"] = round(t_draft * 1e3, 4)
    res["plain_step_L8_ms"] = round(t_step * 1e3, 4)
    res["verify_5_tokens_L8_ms"] = round(t_verify * 1e3, 4)
    round_ms = k * t_draft + t_verify
    res["break_even_accepted_per_round"] = round(round_ms / t_step - 1, 3)
    res["tok_per_s_if_all_accepted"] = round((k + 1) / round_ms, 1)
    # the plain step as an HBM-bound step: weights read once per loop iteration, the
    # lane's K/V at the mean context of the 64-token run
    res["plain_step_hbm"] = hbm_rate(decode_step_bytes(spec, True, [8], plen + new / 2), t_step)
    res["note"] = ("break-even and all-accepted figures are derived from the timed pieces (a round = 4 draft steps + "
                   "one verify pass, yielding accepted + 1 tokens); the verify piece includes a fork of the "
                   "32-token prompt")
    tl.tl_free(model)
    return res


def mall_bench(tl, torch, np, synth, load_model):
    """The pages' L2-residency control ("Benchmark Comparison" page, measured
    benchmarks, section 6: one loop iteration with its weights warm in cache vs
    flushed) moved to the 256 MB Infinity Cache: one-iteration forwards (1 x 128
    tokens, L = 1) of the INT4 model, repeated (the loop block's 26.5 MB stay
    resident) or each after streaming 512 MB through the memory system; kernel-
    class event timing of the loop block's products."""
    spec = synth.SPECS[2]
    log("MALL control: INT4 model, L=1 forwards, warm vs flushed")
    w = synth.make_weights(spec, 0)
    model = load_model(w, max_pos=256)
    toks = torch.tensor(synth.tokens(0, synth.STREAM_TOKENS, 128, spec.vocab), dtype=torch.int32, device="cuda")
    cu = np.array([0, 128], np.int32)
    hid = torch.empty(128, spec.d_model, dtype=torch.float32, device="cuda")
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    loop_cls = ("gemm_qkv_loop", "gemm_o_loop", "gemm_gu_loop", "gemm_down_loop")
    res = {"config": "INT4 model (2048-wide), 1 x 128 tokens, L=1 (one loop iteration per call); flushed = "
                     "256 MiB copied (512 MiB streamed) before each call; per-launch microseconds of the loop "
                     "block's four products (kernel start and end stamped by the runtime; the event pairs around "
                     "the launches in loop_block_event_pair_us) and of the whole call",
           "loop_block_bytes": block_weight_bytes(spec, True)}
    reps = 30
    for name, flush in (("warm", False), ("flushed", True)):
        for _ in range(3):
            tl.tl_forward(model, cu, toks, L=1, out_hidden=hid, stream=0)
        torch.cuda.synchronize()
        tl.tl_timing_enable(model, True)
        call_ms = []
        for _ in range(reps):
            if flush:
                dst.copy_(src)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            tl.tl_forward(model, cu, toks, L=1, out_hidden=hid, stream=0)
            torch.cuda.synchronize()
            call_ms.append((time.perf_counter() - t0) * 1e3)
        cls = tl.tl_timing_read(model)
        kcls = tl.tl_timing_read_kernels(model)
        tl.tl_timing_enable(model, False)
        row = {k: round(kcls[k][0] / cls[k][1] * 1e3, 2) for k in loop_cls if cls[k][1]}
        row["loop_block_us"] = round(sum(kcls[k][0] for k in loop_cls) / reps * 1e3, 2)
        row["loop_block_event_pair_us"] = round(sum(cls[k][0] for k in loop_cls) / reps * 1e3, 2)
        row["call_ms_median"] = round(float(np.median(call_ms)), 4)
        res[name] = row
        log("MALL %s: %s" % (name, row))
    res["flushed_over_warm_loop_block"] = round(res["flushed"]["loop_block_us"] / res["warm"]["loop_block_us"], 3)
    tl.tl_free(model)
    return res


def cfg5_bench(tl, torch, np, synth, kv_bytes, load_model):
    """Continuous-depth decode on the 5280-wide bf16 model (2 pre blocks, a 4-layer
    loop stack, 2 post blocks): 256 sequences, prompts uniform in [32, 512], 64 new
    tokens each (the first from the prefill, 63 cached), per-token depth
    min(32, 1 + Poisson(7)) clamped to never rise.  fp32 activations and K/V on
    split-fp16 matrix cores, batch-invariant kernels.  Times the prefill, the
    continuous-depth decode (tl_decode_run, boundary queue of 64 lanes) and the
    same decode in lockstep (one tl_decode_step per token, iteration-level
    compaction); both give the same tokens bit for bit."""
    spec = synth.SPECS[5]
    log("cfg 5: 5280-wide model, 256 sequences")
    n, new = 256, 64
    w = synth.make_weights(spec, 0)
    plens = synth.prompt_lengths(0, n)
    prompts = [synth.tokens(0, 3000 + i, int(p), spec.vocab) for i, p in enumerate(plens)]
    draws = synth.token_loop_draws(0, n, new)
    L1 = draws[:, 0].copy()
    model = load_model(w, max_lanes=n, max_pos=512 + new, max_L=32,
                       kv_arena_bytes=kv_bytes(spec, L1, plens + new - 1), batch_invariant=1)
    del w
    toks = torch.tensor(np.concatenate(prompts), dtype=torch.int32, device="cuda")
    cu = np.concatenate([[0], np.cumsum(plens)]).astype(np.int32)
    lanes = np.arange(n, dtype=np.int32)
    T = int(cu[-1])
    ds = torch.cuda.Stream()

    def prefill():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tl.tl_forward(model, cu, toks, seq_L=L1, lanes=lanes, max_new_tokens=new - 1, stream=ds)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    t_pre = prefill()
    out_run = torch.empty(n, new - 1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    eff = tl.tl_decode_run(model, lanes, draws[:, 1:], out_run, boundary_min=64, stream=ds)
    torch.cuda.synchronize()
    t_cdb = time.perf_counter() - t0
    prefill()
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    step_tok = torch.empty(n, new - 1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(new - 1):
        tl.tl_decode_step(model, lanes, draws[:, 1 + t], out, stream=ds)
        with torch.cuda.stream(ds):   # ordered after the step that wrote out
            step_tok[:, t].copy_(out)
    torch.cuda.synchronize()
    t_lock = time.perf_counter() - t0
    same = bool(torch.equal(step_tok, out_run))
    tl.tl_free(model)
    iters = int(eff.sum())
    pre_iters = int(np.sum(plens * L1))
    return {"config": "5280-wide bf16 model (2 pre + 4-layer loop stack + 2 post, 55x96 heads, SwiGLU 17920, "
                      "vocab 65536), 256 sequences, prompts uniform in [32, 512] (%d rows), 64 new tokens, per-token "
                      "L = min(32, 1 + Poisson(7)) clamped monotone; fp32 activations, split-fp16 MFMA, "
                      "batch-invariant" % T,
            "prefill_s": round(t_pre, 3), "prefill_token_iterations_per_s": round(pre_iters / t_pre, 1),
            "decode_token_iterations": iters,
            "continuous_depth": {"s": round(t_cdb, 3), "tok_per_s": round(n * (new - 1) / t_cdb, 1),
                                 "token_iterations_per_s": round(iters / t_cdb, 1)},
            "lockstep": {"s": round(t_lock, 3), "tok_per_s": round(n * (new - 1) / t_lock, 1),
                         "token_iterations_per_s": round(iters / t_lock, 1)},
            "lockstep_over_continuous": round(t_lock / t_cdb, 3),
            "same_tokens": same}


def store_h_bench(tl, torch, np, synth, kv_bytes, load_model):
    """Cache modes at batch 1 on the FP16-body model: 512-token prompt, 64 tokens at
    L = 8 (the first from the prompt pass, 63 cached steps fed the same seeded
    tokens in every mode); decode time, the cache bytes one position takes in one
    slot, and how far the last step's hidden state lies from the K/V mode's."""
    spec = synth.SPECS[3]
    log("store-h: FP16-body model, batch 1")
    ds = torch.cuda.Stream()
    w = synth.make_weights(spec, 0)
    plen, new, L = 512, 64, 8
    d, H = spec.d_model, spec.n_heads
    prompt = torch.tensor(synth.tokens(0, synth.STREAM_PROMPT_TOKENS, plen, spec.vocab), dtype=torch.int32,
                          device="cuda")
    feed = torch.tensor(synth.tokens(0, synth.STREAM_PROMPT_TOKENS + 2, new, spec.vocab), dtype=torch.int32,
                        device="cuda")
    cu = np.array([0, plen], np.int32)
    out1 = torch.empty(1, dtype=torch.int32, device="cuda")
    hid = torch.empty(1, d, dtype=torch.float32, device="cuda")
    res = {"config": "FP16-body model (2048-wide), batch 1, 512-token prompt, 63 cached steps at L=8 on the same "
                     "seeded tokens; hidden_rel_vs_kv: relative L2 distance of the last step's hidden state from "
                     "the K/V mode's"}
    # bytes of one position in one loop slot (delta: a slot past the first iteration; the
    # first iteration's anchor slot takes d * 2)
    per_pos = {"kv": 2 * d * 2, "h": d * 2, "h8": d + 2 * H, "h4": d // 2 + 2 * H, "d8": d + 2 * H}
    ref = None
    for name, mode in (("kv", tl.TL_KV_KV), ("h", tl.TL_KV_H), ("h8", tl.TL_KV_H8), ("h4", tl.TL_KV_H4),
                       ("d8", tl.TL_KV_D8)):
        model = load_model(w, max_lanes=1, max_pos=plen + new, max_L=L,
                           kv_arena_bytes=kv_bytes(spec, [L], [plen + new]), kv_mode=mode)
        best = None
        for _ in range(2):
            tl.tl_forward(model, cu, prompt, L=L, lanes=[0], max_new_tokens=new, stream=ds)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for t in range(new - 1):
                tl.tl_decode_step(model, [0], [L], out1, in_tokens=feed[t:t + 1], out_hidden=hid, stream=ds)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            best = el if best is None else min(best, el)
        tl.tl_free(model)
        last = hid.cpu().numpy()[0].astype(np.float64)
        if ref is None:
            ref = last
        res[name] = {"decode_ms": round(best * 1e3, 2), "tok_per_s": round((new - 1) / best, 1),
                     "bytes_per_position_per_slot": per_pos[name],
                     "hidden_rel_vs_kv": float("%.3g" % (np.linalg.norm(last - ref) / np.linalg.norm(ref)))}
        log("store-h %s: %s" % (name, res[name]))
    return res


if __name__ == "__main__":
    main()
