"""Continuous-depth decode on the 5280-wide bf16 model (2 pre blocks, a 4-layer
shared loop stack, 2 post blocks, 55 heads x 96, SwiGLU 17920, vocab 65536).

256 sequences with prompt lengths uniform in [32, 512] are prefilled as lanes at
their first token's depth; 63 more tokens per lane follow through tl_decode_run,
each with depth min(32, 1 + Poisson(7)) clamped to never rise.  The GPU runs the
whole workload; the oracle checks the six shortest lanes through its uncached
ragged-depth forward (equal to cached decode at clamped depths, pinned in
tests/test_oracle_pins.py).  Decode is teacher-forced with seeded tokens.  The
weights are bf16; GEMM operands, activations and the KV cache are fp16 (bf16
activations alone put an exact-arithmetic emulation 2-5e-2 away from the oracle
at this depth, above the 1e-2 / 3e-2 bars).  The same lanes then decode again in
lockstep (one tl_decode_step per token), which must give the same results.
"""
import sys
import time

import numpy as np
import pytest

import oracle
import synth
from tests.harness import ensure_built, kv_bytes, load_model, rel_l2

torch = pytest.importorskip("torch")
import looped_transformer_amd as tl  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-cfg5]", *a, flush=True)
    sys.stdout.flush()


def bar(L):
    return 1e-2 if L <= 8 else 3e-2


def test_cfg5_continuous_depth_decode():
    ensure_built()
    spec = synth.SPECS[5]
    n, new = 256, 64
    t0 = time.time()
    w = synth.make_weights(spec, seed=0)
    say("weights generated in %.1f s" % (time.time() - t0))
    plens = synth.prompt_lengths(0, n)
    prompts = [synth.tokens(0, 3000 + i, int(p), spec.vocab) for i, p in enumerate(plens)]
    draws = synth.token_loop_draws(0, n, new)                     # [n, 64] requests
    L1 = draws[:, 0].copy()                                       # first token: ceiling 32
    forced = synth.tokens(0, 1200, n * (new - 1), spec.vocab).reshape(n, new - 1)
    caps = plens + new - 1
    model = load_model(w, max_lanes=n, max_pos=512 + new, max_L=32, kv_arena_bytes=kv_bytes(spec, L1, caps))
    say("loaded; memory (weights, kv, workspace) =", tl.tl_memory_info(model))
    sample = [int(i) for i in np.argsort(plens, kind="stable")[:6]]
    try:
        toks = torch.tensor(np.concatenate(prompts), dtype=torch.int32, device="cuda")
        cu = np.concatenate([[0], np.cumsum(plens)]).astype(np.int32)
        T = int(cu[-1])
        lanes = np.arange(n, dtype=np.int32)
        hid = torch.empty(T, spec.d_model, dtype=torch.float32, device="cuda")
        nxt = torch.empty(n, dtype=torch.int32, device="cuda")
        t0 = time.time()
        tl.tl_forward(model, cu, toks, seq_L=L1, lanes=lanes, max_new_tokens=new - 1, out_hidden=hid, out_next=nxt)
        torch.cuda.synchronize()
        say("prefill of %d rows in %.2f s" % (T, time.time() - t0))
        run_tok = torch.empty(n, new - 1, dtype=torch.int32, device="cuda")
        run_h = torch.empty(n, new - 1, spec.d_model, dtype=torch.float32, device="cuda")
        feed = torch.tensor(forced, dtype=torch.int32, device="cuda")
        t0 = time.time()
        eff = tl.tl_decode_run(model, lanes, draws[:, 1:], run_tok, in_tokens=feed, out_hidden=run_h, boundary_min=64)
        torch.cuda.synchronize()
        tl.tl_sync_errors(model)
        say("continuous-depth decode of %d x %d tokens in %.2f s" % (n, new - 1, time.time() - t0))
        t_cdb = time.time() - t0
        H_pre = [hid[cu[i]:cu[i + 1]].cpu().numpy() for i in sample]
        H_run = run_h.cpu().numpy()
        T_run = run_tok.cpu().numpy()
        H_dec = H_run[sample]
        T_dec = T_run[sample]
        T_pre = nxt.cpu().numpy()[sample]
        # lockstep: the same lanes prefilled again, then one tl_decode_step per token
        tl.tl_forward(model, cu, toks, seq_L=L1, lanes=lanes, max_new_tokens=new - 1)
        torch.cuda.synchronize()
        out = torch.empty(n, dtype=torch.int32, device="cuda")
        hs = torch.empty(n, spec.d_model, dtype=torch.float32, device="cuda")
        step_h = np.empty_like(H_run)
        step_t = np.empty_like(T_run)
        t0 = time.time()
        dt_run = 0.0
        for t in range(new - 1):
            e2 = tl.tl_decode_step(model, lanes, draws[:, 1 + t], out, in_tokens=feed[:, t].contiguous(), out_hidden=hs)
            assert np.array_equal(e2, eff[:, t])
            torch.cuda.synchronize()
            t1 = time.time()
            step_h[:, t] = hs.cpu().numpy()
            step_t[:, t] = out.cpu().numpy()
            dt_run += time.time() - t1
        t_lock = time.time() - t0 - dt_run
        say("lockstep decode %.2f s vs continuous-depth %.2f s" % (t_lock, t_cdb))
        same = T_run == step_t
        say("continuous-depth vs lockstep: tokens equal %.4f, hidden rel %.2e" % (same.mean(), rel_l2(H_run, step_h)))
        # the two schedules batch rows differently, so split-K partitions (and with
        # them fp32 summation order) differ; fp16 roundings then part at the same
        # ~1e-3 level as the intrinsic error against the oracle
        assert same.mean() >= 0.99
        assert rel_l2(H_run, step_h) <= 3e-3
    finally:
        tl.tl_free(model)
    # the depth schedule: clamped, never rising, equal to the oracle's rule
    for i in range(n):
        assert np.array_equal(eff[i], oracle.clamp_depths(draws[i, 1:], int(L1[i])))
    t0 = time.time()
    m = oracle.OracleModel.from_weights(w)
    say("oracle model in %.1f s" % (time.time() - t0))
    agree, total, gaps = 0, 0, []
    for k, i in enumerate(sample):
        deps = np.concatenate([np.full(plens[i], L1[i]), eff[i]])
        seq = np.concatenate([prompts[i], forced[i]])
        t0 = time.time()
        h_ref, lg_ref = oracle.forward_ragged(m, seq, deps, want_logits="all")
        P = int(plens[i])
        r_pre = rel_l2(H_pre[k], h_ref[:P])
        r_dec = rel_l2(H_dec[k], h_ref[P:])
        say("lane", i, "prompt", P, "L1", L1[i], "prefill rel %.2e decode rel %.2e (oracle %.1f s)"
            % (r_pre, r_dec, time.time() - t0))
        assert r_pre <= bar(int(L1[i]))
        assert r_dec <= bar(int(L1[i]))
        lg = lg_ref[P - 1:]
        top = oracle.greedy_argmax(lg)
        got = np.concatenate([[T_pre[k]], T_dec[k]])
        agree += int(np.sum(top == got))
        total += len(got)
        for t in np.nonzero(top != got)[0]:
            row = lg[t]
            gaps.append(float((row[top[t]] - row[got[t]]) / np.sqrt(np.mean(row * row))))
    say("top-1 agreement", agree, "/", total, "gaps of the differing tokens (x rms):", ["%.3f" % g for g in gaps])
    # With fp16 operands and KV the hidden error after 36-52 block applications is
    # ~5e-3, and an oracle that only rounds its GEMM inputs, q/k/v, attention output,
    # SwiGLU output and P to fp16 is itself 4.7e-3 away from the exact logits (about
    # 7e-3 of a row's rms between two entries).  So a greedy token may differ only
    # where the oracle's own top choices nearly tie: each differing token must lie
    # within 5 % of the rms (~7 sigma) of the oracle's best, and such near-ties stay
    # a small share of the tokens (the count depends on the model, not the path).
    assert all(g <= 0.05 for g in gaps)
    assert agree >= 0.97 * total
