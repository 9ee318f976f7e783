"""Long contexts on the 2048-wide INT4 model against the oracle.

Cached decode after prompts of 520 and 300 tokens (next to a 41-token one), in the
K/V cache mode and in the INT8 store-h mode ("CLI Reference" page, environment
variables TINYLOOP_KV_H_MODE with TINYLOOP_KV_INT8), and the reuse of a prefix of
more than 500 tokens ("Benchmark Comparison" page, measured benchmarks, section 2:
500- and 1024-token shared prefixes): fork, append, decode.

At these lengths the decode attention splits a context over its four waves in
blocks of 64 positions, so each wave runs several blocks and rescales its running
softmax between them, and the prefill attention runs several 32-row tiles per
sequence against several 64-key blocks.  Tokens are seeded (teacher forcing);
hidden states meet the usual bars pooled and per row; logits the same bar; a
greedy token may differ from the oracle's only at a near-tie of the oracle's own
logits.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from tests.harness import ensure_built, kv_bytes, load_model, near_tie_gaps, rel_l2, row_rel_max

torch = pytest.importorskip("torch")
import looped_transformer_amd as tl  # noqa: E402

pytestmark = pytest.mark.gpu

SPEC = synth.SPECS[2]
PLENS = [520, 300, 41]
LS = [3, 2, 3]
NEW = 8


def say(*a):
    print("[gpu-long]", *a, flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), dtype=torch.int32, device="cuda")


@pytest.fixture(scope="module")
def weights():
    ensure_built()
    w = synth.make_weights(SPEC, seed=0)
    return w, oracle.OracleModel.from_weights(w)


def _check_tokens(got, ref_logits, what):
    gaps = near_tie_gaps(got, ref_logits)
    say(what, "differing greedy tokens (gap x rms):", ["%.3f" % g for g in gaps])
    assert all(g <= 0.05 for g in gaps), (what, gaps)


@pytest.mark.parametrize("mode", ["kv", "h8"])
def test_long_prompt_then_decode(weights, mode):
    w, base = weights
    m = base
    if mode != "kv":
        import copy
        m = copy.copy(base)
        m.kv_mode = mode
    bar = 1e-2                                  # depths <= 8; the INT8 store-h bar for fp16 is 1e-2 too
    row_bar = bar if mode == "kv" else 2 * bar  # a row can take several moved int8 codes
    prompts = [synth.tokens(7, 7100 + i, n, SPEC.vocab) for i, n in enumerate(PLENS)]
    feed = synth.tokens(7, 7200, 4 * len(PLENS), SPEC.vocab).reshape(4, len(PLENS))
    lanes = [2, 0, 1]
    kvm = {"kv": tl.TL_KV_KV, "h8": tl.TL_KV_H8}[mode]
    model = load_model(w, max_lanes=4, max_pos=640, max_L=8,
                       kv_arena_bytes=kv_bytes(SPEC, LS, [n + NEW for n in PLENS]), kv_mode=kvm)
    try:
        cu = np.concatenate([[0], np.cumsum(PLENS)]).astype(np.int32)
        hid = torch.empty(int(cu[-1]), SPEC.d_model, dtype=torch.float32, device="cuda")
        lg = torch.empty(len(PLENS), SPEC.vocab, dtype=torch.float32, device="cuda")
        nxt = torch.empty(len(PLENS), dtype=torch.int32, device="cuda")
        say(mode, "prefill", PLENS)
        tl.tl_forward(model, cu, _dev(np.concatenate(prompts)), seq_L=LS, lanes=lanes, max_new_tokens=NEW,
                      out_hidden=hid, out_logits=lg, out_next=nxt)
        torch.cuda.synchronize()
        tl.tl_sync_errors(model)
        H, LG, NX = hid.cpu().numpy(), lg.cpu().numpy(), nxt.cpu().numpy()
        o_lanes = []
        for i, (p, L) in enumerate(zip(prompts, LS)):
            ln, h_ref, l_ref = oracle.prefill(m, p, L)
            o_lanes.append(ln)
            hi = H[cu[i]:cu[i + 1]]
            r, rm, rl = rel_l2(hi, h_ref), row_rel_max(hi, h_ref), rel_l2(LG[i], l_ref)
            say(mode, "prefill lane", lanes[i], "T", PLENS[i], "L", L,
                "hidden %.2e row max %.2e logits %.2e" % (r, rm, rl))
            assert r <= bar and rm <= row_bar and rl <= bar, (i, r, rm, rl)
            _check_tokens([NX[i]], l_ref[None, :], "prefill lane %d" % lanes[i])
        out = torch.empty(len(PLENS), dtype=torch.int32, device="cuda")
        hs = torch.empty(len(PLENS), SPEC.d_model, dtype=torch.float32, device="cuda")
        for t in range(4):
            eff = tl.tl_decode_step(model, lanes, [3, 3, 3], out, in_tokens=_dev(feed[t]), out_logits=lg,
                                    out_hidden=hs)
            torch.cuda.synchronize()
            Hd, LGd, T = hs.cpu().numpy(), lg.cpu().numpy(), out.cpu().numpy()
            refs = [oracle.decode_step(m, ol, 3, token=int(feed[t, i])) for i, ol in enumerate(o_lanes)]
            for i, (h_o, l_o, _, L_o) in enumerate(refs):
                assert eff[i] == L_o
                r, rl = rel_l2(Hd[i], h_o), rel_l2(LGd[i], l_o)
                say(mode, "step", t, "lane", lanes[i], "ctx", PLENS[i] + t + 1, "hidden %.2e logits %.2e" % (r, rl))
                assert r <= row_bar and rl <= bar, (t, i, r, rl)
            _check_tokens(T, np.stack([x[1] for x in refs]), "step %d" % t)
    finally:
        tl.tl_free(model)


def test_long_prefix_fork_append_decode(weights):
    w, m = weights
    P0, L0 = 530, 3
    prefix = synth.tokens(8, 7300, P0, SPEC.vocab)
    suffix = synth.tokens(8, 7301, 12, SPEC.vocab)
    feed = synth.tokens(8, 7302, 9, SPEC.vocab).reshape(3, 3)
    # oracle: source lane, a fork of 512 positions that appends 12 tokens, a fork of
    # the whole lane that decodes from the source's pending token
    o_src, _, _ = oracle.prefill(m, prefix, L0, want_logits="last")
    o_part = oracle.fork(o_src, 512)
    o_whole = oracle.fork(o_src, P0)
    h_app, l_app = oracle.append(m, o_part, suffix, L0)
    model = load_model(w, max_lanes=4, max_pos=640, max_L=8, kv_arena_bytes=kv_bytes(SPEC, [L0] * 3, [P0 + 16] * 3))
    try:
        say("prefix", P0, "fork 512 + append 12, whole fork")
        tl.tl_forward(model, np.array([0, P0], np.int32), _dev(prefix), L=L0, lanes=[0], max_new_tokens=16)
        tl.tl_lane_fork(model, 0, 1, 512, max_new_tokens=16)
        tl.tl_lane_fork(model, 0, 2, P0, max_new_tokens=16)
        hid = torch.empty(12, SPEC.d_model, dtype=torch.float32, device="cuda")
        lg = torch.empty(3, SPEC.vocab, dtype=torch.float32, device="cuda")
        nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        eff = tl.tl_append(model, np.array([0, 12], np.int32), _dev(suffix), [1], [L0], out_hidden=hid,
                           out_logits=lg[:1], out_next=nxt)
        torch.cuda.synchronize()
        assert eff[0] == L0
        H = hid.cpu().numpy()
        r, rm, rl = rel_l2(H, h_app), row_rel_max(H, h_app), rel_l2(lg.cpu().numpy()[0], l_app)
        say("append at 512: hidden %.2e row max %.2e logits %.2e" % (r, rm, rl))
        assert r <= 1e-2 and rm <= 1e-2 and rl <= 1e-2
        _check_tokens(nxt.cpu().numpy(), l_app[None, :], "append")
        lanes = [1, 2, 0]
        o_l = [o_part, o_whole, o_src]
        out = torch.empty(3, dtype=torch.int32, device="cuda")
        hs = torch.empty(3, SPEC.d_model, dtype=torch.float32, device="cuda")
        for t in range(3):
            e = tl.tl_decode_step(model, lanes, [L0] * 3, out, in_tokens=_dev(feed[t]), out_logits=lg, out_hidden=hs)
            torch.cuda.synchronize()
            Hd, LGd = hs.cpu().numpy(), lg.cpu().numpy()
            refs = [oracle.decode_step(m, ol, L0, token=int(feed[t, i])) for i, ol in enumerate(o_l)]
            for i, (h_o, l_o, _, L_o) in enumerate(refs):
                assert e[i] == L_o
                r, rl = rel_l2(Hd[i], h_o), rel_l2(LGd[i], l_o)
                say("decode step", t, "lane", lanes[i], "hidden %.2e logits %.2e" % (r, rl))
                assert r <= 1e-2 and rl <= 1e-2, (t, i, r, rl)
            _check_tokens(out.cpu().numpy(), np.stack([x[1] for x in refs]), "decode step %d" % t)
    finally:
        tl.tl_free(model)


def test_long_prompt_batch1_decode(weights):
    """One lane after a 520-token prompt: with only 16 (row, head) workgroups the
    decode attention splits each row's positions over nine of them per head
    (quarter-size blocks), and a merge kernel combines the runs."""
    w, m = weights
    P, L = PLENS[0], LS[0]
    prompt = synth.tokens(7, 7400, P, SPEC.vocab)
    feed = synth.tokens(7, 7500, 4, SPEC.vocab)
    model = load_model(w, max_lanes=1, max_pos=640, max_L=8, kv_arena_bytes=kv_bytes(SPEC, [L], [P + NEW]))
    try:
        tl.tl_forward(model, np.array([0, P], dtype=np.int32), _dev(prompt), seq_L=[L], lanes=[0],
                      max_new_tokens=NEW)
        torch.cuda.synchronize()
        ln, _, _ = oracle.prefill(m, prompt, L)
        out = torch.empty(1, dtype=torch.int32, device="cuda")
        hs = torch.empty(1, SPEC.d_model, dtype=torch.float32, device="cuda")
        lg = torch.empty(1, SPEC.vocab, dtype=torch.float32, device="cuda")
        for t in range(4):
            tl.tl_decode_step(model, [0], [L], out, in_tokens=_dev(feed[t:t + 1]), out_logits=lg, out_hidden=hs)
            torch.cuda.synchronize()
            h_o, l_o, _, _ = oracle.decode_step(m, ln, L, token=int(feed[t]))
            r, rl = rel_l2(hs.cpu().numpy()[0], h_o), rel_l2(lg.cpu().numpy()[0], l_o)
            say("batch-1 step", t, "ctx", P + t + 1, "hidden %.2e logits %.2e" % (r, rl))
            assert r <= 1e-2 and rl <= 1e-2, (t, r, rl)
            _check_tokens(out.cpu().numpy(), l_o[None, :], "batch-1 step %d" % t)
    finally:
        tl.tl_free(model)
