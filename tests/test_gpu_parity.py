"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: INT4 codes and scales and every per-iteration active-row list bit-exact;
relative L2 of final hidden states <= 1e-2 for L <= 8 and <= 3e-2 above
(fp32 models: 1e-4); top-1 agreement >= 99 % on greedy tokens.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synth
from tests.harness import ensure_built, kv_bytes, load_model, near_tie_gaps, rel_l2, row_rel_max

torch = pytest.importorskip("torch")
import looped_transformer_amd as tl  # noqa: E402

pytestmark = pytest.mark.gpu

TINY = {
    "tiny-f32": synth.SPECS[1],
    "tiny-f16": synth.ModelSpec("tiny-f16", 256, 128, 4, 32, 256, 1, 1, 0, "f16", "f16"),
    "tiny-w4": synth.ModelSpec("tiny-w4", 256, 128, 4, 32, 256, 1, 1, 0, "f16", "w4g128"),
    "tiny-f16body": synth.ModelSpec("tiny-f16body", 256, 128, 4, 32, 256, 1, 1, 0, "f16", "f16body"),
    "tiny-bf16-stack": synth.ModelSpec("tiny-bf16-stack", 320, 192, 2, 96, 384, 2, 2, 1, "bf16", "bf16"),
    # INT4, 16 K groups in the down projection: at decode sizes its K is split 16
    # ways, more than the fused residual + norm reduction loads at once
    "tiny-w4-wide": synth.ModelSpec("tiny-w4-wide", 256, 256, 4, 64, 2048, 1, 1, 0, "f16", "w4g128"),
    # INT4 with SwiGLU 4096: at 65..128 rows gate/up (N = 8192) and down (K = 4096)
    # take the row-tiled INT4 kernel (down with K split 4 ways)
    "mid-w4-ffn4096": synth.ModelSpec("mid-w4-ffn4096", 256, 256, 4, 64, 4096, 1, 1, 0, "f16", "w4g128"),
    # bf16 weights with fp32 activations and K/V: products on fp16 MFMA with the
    # fp32 operands split into two fp16 halves
    "tiny-wide": synth.ModelSpec("tiny-wide", 320, 192, 2, 96, 384, 2, 2, 1, "bf16", "bf16", act="f32"),
}


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


def hidden_bar(spec, L):
    if spec.act_dtype == "f32":
        return 1e-4
    return 1e-2 if L <= 8 else 3e-2


def gpu_forward(model, spec, seqs, Ls, lanes=None, max_new=0, logits=True):
    toks = torch.tensor(np.concatenate(seqs), dtype=torch.int32, device="cuda")
    cu = np.cumsum([0] + [len(s) for s in seqs]).astype(np.int32)
    T = int(cu[-1])
    depth = np.concatenate([np.full(len(s), L) for s, L in zip(seqs, Ls)])
    n_log = int(sum(np.sum(depth >= j) for j in range(1, int(depth.max()) + 1)))
    hid = torch.empty(T, spec.d_model, dtype=torch.float32, device="cuda")
    lg = torch.empty(len(seqs), spec.vocab, dtype=torch.float32, device="cuda") if logits else None
    nxt = torch.empty(len(seqs), dtype=torch.int32, device="cuda")
    log = torch.empty(max(n_log, 1), dtype=torch.int32, device="cuda")
    tl.tl_forward(model, cu, toks, seq_L=Ls, lanes=lanes, max_new_tokens=max_new, out_hidden=hid,
                  out_logits=lg, out_next=nxt, out_active_log=log)
    torch.cuda.synchronize()
    tl.tl_sync_errors(model)
    return (hid.cpu().numpy(), lg.cpu().numpy() if logits else None, nxt.cpu().numpy(),
            log.cpu().numpy()[:n_log], depth)


def check_log(log, depth):
    want = np.concatenate(oracle.active_lists(depth))
    assert np.array_equal(log, want), "active-row lists differ"


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


@pytest.mark.parametrize("name", list(TINY))
def test_tiny_forward_parity(name):
    spec = TINY[name]
    say("tiny forward", name)
    w = synth.make_weights(spec, seed=3)
    m = oracle.OracleModel.from_weights(w)
    seqs = [synth.tokens(3, 3000 + i, n, spec.vocab) for i, n in enumerate([16, 5, 33, 70])]
    Ls = [4, 1, 3, 9]
    model = load_model(w, max_pos=256, max_L=16)
    try:
        hid, lg, nxt, log, depth = gpu_forward(model, spec, seqs, Ls)
    finally:
        tl.tl_free(model)
    check_log(log, depth)
    ref_h, ref_lg, _ = oracle.forward_batch(m, seqs, Ls)
    off = 0
    for i, s in enumerate(seqs):
        r = rel_l2(hid[off:off + len(s)], ref_h[off:off + len(s)])
        rm = row_rel_max(hid[off:off + len(s)], ref_h[off:off + len(s)])
        say(name, "seq", i, "L", Ls[i], "rel %.2e row max %.2e" % (r, rm))
        assert r <= hidden_bar(spec, Ls[i]), (i, r)
        assert rm <= hidden_bar(spec, Ls[i]), (i, rm)
        off += len(s)
    assert rel_l2(lg, ref_lg) <= (1e-4 if spec.act_dtype == "f32" else 1e-2)
    if spec.act_dtype == "f32":
        assert np.array_equal(nxt, oracle.greedy_argmax(ref_lg))
    else:
        # 16-bit operands: a token may differ only where the oracle's own best two
        # logits nearly tie (within 5 % of the row's rms logit)
        gaps = near_tie_gaps(nxt, ref_lg)
        say(name, "differing greedy tokens, gaps x rms:", gaps)
        assert all(g <= 0.05 for g in gaps), gaps


@pytest.mark.parametrize("name", ["tiny-f32", "tiny-f16", "tiny-bf16-stack"])
def test_greedy_ties_take_lowest_index(name):
    """Head rows 37, 40 and 200 are one vector v, every other row is zero, so the
    logits of those three tokens are equal bit for bit and the rest are exactly 0.
    v points along the prefill's last normalised hidden state, so the three tie at
    the maximum there and the greedy token must be 37 (the tie spans head tiles).
    The decode step's logits tie either at 37 (positive) or among the zero rows
    (lowest index 0)."""
    spec = TINY[name]
    w = synth.make_weights(spec, seed=11)
    m = oracle.OracleModel.from_weights(w)
    toks = synth.tokens(11, 7000, 10, spec.vocab)
    _, ref_h, _ = oracle.prefill(m, toks, 2, want_logits="none")
    x = oracle.rmsnorm(ref_h[-1:], m.final_norm, spec.rms_eps)[0]
    v = (0.05 * x / np.linalg.norm(x)).astype(np.float32)
    head = np.zeros((spec.vocab, spec.d_model), np.float32)
    for r in (37, 40, 200):
        head[r] = v
    if spec.boundary_dtype == "f16":
        head = head.astype(np.float16)
    elif spec.boundary_dtype == "bf16":
        head = synth.f32_to_bf16_bits(head)
    w.head = head
    model = load_model(w, max_lanes=1, max_pos=64, max_L=4, kv_arena_bytes=kv_bytes(spec, [2], [16]))
    try:
        dt = torch.tensor(toks, dtype=torch.int32, device="cuda")
        lg = torch.empty(1, spec.vocab, dtype=torch.float32, device="cuda")
        nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        tl.tl_forward(model, np.array([0, 10], np.int32), dt, L=2, lanes=[0], max_new_tokens=4, out_logits=lg,
                      out_next=nxt)
        torch.cuda.synchronize()
        row = lg.cpu().numpy()[0]
        say(name, "tied logit %.4e, next %d" % (row[37], int(nxt.cpu()[0])))
        assert row[37] == row[40] == row[200] and row[37] > 0
        assert np.count_nonzero(row) == 3
        assert int(nxt.cpu()[0]) == 37
        out = torch.empty(1, dtype=torch.int32, device="cuda")
        tl.tl_decode_step(model, [0], [2], out, in_tokens=torch.tensor([5], dtype=torch.int32, device="cuda"),
                          out_logits=lg)
        torch.cuda.synchronize()
        row = lg.cpu().numpy()[0]
        assert row[37] == row[40] == row[200]
        want = 37 if row[37] > 0 else 0
        say(name, "decode tied logit %.4e, next %d" % (row[37], int(out.cpu()[0])))
        assert int(out.cpu()[0]) == want
    finally:
        tl.tl_free(model)


def test_w4_export_bit_exact():
    spec = synth.SPECS[2]
    say("w4 export cfg2")
    w = synth.make_weights(spec, seed=0)
    model = load_model(w, max_pos=256)
    try:
        d, F = spec.d_model, spec.ffn
        shapes = [(3 * d, d, "wqkv"), (d, d, "wo"), (F, d, "wgate"), (F, d, "wup"), (d, F, "wdown")]
        for mi, (N, K, name) in enumerate(shapes):
            q, s = tl.tl_export_w4(model, 1, mi, N, K)
            qo, so = oracle.quantize_w4g128(w.blocks[1][name])
            assert np.array_equal(q, qo), name
            assert np.array_equal(s, so.view(np.uint16)), name
    finally:
        tl.tl_free(model)


def test_cfg1_forward_and_greedy_decode():
    """Tiny fp32 model: 16 tokens at L = 4, then 8 greedy cached decode steps."""
    spec = synth.SPECS[1]
    w = synth.make_weights(spec, seed=0)
    m = oracle.OracleModel.from_weights(w)
    toks = synth.tokens(0, synth.STREAM_TOKENS, 16, spec.vocab)
    model = load_model(w, max_lanes=1, max_pos=64, kv_arena_bytes=kv_bytes(spec, [4], [24]))
    try:
        hid, lg, nxt, log, depth = gpu_forward(model, spec, [toks], [4], lanes=[0], max_new=8)
        lane, ref_h, ref_lg = oracle.prefill(m, toks, 4)
        assert rel_l2(hid, ref_h) <= 1e-5
        assert nxt[0] == lane.pending
        out = torch.empty(1, dtype=torch.int32, device="cuda")
        hs = torch.empty(1, spec.d_model, dtype=torch.float32, device="cuda")
        lgt = torch.empty(1, spec.vocab, dtype=torch.float32, device="cuda")
        for step in range(8):
            eff = tl.tl_decode_step(model, [0], [4], out, out_logits=lgt, out_hidden=hs)
            torch.cuda.synchronize()
            h_ref, l_ref, nxt_ref, L = oracle.decode_step(m, lane, 4)
            assert eff[0] == 4
            assert rel_l2(hs.cpu().numpy()[0], h_ref) <= 1e-5, step
            assert rel_l2(lgt.cpu().numpy()[0], l_ref) <= 1e-5, step
            assert int(out.cpu()[0]) == nxt_ref, step
    finally:
        tl.tl_free(model)


@pytest.mark.parametrize("name", ["tiny-w4", "tiny-bf16-stack", "tiny-w4-wide", "tiny-wide"])
def test_tiny_decode_mixed_and_monotone_depth(name):
    """Lanes at different depths, per-token requests clamped to never rise."""
    spec = TINY[name]
    w = synth.make_weights(spec, seed=5)
    m = oracle.OracleModel.from_weights(w)
    n_lanes, plen, steps = 5, 12, 6
    L0 = [6, 1, 3, 8, 4]
    seqs = [synth.tokens(5, 4000 + i, plen + i, spec.vocab) for i in range(n_lanes)]
    reqs = np.array([[6, 5, 7, 2, 3, 1], [1, 1, 2, 1, 1, 1], [9, 3, 3, 2, 8, 1],
                     [8, 8, 4, 4, 4, 2], [2, 4, 1, 4, 4, 4]], np.int32)
    caps = [plen + i + steps for i in range(n_lanes)]
    model = load_model(w, max_lanes=8, max_pos=64, max_L=16, kv_arena_bytes=kv_bytes(spec, [16] * n_lanes, caps))
    try:
        lanes = [3, 0, 7, 1, 5]
        gpu_forward(model, spec, seqs, L0, lanes=lanes, max_new=steps)
        olanes = [oracle.prefill(m, s, L)[0] for s, L in zip(seqs, L0)]
        out = torch.empty(n_lanes, dtype=torch.int32, device="cuda")
        hs = torch.empty(n_lanes, spec.d_model, dtype=torch.float32, device="cuda")
        for t in range(steps):
            # teacher-force both sides with the oracle's greedy tokens
            feed = torch.tensor([ol.pending for ol in olanes], dtype=torch.int32, device="cuda")
            eff = tl.tl_decode_step(model, lanes, reqs[:, t], out, in_tokens=feed, out_hidden=hs)
            torch.cuda.synchronize()
            for i, ol in enumerate(olanes):
                h_ref, l_ref, nxt_ref, L = oracle.decode_step(m, ol, int(reqs[i, t]))
                assert eff[i] == L
                r = rel_l2(hs.cpu().numpy()[i], h_ref)
                assert r <= hidden_bar(spec, L), (t, i, r)
    finally:
        tl.tl_free(model)


def test_cfg2_forward_full_size():
    """Forward scoring on the 2048-wide INT4-loop model, 1 x 128 tokens, L = 8, no logits."""
    spec = synth.SPECS[2]
    say("cfg2 forward")
    w = synth.make_weights(spec, seed=0)
    m = oracle.OracleModel.from_weights(w)
    toks = synth.tokens(0, synth.STREAM_TOKENS, 128, spec.vocab)
    model = load_model(w, max_pos=256)
    try:
        hid, _, _, log, depth = gpu_forward(model, spec, [toks], [8], logits=False)
    finally:
        tl.tl_free(model)
    check_log(log, depth)
    _, ref_h, _ = oracle.prefill(m, toks, 8, want_logits="none")
    r = rel_l2(hid, ref_h)
    say("cfg2 rel", r)
    assert r <= 1e-2


@pytest.mark.parametrize("name", ["tiny-w4", "tiny-bf16-stack"])
def test_graph_replay_matches_eager(name):
    """Repeated scoring calls on a stream replay a captured graph; every replay,
    with eager work and synchronisations between them, equals the eager pass."""
    spec = TINY[name]
    w = synth.make_weights(spec, seed=21)
    seqs = [synth.tokens(21, 6000 + i, n, spec.vocab) for i, n in enumerate([40, 7, 66])]
    Ls = [3, 1, 5]
    model = load_model(w, max_pos=128, max_L=8)
    try:
        toks = torch.tensor(np.concatenate(seqs), dtype=torch.int32, device="cuda")
        cu = np.cumsum([0] + [len(s) for s in seqs]).astype(np.int32)
        T = int(cu[-1])
        ref = torch.empty(T, spec.d_model, dtype=torch.float32, device="cuda")
        ref_next = torch.empty(3, dtype=torch.int32, device="cuda")
        tl.tl_forward(model, cu, toks, seq_L=Ls, out_hidden=ref, out_next=ref_next, stream=0)   # eager
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        hid = torch.empty(T, spec.d_model, dtype=torch.float32, device="cuda")
        nxt = torch.empty(3, dtype=torch.int32, device="cuda")
        other = torch.empty(T, spec.d_model, dtype=torch.float32, device="cuda")
        for rep in range(4):
            hid.fill_(float("nan"))
            nxt.fill_(-1)
            torch.cuda.synchronize()
            tl.tl_forward(model, cu, toks, seq_L=Ls, out_hidden=hid, out_next=nxt, stream=side)
            side.synchronize()
            assert torch.equal(hid, ref), rep
            assert torch.equal(nxt, ref_next), rep
            # eager work on the same model between replays
            tl.tl_forward(model, cu, toks, seq_L=[1, 1, 1], out_hidden=other, stream=0)
            torch.cuda.synchronize()
    finally:
        tl.tl_free(model)


@pytest.mark.parametrize("name", ["tiny-f32", "tiny-w4"])
def test_degenerate_sizes_and_forward_errors(name):
    """One-token prompts at depth 1 and at the model's max_L, next to a prompt
    whose new tokens fill max_pos exactly, against the oracle; then calls that
    break tl_forward's rules (an empty sequence, depth 0 or above max_L, a
    cu_seqlens not starting at 0, a prompt that leaves too few positions for its
    new tokens) fail before any device work, and one cached step per lane still
    matches the oracle."""
    spec = TINY[name]
    say("degenerate sizes", name)
    w = synth.make_weights(spec, seed=6)
    m = oracle.OracleModel.from_weights(w)
    MAXP, MAXL, NEW = 64, 16, 8
    seqs = [synth.tokens(6, 600, 1, spec.vocab), synth.tokens(6, 601, 1, spec.vocab),
            synth.tokens(6, 602, MAXP - NEW, spec.vocab)]
    Ls = [1, MAXL, 3]
    model = load_model(w, max_lanes=4, max_pos=MAXP, max_L=MAXL,
                       kv_arena_bytes=kv_bytes(spec, Ls, [len(s) + NEW for s in seqs]))
    try:
        hid, lg, nxt, log, depth = gpu_forward(model, spec, seqs, Ls, lanes=[0, 1, 2], max_new=NEW)
        check_log(log, depth)
        ref_h, ref_lg, _ = oracle.forward_batch(m, seqs, Ls)
        off = 0
        for i, s in enumerate(seqs):
            r = rel_l2(hid[off:off + len(s)], ref_h[off:off + len(s)])
            say(name, "prompt", len(s), "L", Ls[i], "hidden rel %.2e" % r)
            assert r <= hidden_bar(spec, Ls[i]), (i, r)
            off += len(s)
        assert rel_l2(lg, ref_lg) <= (1e-4 if spec.act_dtype == "f32" else 1e-2)
        gaps = near_tie_gaps(nxt, ref_lg)
        assert (not gaps) if spec.act_dtype == "f32" else all(g <= 0.05 for g in gaps), gaps

        one = torch.tensor(seqs[0], dtype=torch.int32, device="cuda")
        longer = torch.tensor(synth.tokens(6, 604, MAXP - NEW + 1, spec.vocab), dtype=torch.int32, device="cuda")
        bad = [(dict(cu_seqlens=[0, 0], tokens=one, L=1), tl.TL_E_ARG),            # empty sequence
               (dict(cu_seqlens=[0, 1], tokens=one, L=0), tl.TL_E_ARG),            # depth 0
               (dict(cu_seqlens=[0, 1], tokens=one, L=MAXL + 1), tl.TL_E_ARG),     # above max_L
               (dict(cu_seqlens=[1, 2], tokens=one, L=1), tl.TL_E_ARG),            # cu_seqlens[0] != 0
               (dict(cu_seqlens=[0, MAXP - NEW + 1], tokens=longer, L=1, lanes=[3], max_new_tokens=NEW),
                tl.TL_E_STATE)]                                                     # 65 positions > 64
        for kw, want in bad:
            with pytest.raises(tl.TLError) as ei:
                tl.tl_forward(model, **kw)
            say(name, "rejected:", ei.value)
            assert ei.value.status == want, (kw, ei.value)

        feed = synth.tokens(6, 603, 3, spec.vocab)
        out = torch.empty(3, dtype=torch.int32, device="cuda")
        hs = torch.empty(3, spec.d_model, dtype=torch.float32, device="cuda")
        lgd = torch.empty(3, spec.vocab, dtype=torch.float32, device="cuda")
        eff = tl.tl_decode_step(model, [0, 1, 2], Ls, out,
                                in_tokens=torch.tensor(feed, dtype=torch.int32, device="cuda"),
                                out_logits=lgd, out_hidden=hs)
        torch.cuda.synchronize()
        Hd, LGd = hs.cpu().numpy(), lgd.cpu().numpy()
        for i, (s, L) in enumerate(zip(seqs, Ls)):
            lane, _, _ = oracle.prefill(m, s, L)
            h_o, l_o, _, L_o = oracle.decode_step(m, lane, L, token=int(feed[i]))
            r, rl = rel_l2(Hd[i], h_o), rel_l2(LGd[i], l_o)
            say(name, "step lane", i, "ctx", len(s) + 1, "L", L, "hidden %.2e logits %.2e" % (r, rl))
            assert eff[i] == L_o
            assert r <= hidden_bar(spec, L) and rl <= (1e-4 if spec.act_dtype == "f32" else 1e-2), (i, r, rl)
    finally:
        tl.tl_free(model)
