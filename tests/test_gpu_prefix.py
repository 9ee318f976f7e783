"""Shared-prefix reuse on the device against the oracle ("Benchmark Comparison"
page, measured benchmarks, section 2: a prefix's cache is computed once and
reused by many requests, in every loop iteration's slot).

tl_lane_fork copies a prefix of every cache slot into a new lane; tl_append runs
the cached forward of several new tokens per lane.  A request built from a forked
prefix must match the oracle's fork + append (which the CPU pins tie to a full
prefill of the request), then decode from it.  Tokens are seeded (teacher
forcing); hidden states and logits meet the usual bars; depths are exact.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from tests.harness import ensure_built, kv_bytes, load_model, rel_l2

torch = pytest.importorskip("torch")
import looped_transformer_amd as tl  # noqa: E402

pytestmark = pytest.mark.gpu

SPECS = {
    "tiny-fp32": synth.SPECS[1],
    "tiny-w4": synth.ModelSpec("tiny-w4", 256, 128, 4, 32, 256, 1, 1, 0, "f16", "w4g128"),
    "tiny-bf16-stack": synth.ModelSpec("tiny-bf16-stack", 320, 192, 2, 96, 384, 2, 2, 1, "bf16", "bf16"),
    "mid-w4": synth.ModelSpec("mid-w4", 256, 512, 8, 64, 1024, 1, 1, 0, "f16", "w4g128"),
}
L0, PLEN, CAP_NEW = 6, 13, 64


def say(*a):
    print("[gpu-prefix]", *a, flush=True)
    sys.stdout.flush()


def bar(spec, L):
    if spec.act_dtype == "f32":
        return 1e-4
    return 1e-2 if L <= 8 else 3e-2


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _dev(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("name", list(SPECS))
def test_fork_and_append_match_oracle(name):
    spec = SPECS[name]
    w = synth.make_weights(spec, 41)
    m = oracle.OracleModel.from_weights(w)
    prefix = synth.tokens(41, 6000, PLEN, spec.vocab)
    # (dst lane, prefix length, suffix length, requested depth of the suffix)
    forks = [(5, PLEN, 45, 6), (0, 7, 4, 9), (7, 1, 20, 3)]
    src = 2
    src_more, src_L = 3, 5                      # the source itself is appended to as well
    suffixes = {d: synth.tokens(41, 6100 + d, n, spec.vocab) for d, _, n, _ in forks}
    suffixes[src] = synth.tokens(41, 6200, src_more, spec.vocab)

    # ---- oracle
    o_src = oracle.prefill(m, prefix, L0)[0]
    o_lanes = {d: oracle.fork(o_src, P) for d, P, _, _ in forks}
    o_lanes[src] = o_src
    req = {d: Lr for d, _, _, Lr in forks}
    req[src] = src_L
    order = [5, 0, 7, src]
    o_h, o_lg = {}, {}
    for d in order:
        o_h[d], o_lg[d] = oracle.append(m, o_lanes[d], suffixes[d], req[d])

    # ---- device
    caps = [PLEN + CAP_NEW] * 4
    model = load_model(w, max_lanes=8, max_pos=128, max_L=16, kv_arena_bytes=kv_bytes(spec, [L0] * 4, caps))
    try:
        tl.tl_forward(model, np.array([0, PLEN], np.int32), _dev(prefix), L=L0, lanes=[src], max_new_tokens=CAP_NEW)
        for d, P, _, _ in forks:
            tl.tl_lane_fork(model, src, d, P, max_new_tokens=CAP_NEW)
        lens = [len(suffixes[d]) for d in order]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        toks = _dev(np.concatenate([suffixes[d] for d in order]))
        hid = torch.empty(int(cu[-1]), spec.d_model, dtype=torch.float32, device="cuda")
        lg = torch.empty(len(order), spec.vocab, dtype=torch.float32, device="cuda")
        nxt = torch.empty(len(order), dtype=torch.int32, device="cuda")
        eff = tl.tl_append(model, cu, toks, order, [req[d] for d in order], out_hidden=hid, out_logits=lg,
                           out_next=nxt)
        torch.cuda.synchronize()
        H, LG = hid.cpu().numpy(), lg.cpu().numpy()
        for i, d in enumerate(order):
            want_L = o_lanes[d].ceiling
            assert eff[i] == want_L, (d, eff[i], want_L)
            r = rel_l2(H[cu[i]:cu[i + 1]], o_h[d])
            rl = rel_l2(LG[i], o_lg[d])
            say(name, "lane", d, "rows", lens[i], "L", int(eff[i]), "hidden rel %.2e logits rel %.2e" % (r, rl))
            assert r <= bar(spec, want_L) and rl <= bar(spec, want_L), (d, r, rl)

        # three teacher-forced decode steps on every lane, from the appended state
        feed = synth.tokens(41, 6300, 3 * len(order), spec.vocab).reshape(3, len(order))
        out = torch.empty(len(order), dtype=torch.int32, device="cuda")
        hs = torch.empty(len(order), spec.d_model, dtype=torch.float32, device="cuda")
        for t in range(3):
            e = tl.tl_decode_step(model, order, [8] * len(order), out, in_tokens=_dev(feed[t]), out_hidden=hs)
            torch.cuda.synchronize()
            Hd = hs.cpu().numpy()
            for i, d in enumerate(order):
                h_o, _, _, L_o = oracle.decode_step(m, o_lanes[d], 8, token=int(feed[t, i]))
                assert e[i] == L_o
                assert rel_l2(Hd[i], h_o) <= bar(spec, L_o), (t, d, rel_l2(Hd[i], h_o))
    finally:
        tl.tl_free(model)


def test_full_fork_takes_the_pending_token():
    """A fork of the whole lane decodes from the source's pending token: the same
    step fed that token explicitly (device against device, single-lane calls)."""
    spec = SPECS["tiny-w4"]
    w = synth.make_weights(spec, 43)
    prefix = synth.tokens(43, 6400, 21, spec.vocab)
    model = load_model(w, max_lanes=8, max_pos=128, max_L=16, kv_arena_bytes=kv_bytes(spec, [L0] * 3, [60] * 3))
    try:
        nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        tl.tl_forward(model, np.array([0, 21], np.int32), _dev(prefix), L=L0, lanes=[1], max_new_tokens=20,
                      out_next=nxt)
        tl.tl_lane_fork(model, 1, 4, 21, max_new_tokens=20)
        tl.tl_lane_fork(model, 1, 6, 21, max_new_tokens=20)
        outs, hids = [], []
        for lane, feed in [(4, None), (6, nxt)]:
            o = torch.empty(1, dtype=torch.int32, device="cuda")
            h = torch.empty(1, spec.d_model, dtype=torch.float32, device="cuda")
            tl.tl_decode_step(model, [lane], [L0], o, in_tokens=feed, out_hidden=h)
            torch.cuda.synchronize()
            outs.append(int(o.item()))
            hids.append(h.cpu().numpy())
        assert outs[0] == outs[1] and np.array_equal(hids[0], hids[1])
    finally:
        tl.tl_free(model)


def test_fork_after_the_ceiling_dropped():
    """The source decoded at a lower depth: the fork takes the lower ceiling and a
    deeper request on the child is clamped to it (oracle: same clamping)."""
    spec = SPECS["tiny-w4"]
    w = synth.make_weights(spec, 47)
    m = oracle.OracleModel.from_weights(w)
    prefix = synth.tokens(47, 6500, 11, spec.vocab)
    feed = synth.tokens(47, 6501, 2, spec.vocab)
    suffix = synth.tokens(47, 6502, 9, spec.vocab)
    o_src = oracle.prefill(m, prefix, 7)[0]
    for t in range(2):
        oracle.decode_step(m, o_src, 3, token=int(feed[t]))
    o_child = oracle.fork(o_src, 12)
    o_h, o_lg = oracle.append(m, o_child, suffix, 7)
    model = load_model(w, max_lanes=8, max_pos=128, max_L=16, kv_arena_bytes=kv_bytes(spec, [7] * 2, [60] * 2))
    try:
        tl.tl_forward(model, np.array([0, 11], np.int32), _dev(prefix), L=7, lanes=[3], max_new_tokens=30)
        out = torch.empty(1, dtype=torch.int32, device="cuda")
        for t in range(2):
            tl.tl_decode_step(model, [3], [3], out, in_tokens=_dev(feed[t:t + 1]))
        tl.tl_lane_fork(model, 3, 0, 12, max_new_tokens=20)
        hid = torch.empty(9, spec.d_model, dtype=torch.float32, device="cuda")
        lg = torch.empty(1, spec.vocab, dtype=torch.float32, device="cuda")
        eff = tl.tl_append(model, [0, 9], _dev(suffix), [0], [7], out_hidden=hid, out_logits=lg)
        torch.cuda.synchronize()
        assert eff[0] == 3 == o_child.ceiling
        assert rel_l2(hid.cpu().numpy(), o_h) <= 1e-2 and rel_l2(lg.cpu().numpy()[0], o_lg) <= 1e-2
    finally:
        tl.tl_free(model)


def test_fork_and_append_errors():
    spec = SPECS["tiny-w4"]
    w = synth.make_weights(spec, 53)
    prefix = synth.tokens(53, 6600, 9, spec.vocab)
    model = load_model(w, max_lanes=4, max_pos=64, max_L=16, kv_arena_bytes=kv_bytes(spec, [4] * 4, [64] * 4))
    try:
        tl.tl_forward(model, np.array([0, 9], np.int32), _dev(prefix), L=4, lanes=[0], max_new_tokens=4)

        def status(fn, *a, **k):
            with pytest.raises(tl.TLError) as ei:
                fn(*a, **k)
            return ei.value.status

        assert status(tl.tl_lane_fork, model, 0, 0, 5) == tl.TL_E_ARG            # onto itself
        assert status(tl.tl_lane_fork, model, 0, 1, 10) == tl.TL_E_ARG           # longer than the lane
        assert status(tl.tl_lane_fork, model, 0, 1, 0) == tl.TL_E_ARG            # empty prefix
        assert status(tl.tl_lane_fork, model, 0, 9, 3) == tl.TL_E_ARG            # lane out of range
        assert status(tl.tl_lane_fork, model, 2, 1, 1) == tl.TL_E_STATE          # source never prefilled
        assert status(tl.tl_lane_fork, model, 0, 1, 9, max_new_tokens=60) == tl.TL_E_STATE   # beyond max_pos
        five = _dev(np.arange(5))
        assert status(tl.tl_append, model, [0, 5], five, [0], [4]) == tl.TL_E_STATE   # capacity 13, 14 needed
        assert status(tl.tl_append, model, [0, 2], five, [3], [4]) == tl.TL_E_STATE   # never prefilled
        assert status(tl.tl_append, model, [0, 2], five, [0], [0]) == tl.TL_E_ARG     # L < 1
        tl.tl_lane_fork(model, 0, 1, 5, max_new_tokens=4)                           # partial: no pending token
        out = torch.empty(1, dtype=torch.int32, device="cuda")
        assert status(tl.tl_decode_step, model, [1], [4], out) == tl.TL_E_STATE
        tl.tl_append(model, [0, 2], five, [1], [4])                                 # now it has one
        tl.tl_decode_step(model, [1], [4], out)
        torch.cuda.synchronize()
        tl.tl_sync_errors(model)
    finally:
        tl.tl_free(model)
