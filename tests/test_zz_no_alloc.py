"""tl_decode_step_noalloc (the decode step that allocates nothing, running on the
library's per-device scratch array) against tl_decode_step on the same lanes.

Two copies of each lane are prefilled identically; every step runs once through
each entry point (three calls in a row, the second with fewer lanes than the
first, one fed from the lanes' pending tokens).  The two paths launch the same
kernels with the same split choices, so tokens, logits, hidden states and depths
must be equal bit for bit.  Also: the scratch-size limit and the store-h modes
are refused with their status codes.
"""
import sys

import numpy as np
import pytest

import synth
from tests.harness import ensure_built, kv_bytes, load_model

torch = pytest.importorskip("torch")
import looped_transformer_amd as tl  # noqa: E402

pytestmark = pytest.mark.gpu

SPECS = {
    "tiny-w4": synth.ModelSpec("tiny-w4", 256, 128, 4, 32, 256, 1, 1, 0, "f16", "w4g128"),
    "tiny-w4-wide": synth.ModelSpec("tiny-w4-wide", 256, 256, 4, 64, 2048, 1, 1, 0, "f16", "w4g128"),
    "tiny-bf16-stack": synth.ModelSpec("tiny-bf16-stack", 320, 192, 2, 96, 384, 2, 2, 1, "bf16", "bf16"),
    "tiny-f32": synth.SPECS[1],
    "mid-w4": synth.ModelSpec("mid-w4", 4096, 1024, 8, 128, 2816, 1, 1, 0, "f16", "w4g128"),
}


def say(*a):
    print("[gpu-noalloc]", *a, flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), dtype=torch.int32, device="cuda")


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


@pytest.mark.parametrize("name", list(SPECS))
def test_noalloc_equals_decode_step(name):
    spec = SPECS[name]
    w = synth.make_weights(spec, seed=17)
    plens = [5, 17, 40, 9, 66, 23]
    Ls = [3, 1, 4, 2, 4, 3]
    n = len(plens)
    prompts = [synth.tokens(17, 5000 + i, p, spec.vocab) for i, p in enumerate(plens)]
    model = load_model(w, max_lanes=16, max_pos=128, max_L=8,
                       kv_arena_bytes=kv_bytes(spec, Ls * 2, [p + 8 for p in plens] * 2))
    try:
        cu = np.concatenate([[0], np.cumsum(plens)]).astype(np.int32)
        toks = _dev(np.concatenate(prompts))
        A = list(range(n))                      # lanes of tl_decode_step
        B = list(range(8, 8 + n))               # lanes of tl_decode_step_noalloc
        tl.tl_forward(model, cu, toks, seq_L=Ls, lanes=A, max_new_tokens=8)
        tl.tl_forward(model, cu, toks, seq_L=Ls, lanes=B, max_new_tokens=8)
        torch.cuda.synchronize()
        calls = [
            (list(range(n)), [4, 4, 2, 3, 1, 3], synth.tokens(17, 5100, n, spec.vocab)),
            ([1, 4], [2, 4], None),             # fewer lanes; their pending tokens
            ([0, 2, 3, 5], [1, 4, 4, 2], synth.tokens(17, 5101, 4, spec.vocab)),
        ]
        for c, (idx, req, feed) in enumerate(calls):
            k = len(idx)
            outs = []
            for fn, lanes in ((tl.tl_decode_step, A), (tl.tl_decode_step_noalloc, B)):
                ot = torch.full((k,), -1, dtype=torch.int32, device="cuda")
                lg = torch.full((k, spec.vocab), float("nan"), dtype=torch.float32, device="cuda")
                hs = torch.full((k, spec.d_model), float("nan"), dtype=torch.float32, device="cuda")
                eff = fn(model, [lanes[i] for i in idx], req, ot, in_tokens=None if feed is None else _dev(feed),
                         out_logits=lg, out_hidden=hs)
                torch.cuda.synchronize()
                outs.append((eff, ot.cpu().numpy(), lg.cpu().numpy(), hs.cpu().numpy()))
            (e0, t0, l0, h0), (e1, t1, l1, h1) = outs
            say(name, "call", c, "lanes", k, "depths", list(e1), "tokens", list(t1))
            assert np.array_equal(e0, e1), c
            assert np.array_equal(t0, t1), c
            assert np.array_equal(l0, l1), c
            assert np.array_equal(h0, h1), c
            assert np.all(np.isfinite(h1)) and np.all(t1 >= 0)
    finally:
        tl.tl_free(model)


def test_noalloc_limits():
    spec = SPECS["tiny-w4"]
    w = synth.make_weights(spec, seed=18)
    model = load_model(w, max_lanes=20000, max_pos=64, max_L=4)
    try:
        out = torch.empty(20000, dtype=torch.int32, device="cuda")
        with pytest.raises(tl.TLError) as ei:
            tl.tl_decode_step_noalloc(model, np.arange(20000), np.ones(20000, np.int32), out)
        say("20000 lanes:", ei.value)
        assert ei.value.status == tl.TL_E_ARG and "scratch" in ei.value.message
    finally:
        tl.tl_free(model)
    model = load_model(w, max_lanes=2, max_pos=64, max_L=4, kv_arena_bytes=kv_bytes(spec, [2], [32]),
                       kv_mode=tl.TL_KV_H)
    try:
        out = torch.empty(1, dtype=torch.int32, device="cuda")
        with pytest.raises(tl.TLError) as ei:
            tl.tl_decode_step_noalloc(model, [0], [2], out)
        assert ei.value.status == tl.TL_E_UNSUPPORTED
    finally:
        tl.tl_free(model)
