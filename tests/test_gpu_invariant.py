"""Batch invariance (tl_config.batch_invariant = 1): a row's results do not depend
on the other rows of its passes, bit for bit.

* a mixed-depth batch of sequences equals each sequence scored alone ("Dynamic-L
  Inference" page, "L-Aware Batching": lanes of one batch run at their own depth);
* continuous-depth decoding (tl_decode_run, "Continuous Depth Batching" summary
  page: work scheduled one loop iteration at a time across lanes) equals
  step-by-step decoding, and a decode step of many lanes equals each lane alone;
* a product whose split-K partials exceed the workspace runs in row chunks with
  the same arithmetic (a 5000-row forward equals its sequences alone).
Models: INT4 loop block (fp16 operands), a bf16 loop stack, and bf16 weights with
fp32 activations (split fp16 operands).
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
    "tiny-wide": synth.ModelSpec("tiny-wide", 320, 192, 2, 96, 384, 2, 2, 1, "bf16", "bf16", act="f32"),
}


def say(*a):
    print("[gpu-invariant]", *a, flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), dtype=torch.int32, device="cuda")


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _score(model, spec, seqs, Ls):
    cu = np.concatenate([[0], np.cumsum([len(s) for s in seqs])]).astype(np.int32)
    hid = torch.empty(int(cu[-1]), spec.d_model, dtype=torch.float32, device="cuda")
    lg = torch.empty(len(seqs), spec.vocab, dtype=torch.float32, device="cuda")
    tl.tl_forward(model, cu, _dev(np.concatenate(seqs)), seq_L=Ls, out_hidden=hid, out_logits=lg, stream=0)
    torch.cuda.synchronize()
    return hid.cpu().numpy(), lg.cpu().numpy(), cu


@pytest.mark.parametrize("name", list(SPECS))
def test_mixed_batch_equals_each_alone(name):
    spec = SPECS[name]
    w = synth.make_weights(spec, seed=31)
    seqs = [synth.tokens(31, 8000 + i, n, spec.vocab) for i, n in enumerate([37, 5, 70, 1, 19])]
    Ls = [3, 6, 1, 4, 2]
    model = load_model(w, max_pos=256, max_L=8, batch_invariant=1)
    try:
        H, LG, cu = _score(model, spec, seqs, Ls)
        for i, (sq, L) in enumerate(zip(seqs, Ls)):
            h1, l1, _ = _score(model, spec, [sq], [L])
            assert np.array_equal(H[cu[i]:cu[i + 1]], h1), (name, i)
            assert np.array_equal(LG[i], l1[0]), (name, i)
    finally:
        tl.tl_free(model)


@pytest.mark.parametrize("name", list(SPECS))
def test_continuous_depth_equals_lockstep(name):
    spec = SPECS[name]
    w = synth.make_weights(spec, seed=32)
    n, steps = 6, 7
    plens = [9, 30, 4, 17, 45, 12]
    L1 = np.array([5, 2, 8, 3, 6, 1], np.int32)
    prompts = [synth.tokens(32, 8100 + i, p, spec.vocab) for i, p in enumerate(plens)]
    reqs = np.minimum(8, 1 + synth.poisson(32, 8200, n * steps, 3.0).reshape(n, steps)).astype(np.int32)
    feed = synth.tokens(32, 8300, n * steps, spec.vocab).reshape(n, steps)
    model = load_model(w, max_lanes=n, max_pos=128, max_L=8, batch_invariant=1,
                       kv_arena_bytes=kv_bytes(spec, L1, [p + steps for p in plens]))
    try:
        cu = np.concatenate([[0], np.cumsum(plens)]).astype(np.int32)
        toks = _dev(np.concatenate(prompts))
        lanes = np.arange(n, dtype=np.int32)

        def prefill():
            tl.tl_forward(model, cu, toks, seq_L=L1, lanes=lanes, max_new_tokens=steps, stream=0)

        prefill()
        run_t = torch.empty(n, steps, dtype=torch.int32, device="cuda")
        run_h = torch.empty(n, steps, spec.d_model, dtype=torch.float32, device="cuda")
        eff = tl.tl_decode_run(model, lanes, reqs, run_t, in_tokens=_dev(feed), out_hidden=run_h, boundary_min=2,
                               stream=0)
        torch.cuda.synchronize()
        RT, RH = run_t.cpu().numpy(), run_h.cpu().numpy()
        # lockstep, all lanes per step
        prefill()
        out = torch.empty(n, dtype=torch.int32, device="cuda")
        hs = torch.empty(n, spec.d_model, dtype=torch.float32, device="cuda")
        for t in range(steps):
            e2 = tl.tl_decode_step(model, lanes, reqs[:, t], out, in_tokens=_dev(feed[:, t]), out_hidden=hs, stream=0)
            torch.cuda.synchronize()
            assert np.array_equal(e2, eff[:, t])
            assert np.array_equal(out.cpu().numpy(), RT[:, t]), (name, t)
            assert np.array_equal(hs.cpu().numpy(), RH[:, t]), (name, t)
        # one lane at a time
        prefill()
        o1 = torch.empty(1, dtype=torch.int32, device="cuda")
        h1 = torch.empty(1, spec.d_model, dtype=torch.float32, device="cuda")
        for t in range(steps):
            for i in range(n):
                tl.tl_decode_step(model, [i], [reqs[i, t]], o1, in_tokens=_dev(feed[i:i + 1, t]), out_hidden=h1,
                                  stream=0)
                torch.cuda.synchronize()
                assert int(o1.cpu()[0]) == RT[i, t], (name, t, i)
                assert np.array_equal(h1.cpu().numpy()[0], RH[i, t]), (name, t, i)
        say(name, "continuous depth == lockstep == lanes alone over", n, "lanes x", steps, "steps")
    finally:
        tl.tl_free(model)


def test_split_partials_in_row_chunks():
    """The wide INT4 model's down projection (K = 2048, N = 256) splits K 8 ways, so
    a product of more than 4096 rows would overflow the partial workspace and runs
    in row chunks."""
    spec = SPECS["tiny-w4-wide"]
    w = synth.make_weights(spec, seed=33)
    seqs = [synth.tokens(33, 8400, 2600, spec.vocab), synth.tokens(33, 8401, 2400, spec.vocab)]
    model = load_model(w, max_pos=4096, max_L=4, batch_invariant=1)
    try:
        H, LG, cu = _score(model, spec, seqs, [2, 2])
        for i, sq in enumerate(seqs):
            h1, l1, _ = _score(model, spec, [sq], [2])
            assert np.array_equal(H[cu[i]:cu[i + 1]], h1), i
            assert np.array_equal(LG[i], l1[0]), i
    finally:
        tl.tl_free(model)
