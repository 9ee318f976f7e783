"""Error paths that need the device: an allocator that runs out of memory
(TL_E_OOM, with the model left usable and every byte given back), and calls of
one model on two streams in turn.
"""
import sys

import numpy as np
import pytest

import synth
from tests.harness import ensure_built, make_config

torch = pytest.importorskip("torch")
import looped_transformer_amd as tl  # noqa: E402

pytestmark = pytest.mark.gpu

SPEC = synth.ModelSpec("tiny-w4", 256, 128, 4, 32, 256, 1, 1, 0, "f16", "w4g128")


def say(*a):
    print("[gpu-errors]", *a, flush=True)
    sys.stdout.flush()


class BudgetAllocator(tl.TorchAllocator):
    """torch's caching allocator with a byte budget: requests beyond it get NULL."""

    def __init__(self, budget):
        self.budget = budget
        self.used = 0
        self.sizes = {}
        super().__init__()

    def _alloc(self, nbytes, user):
        if self.used + nbytes > self.budget:
            return None
        p = super()._alloc(nbytes, user)
        if p:
            self.used += int(nbytes)
            self.sizes[p] = int(nbytes)
        return p

    def _free(self, p, user):
        self.used -= self.sizes.pop(p, 0)
        super()._free(p, user)


def _load(w, alloc):
    cfg = make_config(w.spec, max_pos=512, max_L=8)
    return tl.tl_load_weights(cfg, w.embed, w.head, w.final_norm, w.blocks, allocator=alloc)


def _score(model, toks, n):
    cu = np.array([0, n], np.int32)
    hid = torch.empty(n, SPEC.d_model, dtype=torch.float32, device="cuda")
    tl.tl_forward(model, cu, toks[:n], L=3, out_hidden=hid, stream=0)
    torch.cuda.synchronize()
    return hid.cpu().numpy()


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def test_load_out_of_memory_returns_every_byte():
    w = synth.make_weights(SPEC, seed=2)
    alloc = BudgetAllocator(256 << 10)
    with pytest.raises(tl.TLError) as ei:
        _load(w, alloc)
    say("load with 256 KiB:", ei.value)
    assert ei.value.status == tl.TL_E_OOM
    assert alloc.used == 0 and not alloc.live


def test_call_out_of_memory_leaves_model_usable():
    w = synth.make_weights(SPEC, seed=2)
    toks = torch.tensor(synth.tokens(2, 50, 400, SPEC.vocab), dtype=torch.int32, device="cuda")
    # how much a 16-row scoring call needs, with a generous budget
    probe = BudgetAllocator(1 << 34)
    model = _load(w, probe)
    try:
        ref = _score(model, toks, 16)
        need = probe.used
    finally:
        tl.tl_free(model)
    assert probe.used == 0
    # a budget that fits the 16-row call but not a 400-row one
    alloc = BudgetAllocator(need + (64 << 10))
    model = _load(w, alloc)
    try:
        a = _score(model, toks, 16)
        assert np.array_equal(a, ref)
        with pytest.raises(tl.TLError) as ei:
            _score(model, toks, 400)
        say("400-row call within %d bytes:" % alloc.budget, ei.value)
        assert ei.value.status == tl.TL_E_OOM
        b = _score(model, toks, 16)          # the model still works and gives the same result
        assert np.array_equal(b, ref)
    finally:
        tl.tl_free(model)
    assert alloc.used == 0 and not alloc.live


def test_calls_on_alternating_streams():
    """Calls of one model on two streams in turn: each waits for the other's work
    on the shared staging area and workspaces, so every result equals the first."""
    w = synth.make_weights(SPEC, seed=4)
    toks = torch.tensor(synth.tokens(4, 60, 300, SPEC.vocab), dtype=torch.int32, device="cuda")
    model = _load(w, "torch")
    try:
        ref = _score(model, toks, 300)
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        outs = []
        cu_long = np.array([0, 300], np.int32)
        cu_short = np.array([0, 7], np.int32)
        for rep in range(6):
            st = streams[rep % 2]
            hid = torch.empty(300, SPEC.d_model, dtype=torch.float32, device="cuda")
            small = torch.empty(7, SPEC.d_model, dtype=torch.float32, device="cuda")
            # a long call, then at once a short one on the other stream (different
            # descriptors in the shared staging area), no host wait in between
            tl.tl_forward(model, cu_long, toks, L=3, out_hidden=hid, stream=st.cuda_stream)
            tl.tl_forward(model, cu_short, toks, L=1, out_hidden=small, stream=streams[1 - rep % 2].cuda_stream)
            outs.append(hid)
        torch.cuda.synchronize()
        for rep, h in enumerate(outs):
            assert np.array_equal(h.cpu().numpy(), ref), rep
    finally:
        tl.tl_free(model)
