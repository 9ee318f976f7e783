"""Kernel-class timing on the device: the event pairs recorded around each launch
group (tl_timing_read) and the pairs the runtime stamps with each kernel's own start
and end (tl_timing_read_kernels).  Timing must not change a result, every
product, attention and embedding group must hold at least one stamped kernel,
and the kernels' own time must lie within the groups'.
"""
import sys

import numpy as np
import pytest

import synth
from tests.harness import ensure_built, load_model

torch = pytest.importorskip("torch")
import looped_transformer_amd as tl  # noqa: E402

pytestmark = pytest.mark.gpu

SPEC = synth.ModelSpec("tiny-w4", 256, 128, 4, 32, 256, 1, 1, 0, "f16", "w4g128")
PRODUCTS = ("gemm_qkv_loop", "gemm_o_loop", "gemm_gu_loop", "gemm_down_loop", "gemm_qkv_boundary",
            "gemm_o_boundary", "gemm_gu_boundary", "gemm_down_boundary", "head")


def say(*a):
    print("[gpu-timing]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("rows", [3, 128])
def test_kernel_stamped_timing(rows):
    ensure_built()
    w = synth.make_weights(SPEC, seed=5)
    toks = torch.tensor(synth.tokens(5, 11, rows, SPEC.vocab), dtype=torch.int32, device="cuda")
    model = load_model(w, max_lanes=1, max_pos=256, max_L=8)
    try:
        cu = np.array([0, rows], np.int32)
        hid = [torch.empty(rows, SPEC.d_model, dtype=torch.float32, device="cuda") for _ in range(2)]
        lg = [torch.empty(1, SPEC.vocab, dtype=torch.float32, device="cuda") for _ in range(2)]
        tl.tl_forward(model, cu, toks, L=3, out_hidden=hid[0], out_logits=lg[0], stream=0)
        torch.cuda.synchronize()
        tl.tl_timing_enable(model, True)
        reps = 3
        for _ in range(reps):
            tl.tl_forward(model, cu, toks, L=3, out_hidden=hid[1], out_logits=lg[1], stream=0)
        torch.cuda.synchronize()
        cls = tl.tl_timing_read(model)
        kcls = tl.tl_timing_read_kernels(model)
        tl.tl_timing_enable(model, False)
        assert np.array_equal(hid[0].cpu().numpy(), hid[1].cpu().numpy())
        assert np.array_equal(lg[0].cpu().numpy(), lg[1].cpu().numpy())
        for k in PRODUCTS:
            (ms, n), (kms, nk) = cls[k], kcls[k]
            say("rows", rows, k, "groups", n, "event %.1f us" % (ms * 1e3), "kernels", nk, "stamped %.1f us" % (kms * 1e3))
            if k.endswith("_boundary"):
                continue                          # the tiny model has one pre block and no post block
            assert n > 0 and nk >= n, (k, n, nk)
            assert 0.0 < kms <= ms, (k, kms, ms)
        assert cls["gemm_gu_loop"][1] == 3 * reps
        for k in ("attention", "embed"):       # groups that always launch
            (ms, n), (kms, nk) = cls[k], kcls[k]
            say("rows", rows, k, "groups", n, "event %.1f us" % (ms * 1e3), "kernels", nk, "stamped %.1f us" % (kms * 1e3))
            assert n > 0 and nk >= n and 0.0 < kms <= ms, (k, n, nk, kms, ms)
        for k, (kms, nk) in kcls.items():
            assert kms <= cls[k][0] and (nk == 0) == (kms == 0.0), (k, kms, nk, cls[k])
        # a second read starts from zero
        assert all(v == (0.0, 0) for v in tl.tl_timing_read_kernels(model).values())
    finally:
        tl.tl_free(model)
