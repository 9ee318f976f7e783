"""Pins of three oracle parts that the whole-model pins do not reach on their own:

* ``fp16_body``: the FP16 body is fp16(q * s), one round-to-nearest-even of the
  exact product ("CLI Reference" page, environment variable
  TINYLOOP_EXPERIMENTAL_FP16_BODY: the body is dequantised once to an fp16 cache);
* ``bf16_bits_to_float``: decoding of stored bf16 weights;
* the order of block applications for a loop *stack* with pre and post blocks
  ("Benchmark Comparison / vs generic runtimes" page, "Where Generic Runtimes Lose
  On Looped Checkpoints": embed -> pre blocks -> shared loop block x L -> head; the
  loop stack is applied as a whole, iteration after iteration), with one cache slot
  per block application.

Each pin compares with an independent routine (torch's own conversions and
layers) or with hand values at the cases a plausible mistake would change.
CPU only.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


# ---------------------------------------------------------------------------
# FP16 body


def _all_finite_f16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


def test_fp16_body_equals_torch_half_of_exact_product():
    # every code q in [-8, 7] against every finite fp16 scale: torch rounds the
    # exact fp32 product (a 4-bit integer times an fp16 is exact in fp32) once
    scales = _all_finite_f16()
    n = scales.size
    for qv in range(-8, 8):
        q = np.full((n, 128), qv, dtype=np.int8)
        s = scales.reshape(n, 1)
        with np.errstate(over="ignore"):   # |q s| above 65504 is inf on both sides
            got = oracle.fp16_body(q, s)
        ref = (torch.full((n,), qv, dtype=torch.float32) * torch.from_numpy(scales.astype(np.float32))).half()
        g = got[:, 0].view(np.uint16)
        r = ref.numpy().view(np.uint16)
        # +0 and -0 are the same value (q = 0 or s = -0)
        assert np.array_equal(g[r != 0x8000], r[r != 0x8000])
        assert got.dtype == np.float16


def test_fp16_body_ties_round_to_even():
    # 3 * (1 + 2^-10) = 3 + 1.5 * 2^-9 sits halfway between two fp16 neighbours
    # (spacing 2^-9 in [2, 4)); ties to even give 3 + 2^-8.  Truncation gives
    # 3 + 2^-9; rounding half away from zero agrees here but not below.
    s1 = np.float16(1 + 2 ** -10)
    out = oracle.fp16_body(np.full((1, 128), 3, np.int8), np.array([[s1]], np.float16))
    assert float(out[0, 0]) == 3 + 2 ** -8
    # 3 * (1 + 3 * 2^-10) = 3 + 4.5 * 2^-9: ties to even give 3 + 4 * 2^-9 (half away
    # from zero would give 3 + 5 * 2^-9)
    s3 = np.float16(1 + 3 * 2 ** -10)
    out = oracle.fp16_body(np.full((1, 128), 3, np.int8), np.array([[s3]], np.float16))
    assert float(out[0, 0]) == 3 + 4 * 2 ** -9
    # -7 * (1 + 2^-10) = -(7 + 7 * 2^-10): spacing 2^-8 in [4, 8), 7 * 2^-10 = 1.75 * 2^-8
    # rounds up in magnitude to 7 + 2^-7
    out = oracle.fp16_body(np.full((1, 128), -7, np.int8), np.array([[s1]], np.float16))
    assert float(out[0, 0]) == -(7 + 2 ** -7)


def test_fp16_body_group_indexing():
    # two output rows, K = 256 (two groups): element (n, k) takes scale (n, k // 128)
    q = np.zeros((2, 256), np.int8)
    q[0, 0], q[0, 127], q[0, 128], q[1, 255] = 1, 2, 3, -4
    s = np.array([[0.5, 0.25], [2.0, 4.0]], np.float16)
    out = oracle.fp16_body(q, s).astype(np.float64)
    exp = np.zeros((2, 256))
    exp[0, 0], exp[0, 127], exp[0, 128], exp[1, 255] = 0.5, 1.0, 0.75, -16.0
    assert np.array_equal(out, exp)


# ---------------------------------------------------------------------------
# bf16 decoding


def test_bf16_bits_to_float_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_bits_to_float(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # hand values: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3C00 = 2^-7, 0x0001 = 2^-133 (subnormal)
    hv = oracle.bf16_bits_to_float(np.array([0x3F80, 0xC000, 0x3C00, 0x0001], np.uint16))
    assert list(hv) == [1.0, -2.0, 2.0 ** -7, 2.0 ** -133]


# ---------------------------------------------------------------------------
# loop stack with pre and post blocks (bf16 weights)

STACK = synth.ModelSpec("pin-bf16-stack", 96, 64, 2, 32, 128, 2, 2, 1, "bf16", "bf16")


@pytest.fixture(scope="module")
def stack_model():
    w = synth.make_weights(STACK, seed=3)
    return w, oracle.OracleModel.from_weights(w)


def _t_bf16(bits):
    """bf16 bits -> float64 tensor through torch's own bf16 type."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double()


def _torch_block(blk, h, pos, spec):
    """One pre-norm block with torch CPU layers (rms_norm, linear, complex rotation,
    scaled_dot_product_attention, silu), weights decoded by torch from bf16."""
    d, H, dh = spec.d_model, spec.n_heads, spec.head_dim
    T = h.shape[0]
    W = {k: _t_bf16(blk[k]) for k in ("wqkv", "wo", "wgate", "wup", "wdown")}
    g1 = torch.from_numpy(blk["norm1"].astype(np.float64))
    g2 = torch.from_numpy(blk["norm2"].astype(np.float64))
    x = F.rms_norm(h, (d,), g1, spec.rms_eps)
    q, k, v = F.linear(x, W["wqkv"]).split(d, dim=1)
    half = dh // 2
    inv = spec.rope_base ** (-torch.arange(half, dtype=torch.float64) * 2 / dh)
    rot = torch.polar(torch.ones(T, half, dtype=torch.float64),
                      torch.outer(torch.from_numpy(np.asarray(pos, np.float64)), inv))

    def rope(z):
        z = z.reshape(T, H, dh)
        c = torch.complex(z[..., :half], z[..., half:]) * rot[:, None, :]
        return torch.cat([c.real, c.imag], dim=-1)

    q, k, v = rope(q).transpose(0, 1), rope(k).transpose(0, 1), v.reshape(T, H, dh).transpose(0, 1)
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1).reshape(T, d)
    h = h + F.linear(o, W["wo"])
    x2 = F.rms_norm(h, (d,), g2, spec.rms_eps)
    return h + F.linear(F.silu(F.linear(x2, W["wgate"])) * F.linear(x2, W["wup"]), W["wdown"])


def _torch_forward(w, toks, L):
    spec = w.spec
    pos = np.arange(len(toks))
    h = _t_bf16(w.embed[toks])
    for b in range(spec.n_pre):
        h = _torch_block(w.blocks[b], h, pos, spec)
    for _ in range(L):                          # the stack as a whole, iteration-major
        for l in range(spec.n_loop):
            h = _torch_block(w.blocks[spec.n_pre + l], h, pos, spec)
    for b in range(spec.n_post):
        h = _torch_block(w.blocks[spec.n_pre + spec.n_loop + b], h, pos, spec)
    logits = F.linear(F.rms_norm(h, (spec.d_model,), torch.from_numpy(w.final_norm.astype(np.float64)),
                                 spec.rms_eps), _t_bf16(w.head))
    return h.numpy(), logits.numpy()


@pytest.mark.parametrize("L", [1, 3])
def test_stack_model_matches_torch_transcription(stack_model, L):
    w, m = stack_model
    toks = synth.tokens(3, synth.STREAM_TOKENS, 12, STACK.vocab)
    _, hid, logits = oracle.prefill(m, toks, L, want_logits="all")
    ref_h, ref_l = _torch_forward(w, toks, L)
    assert np.allclose(hid, ref_h, rtol=1e-12, atol=1e-13)
    assert np.allclose(logits, ref_l, rtol=1e-11, atol=1e-13)


def _layer_major(w, toks, L):
    """The plausible mistake: each stack layer run L times before the next one."""
    spec = w.spec
    pos = np.arange(len(toks))
    h = _t_bf16(w.embed[toks])
    for b in range(spec.n_pre):
        h = _torch_block(w.blocks[b], h, pos, spec)
    for l in range(spec.n_loop):
        for _ in range(L):
            h = _torch_block(w.blocks[spec.n_pre + l], h, pos, spec)
    for b in range(spec.n_post):
        h = _torch_block(w.blocks[spec.n_pre + spec.n_loop + b], h, pos, spec)
    return h.numpy()


def test_stack_order_distinguishes_layer_major(stack_model):
    # the pin above would catch a layer-major oracle: at L = 3 the two orders differ
    w, m = stack_model
    toks = synth.tokens(3, synth.STREAM_TOKENS, 12, STACK.vocab)
    _, hid, _ = oracle.prefill(m, toks, 3, want_logits="none")
    wrong = _layer_major(w, toks, 3)
    assert np.linalg.norm(hid - wrong) / np.linalg.norm(hid) > 1e-3


def test_stack_slots_one_per_application(stack_model):
    # slot keys in pipeline order: pre blocks, (iteration, layer) iteration-major,
    # post blocks; all distinct
    _, m = stack_model
    seq = m.slots(3)
    assert [b for b, _ in seq] == [0, 1, 2, 3, 2, 3, 2, 3, 4]
    keys = [k for _, k in seq]
    assert keys == [("pre", 0), ("pre", 1), ("loop", 1, 0), ("loop", 1, 1), ("loop", 2, 0), ("loop", 2, 1),
                    ("loop", 3, 0), ("loop", 3, 1), ("post", 0)]
    assert len(set(keys)) == len(keys)


def test_stack_cached_decode_equals_uncached(stack_model):
    # a cached step at depth 3 over slots keyed by (iteration, layer) equals the
    # last row of the uncached forward of the extended sequence; sharing one slot
    # between the two layers of an iteration would break this
    w, m = stack_model
    toks = synth.tokens(3, synth.STREAM_TOKENS, 10, STACK.vocab)
    lane, _, _ = oracle.prefill(m, toks[:9], 3, want_logits="none")
    h1, lg1, _, _ = oracle.decode_step(m, lane, 3, token=int(toks[9]))
    ref_h, ref_l = _torch_forward(w, toks, 3)
    assert np.allclose(h1, ref_h[-1], rtol=1e-11, atol=1e-12)
    assert np.allclose(lg1, ref_l[-1], rtol=1e-10, atol=1e-12)
