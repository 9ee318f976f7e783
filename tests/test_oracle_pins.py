"""Pins of the CPU oracle against closed forms, invariants, brute force and
independent library routines (torch CPU ops).  None of these re-types the oracle's
own formulas: each compares against something the mathematics or another library
fixes.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


# ---------------------------------------------------------------------------
# RMSNorm: closed forms


def test_rmsnorm_hand_value():
    h = np.array([[3.0, 4.0]])
    out = oracle.rmsnorm(h, np.ones(2), 0.0)
    # mean square 12.5 -> divide by sqrt(12.5)
    assert np.allclose(out, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=0, atol=1e-15)
    out = oracle.rmsnorm(h, np.array([2.0, -1.0]), 0.0)
    assert np.allclose(out, [[6 / math.sqrt(12.5), -4 / math.sqrt(12.5)]], rtol=0, atol=1e-15)


def test_rmsnorm_rms_identity():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((7, 33)) * 0.01
    eps = 1e-5
    out = oracle.rmsnorm(h, np.ones(33), eps)
    ms = np.mean(h * h, axis=1)
    rms_out = np.sqrt(np.mean(out * out, axis=1))
    assert np.allclose(rms_out, np.sqrt(ms / (ms + eps)), rtol=1e-13)
    ref = F.rms_norm(torch.from_numpy(h), (33,), torch.ones(33, dtype=torch.float64), eps).numpy()
    assert np.allclose(out, ref, rtol=1e-13, atol=0)


# ---------------------------------------------------------------------------
# RoPE: textbook rotations and invariants


def test_rope_dh2_is_plane_rotation():
    # head_dim 2: theta_0 = base^0 = 1, so position p rotates (x, y) by p radians
    x = np.array([[[0.3, -1.2]]] * 4)              # [T=4, H=1, 2]
    pos = np.arange(4)
    c, s = oracle.rope_angles(pos, 2, 10000.0)
    out = oracle.apply_rope(x, c, s)
    for p in range(4):
        R = np.array([[math.cos(p), -math.sin(p)], [math.sin(p), math.cos(p)]])
        assert np.allclose(out[p, 0], R @ x[p, 0], atol=1e-15)


def test_rope_dh4_frequencies():
    # head_dim 4, base 10000: pairs (0,2) turn at 1 rad/pos, (1,3) at 10000^(-1/2) = 0.01 rad/pos
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    p = 5
    c, s = oracle.rope_angles(np.array([p]), 4, 10000.0)
    out = oracle.apply_rope(x, c, s)[0, 0]
    a0, a1 = 5.0, 0.05
    assert np.allclose(out[[0, 2]], [1 * math.cos(a0) - 3 * math.sin(a0), 3 * math.cos(a0) + 1 * math.sin(a0)])
    assert np.allclose(out[[1, 3]], [2 * math.cos(a1) - 4 * math.sin(a1), 4 * math.cos(a1) + 2 * math.sin(a1)])


def test_rope_invariants():
    rng = np.random.default_rng(2)
    dh = 16
    q = rng.standard_normal((1, 3, dh))
    k = rng.standard_normal((1, 3, dh))
    c0, s0 = oracle.rope_angles(np.array([0]), dh, 10000.0)
    assert np.array_equal(oracle.apply_rope(q, c0, s0), q)          # identity at p = 0
    for p in (1, 7, 300):
        c, s = oracle.rope_angles(np.array([p]), dh, 10000.0)
        r = oracle.apply_rope(q, c, s)
        assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-14)
    # scores depend only on the position difference
    def score(pq, pk, shift):
        cq, sq = oracle.rope_angles(np.array([pq + shift]), dh, 10000.0)
        ck, sk = oracle.rope_angles(np.array([pk + shift]), dh, 10000.0)
        return np.sum(oracle.apply_rope(q, cq, sq) * oracle.apply_rope(k, ck, sk), axis=-1)
    assert np.allclose(score(9, 4, 0), score(9, 4, 123), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# attention: torch's SDPA (an independent library routine) and special cases


def _sdpa(q, k, v, mask):
    # q [T,H,dh] -> [H,T,dh]
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask))
    return o.numpy().transpose(1, 0, 2).reshape(q.shape[0], -1)


def test_attention_matches_sdpa_causal_and_with_past():
    rng = np.random.default_rng(3)
    T, H, dh, past = 9, 3, 8, 5
    q = rng.standard_normal((T, H, dh))
    k = rng.standard_normal((past + T, H, dh))
    v = rng.standard_normal((past + T, H, dh))
    pos = np.arange(past, past + T)
    out = oracle.causal_attention(q, k, v, pos)
    allowed = np.arange(past + T)[None, :] <= pos[:, None]
    assert np.allclose(out, _sdpa(q, k, v, allowed), rtol=1e-12, atol=1e-13)
    # no past: standard causal mask
    out0 = oracle.causal_attention(q, k[:T], v[:T], np.arange(T))
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    tk = torch.from_numpy(np.ascontiguousarray(k[:T].transpose(1, 0, 2)))
    tv = torch.from_numpy(np.ascontiguousarray(v[:T].transpose(1, 0, 2)))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy().transpose(1, 0, 2).reshape(T, -1)
    assert np.allclose(out0, ref, rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(4)
    H, dh = 2, 4
    v = rng.standard_normal((6, H, dh))
    k = rng.standard_normal((6, H, dh))
    # a single key: output is that value exactly
    q = rng.standard_normal((1, H, dh))
    assert np.array_equal(oracle.causal_attention(q, k[:1], v[:1], np.array([0])), v[0].reshape(1, -1))
    # zero query: uniform weights -> running means of the values
    out = oracle.causal_attention(np.zeros((6, H, dh)), k, v, np.arange(6))
    means = np.cumsum(v, axis=0) / np.arange(1, 7)[:, None, None]
    assert np.allclose(out, means.reshape(6, -1), rtol=1e-14)


# ---------------------------------------------------------------------------
# INT4: definitions, fixtures and exhaustive checks


def _read_lines(path):
    with open(path) as f:
        return [ln.split("#")[0].strip() for ln in f if ln.split("#")[0].strip()]


def test_nibble_table_matches_golden(golden_dir):
    rows = _read_lines(os.path.join(golden_dir, "int4_nibbles.txt"))
    table = {int(a, 16): int(b) for a, b in (r.split() for r in rows)}
    assert len(table) == 16
    for byte in range(256):
        got = oracle.unpack_nibbles(np.array([[byte]], dtype=np.uint8))[0]
        assert got[0] == table[byte & 0xF] and got[1] == table[byte >> 4]


def test_pack_example_matches_golden(golden_dir):
    rows = _read_lines(os.path.join(golden_dir, "int4_pack_example.txt"))
    q = np.array([[int(t) for t in rows[0].split()]], dtype=np.int8)
    want = np.array([[int(t, 16) for t in rows[1].split()]], dtype=np.uint8)
    assert np.array_equal(oracle.pack_nibbles(q), want)
    assert np.array_equal(oracle.unpack_nibbles(want), q)


def test_pack_unpack_exhaustive_pairs():
    vals = np.arange(-8, 8, dtype=np.int8)
    a, b = np.meshgrid(vals, vals, indexing="ij")
    q = np.stack([a.ravel(), b.ravel()], axis=1).reshape(1, -1)
    assert np.array_equal(oracle.unpack_nibbles(oracle.pack_nibbles(q)), q)


def test_dequant_exact_for_all_nibbles_and_all_finite_fp16_scales():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = bits.view(np.float16)
    s = s[np.isfinite(s)]                                     # 63,488 finite scales
    assert s.size == 63488
    q = np.arange(-8, 8, dtype=np.int8)
    # one row per nibble value, one group per scale
    Q = np.repeat(q[:, None], s.size * 128, axis=1)[:, ::128].repeat(128, axis=1)
    S = np.broadcast_to(s[None, :], (16, s.size))
    w = oracle.dequant_w4g128(Q, S)
    exact = q.astype(np.float64)[:, None] * s.astype(np.float64)[None, :]
    assert np.array_equal(w[:, ::128].astype(np.float64), exact)


def test_quantizer_hand_example(golden_dir):
    rows = _read_lines(os.path.join(golden_dir, "int4_quant_example.txt"))
    scale_bits = int(rows[0].split()[1], 16)
    w = np.zeros((1, 128), np.float32)
    want = np.zeros(128, np.int8)
    for r in rows[1:]:
        i, x, qq = r.split()
        w[0, int(i)] = np.float32(float(x))
        want[int(i)] = int(qq)
    q, s = oracle.quantize_w4g128(w)
    assert s.view(np.uint16)[0, 0] == scale_bits
    assert np.array_equal(q[0], want)


def test_quantizer_properties():
    w = synth.normal(7, 99, (64, 512), 0.02)
    w[3, :128] = 0.0                                        # an all-zero group
    q, s = oracle.quantize_w4g128(w)
    assert q.min() >= -7 and q.max() <= 7
    assert np.all(q[3, :128] == 0) and s[3, 0] == 0
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(w.astype(np.float64) - q * sf)
    # rounding to the nearest level: error at most half a step (plus fp32 division slack)
    assert np.all(err <= sf * 0.5 * (1 + 1e-6) + 1e-12)
    # the largest-magnitude element of every non-zero group lands on +-7
    g = np.abs(q.reshape(64, 4, 128)).max(axis=2)
    assert np.all(g[s > 0] == 7)


# ---------------------------------------------------------------------------
# argmax, depth clamp and active lists: brute force


def test_argmax_ties_lowest_index():
    x = np.array([[0.5, 2.0, 2.0, -1.0], [3.0, 3.0, 3.0, 3.0], [-5.0, -4.0, -4.5, -4.0]])
    assert list(oracle.greedy_argmax(x)) == [1, 0, 1]
    rng = np.random.default_rng(5)
    y = rng.integers(0, 4, size=(50, 33)).astype(np.float32)
    for r in range(50):
        best = max(y[r])
        assert oracle.greedy_argmax(y[r]) == min(i for i in range(33) if y[r, i] == best)


def test_clamp_depths_brute_force():
    rng = np.random.default_rng(6)
    for _ in range(20):
        req = rng.integers(1, 33, size=40)
        L0 = int(rng.integers(1, 33))
        out = oracle.clamp_depths(req, L0)
        for i in range(40):
            assert out[i] == min([L0] + list(req[: i + 1]))
        assert np.all(np.diff(out) <= 0)


def test_active_lists_brute_force():
    rng = np.random.default_rng(7)
    d = rng.choice([2, 4, 8, 16, 32], size=64)
    lists = oracle.active_lists(d)
    assert len(lists) == 32
    for j, act in enumerate(lists, start=1):
        assert list(act) == [r for r in range(64) if d[r] >= j]
        assert len(act) == int(np.sum(d >= j))


# ---------------------------------------------------------------------------
# whole-model properties on the tiny fp32 model


@pytest.fixture(scope="module")
def tiny():
    spec = synth.SPECS[1]
    w = synth.make_weights(spec, seed=0)
    return w, oracle.OracleModel.from_weights(w)


def _torch_block(Wb, h, pos, spec):
    """Independent transcription with torch CPU routines: F.rms_norm, F.linear,
    complex-number rotation for RoPE, F.scaled_dot_product_attention, F.silu."""
    d, H, dh = spec.d_model, spec.n_heads, spec.head_dim
    T = h.shape[0]
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x = F.rms_norm(h, (d,), t(Wb["norm1"]), spec.rms_eps)
    qkv = F.linear(x, t(Wb["wqkv"]))
    q, k, v = qkv.split(d, dim=1)
    half = dh // 2
    inv = spec.rope_base ** (-torch.arange(half, dtype=torch.float64) * 2 / dh)
    rot = torch.polar(torch.ones(T, half, dtype=torch.float64), torch.outer(t(pos), inv))

    def rope(z):
        z = z.reshape(T, H, dh)
        c = torch.complex(z[..., :half], z[..., half:]) * rot[:, None, :]
        return torch.cat([c.real, c.imag], dim=-1)

    q, k, v = rope(q).transpose(0, 1), rope(k).transpose(0, 1), v.reshape(T, H, dh).transpose(0, 1)
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1).reshape(T, d)
    h = h + F.linear(o, t(Wb["wo"]))
    x2 = F.rms_norm(h, (d,), t(Wb["norm2"]), spec.rms_eps)
    return h + F.linear(F.silu(F.linear(x2, t(Wb["wgate"]))) * F.linear(x2, t(Wb["wup"])), t(Wb["wdown"]))


@pytest.mark.parametrize("L", [1, 3])
def test_model_matches_torch_transcription(tiny, L):
    w, m = tiny
    spec = w.spec
    toks = synth.tokens(0, synth.STREAM_TOKENS, 16, spec.vocab)
    lane, hid, logits = oracle.prefill(m, toks, L, want_logits="all")
    h = torch.from_numpy(w.embed[toks].astype(np.float64))
    pos = np.arange(16)
    h = _torch_block(w.blocks[0], h, pos, spec)
    for _ in range(L):
        h = _torch_block(w.blocks[1], h, pos, spec)
    ref_logits = F.linear(F.rms_norm(h, (spec.d_model,), torch.ones(spec.d_model, dtype=torch.float64),
                                     spec.rms_eps), torch.from_numpy(w.head.astype(np.float64)))
    assert np.allclose(hid, h.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(logits, ref_logits.numpy(), rtol=1e-11, atol=1e-13)


def test_loop_equals_unrolled_stack(tiny):
    """L iterations of the shared block == L explicit applications of copies of it."""
    w, m = tiny
    toks = synth.tokens(0, synth.STREAM_TOKENS, 16, 256)
    _, h_loop, _ = oracle.prefill(m, toks, 4, want_logits="none")
    import copy
    spec2 = copy.copy(w.spec)
    spec2.n_loop = 4
    m2 = copy.copy(m)
    m2.spec = spec2
    m2.blocks = [m.blocks[0]] + [m.blocks[1]] * 4
    _, h_unrolled, _ = oracle.prefill(m2, toks, 1, want_logits="none")
    assert np.array_equal(h_loop, h_unrolled)


def test_causality(tiny):
    w, m = tiny
    toks = synth.tokens(0, synth.STREAM_TOKENS, 16, 256)
    _, h0, _ = oracle.prefill(m, toks, 3, want_logits="none")
    for p in (5, 11):
        t2 = toks.copy()
        t2[p] = (t2[p] + 17) % 256
        t2[-1] = (t2[-1] + 3) % 256
        _, h1, _ = oracle.prefill(m, t2, 3, want_logits="none")
        assert np.allclose(h1[:p], h0[:p], rtol=0, atol=1e-14)
        assert not np.allclose(h1[p], h0[p])


def test_mixed_batch_equals_each_lane_alone(tiny):
    w, m = tiny
    rng = np.random.default_rng(8)
    seqs = [synth.tokens(0, 3000 + i, n, 256) for i, n in enumerate([5, 9, 3, 12])]
    Ls = [4, 1, 7, 2]
    h, logits, lists = oracle.forward_batch(m, seqs, Ls)
    off = 0
    for i, s in enumerate(seqs):
        _, hi, li = oracle.prefill(m, s, Ls[i])
        assert np.allclose(h[off:off + len(s)], hi, rtol=1e-13, atol=1e-14)
        assert np.allclose(logits[i], li, rtol=1e-12, atol=1e-13)
        off += len(s)
    assert len(lists) == 7


def test_cached_decode_equals_uncached_forward(tiny):
    """The cached path agrees with re-running the whole extended sequence."""
    w, m = tiny
    toks = list(synth.tokens(0, synth.STREAM_TOKENS, 16, 256))
    lane, _, _ = oracle.prefill(m, toks, 4)
    seq = list(toks)
    for step in range(5):
        tok = lane.pending
        h, logits, nxt, L = oracle.decode_step(m, lane, 4)
        seq.append(tok)
        _, h_full, lg_full = oracle.prefill(m, seq, 4, want_logits="last")
        assert L == 4
        assert np.allclose(h, h_full[-1], rtol=1e-11, atol=1e-13)
        assert np.allclose(logits, lg_full, rtol=1e-10, atol=1e-12)
        assert nxt == oracle.greedy_argmax(lg_full)


def test_monotone_depth_cached_equals_ragged(tiny):
    w, m = tiny
    toks = list(synth.tokens(0, synth.STREAM_TOKENS, 16, 256))
    L1 = 6
    req = [9, 5, 5, 7, 3, 4, 1, 2]
    deps = oracle.clamp_depths(req, L1)
    lane, _, _ = oracle.prefill(m, toks, L1)
    seq = list(toks)
    hs = []
    for r in req:
        seq.append(lane.pending)
        h, _, _, L = oracle.decode_step(m, lane, r)
        hs.append(h)
    assert list(deps) == [6, 5, 5, 5, 3, 3, 1, 1]
    h_rag, lg = oracle.forward_ragged(m, seq, [L1] * 16 + list(deps))
    assert np.allclose(np.array(hs), h_rag[16:], rtol=1e-11, atol=1e-13)


def test_fp32_vs_fp64_conditioning_tiny(tiny):
    """Intrinsic sensitivity of the synthetic model: the oracle in fp32 vs fp64."""
    w, m64 = tiny
    m32 = oracle.OracleModel.from_weights(w, dt=np.float32)
    toks = synth.tokens(0, synth.STREAM_TOKENS, 16, 256)
    for L in (4, 32):
        _, h64, _ = oracle.prefill(m64, toks, L, want_logits="none")
        _, h32, _ = oracle.prefill(m32, toks, L, want_logits="none")
        rel = np.linalg.norm(h32 - h64) / np.linalg.norm(h64)
        assert rel < 1e-5, (L, rel)


@pytest.mark.slow
def test_fp32_vs_fp64_conditioning_int4_model():
    """Same check on the 2048-wide INT4-loop model at L = 8 and 32 (32 tokens)."""
    spec = synth.SPECS[2]
    w = synth.make_weights(spec, 0)
    m64 = oracle.OracleModel.from_weights(w)
    m32 = oracle.OracleModel.from_weights(w, dt=np.float32)
    toks = synth.tokens(0, synth.STREAM_TOKENS, 32, spec.vocab)
    for L in (8, 32):
        _, h64, _ = oracle.prefill(m64, toks, L, want_logits="none")
        _, h32, _ = oracle.prefill(m32, toks, L, want_logits="none")
        rel = np.linalg.norm(h32 - h64) / np.linalg.norm(h64)
        assert rel < 1e-4, (L, rel)


# ---------------------------------------------------------------------------
# early exit ([CLI] "generate": --early-exit-* options)


def test_ee_relative_delta_and_margin_hand_values():
    # ||(0, 0, 12)|| / ||(3, 4, 12)|| = 12 / 13
    assert abs(oracle.relative_delta(np.array([3.0, 4.0, 0.0]), np.array([3.0, 4.0, 12.0])) - 12.0 / 13.0) < 1e-15
    assert oracle.logit_margin(np.array([0.5, 2.0, -1.0])) == 1.5
    assert oracle.logit_margin(np.array([1.0, 5.0, 2.0, 5.0])) == 0.0   # tied top-1


def test_ee_probe_schedule_brute_force():
    ee = oracle.EarlyExit(patience=1, min_L=3, peek_every=2)
    assert [j for j in range(1, 11) if oracle.probe_iteration(ee, j, 10)] == [3, 5, 7, 9]
    assert [j for j in range(1, 10) if oracle.probe_iteration(ee, j, 9)] == [3, 5, 7]   # never at j = L
    assert not any(oracle.probe_iteration(oracle.EarlyExit(patience=0), j, 10) for j in range(1, 11))


def _tiny_lane(seed=11, plen=9, L=6):
    spec = synth.SPECS[1]
    w = synth.make_weights(spec, seed)
    m = oracle.OracleModel.from_weights(w)
    toks = synth.tokens(seed, 77, plen, spec.vocab)
    return m, (lambda: oracle.prefill(m, toks, L)[0])


def _same_lane(a, b):
    assert a.tokens == b.tokens and a.ceiling == b.ceiling and a.pending == b.pending
    assert set(a.kv) == set(b.kv)
    for k in a.kv:
        assert np.array_equal(a.kv[k][0], b.kv[k][0]) and np.array_equal(a.kv[k][1], b.kv[k][1])


def test_ee_disabled_equals_plain_decode():
    m, fresh = _tiny_lane()
    a, b = fresh(), fresh()
    for t, L in enumerate([6, 5, 6, 3]):
        ha, la, na, Ea = oracle.decode_step(m, a, L)
        hb, lb, nb, Eb = oracle.decode_step_ee(m, b, L, oracle.EarlyExit(patience=0, tau=1e9))
        assert np.array_equal(ha, hb) and np.array_equal(la, lb) and na == nb and Ea == Eb
        _same_lane(a, b)


@pytest.mark.parametrize("patience,min_L,peek,exit_at", [(1, 2, 1, 2), (2, 2, 1, 3), (2, 2, 2, 4), (1, 5, 1, 5)])
def test_ee_always_stable_equals_decode_at_exit_depth(patience, min_L, peek, exit_at):
    """tau = inf: every probe is stable, so the loop stops at the patience-th probe,
    which must equal plain cached decode requested at that depth."""
    m, fresh = _tiny_lane()
    a, b = fresh(), fresh()
    ee = oracle.EarlyExit(patience=patience, min_L=min_L, tau=np.inf, peek_every=peek)
    hb, lb, nb, Eb = oracle.decode_step_ee(m, b, 6, ee)
    ha, la, na, Ea = oracle.decode_step(m, a, exit_at)
    assert Eb == exit_at == Ea
    assert np.array_equal(ha, hb) and np.array_equal(la, lb) and na == nb
    _same_lane(a, b)
    # the lowered ceiling holds for the next token
    hb2, _, _, Eb2 = oracle.decode_step_ee(m, b, 6, oracle.EarlyExit(patience=0))
    ha2, _, _, Ea2 = oracle.decode_step(m, a, 6)
    assert Eb2 == Ea2 == exit_at and np.array_equal(ha2, hb2)


def test_ee_never_stable_runs_full_depth():
    m, fresh = _tiny_lane()
    a, b = fresh(), fresh()
    hb, _, _, Eb = oracle.decode_step_ee(m, b, 6, oracle.EarlyExit(patience=1, min_L=1, tau=0.0))
    ha, _, _, Ea = oracle.decode_step(m, a, 6)
    assert Eb == Ea == 6 and np.array_equal(ha, hb)
    hb, _, _, Eb = oracle.decode_step_ee(m, b, 6, oracle.EarlyExit(patience=1, min_L=1, logit_margin=1e300))
    ha, _, _, Ea = oracle.decode_step(m, a, 6)
    assert Eb == Ea == 6 and np.array_equal(ha, hb)


def test_ee_logit_rule_tiny_margin_exits_at_first_probe():
    m, fresh = _tiny_lane()
    a, b = fresh(), fresh()
    hb, lb, _, Eb = oracle.decode_step_ee(m, b, 6, oracle.EarlyExit(patience=1, min_L=3, logit_margin=1e-300))
    ha, la, _, Ea = oracle.decode_step(m, a, 3)
    assert Eb == Ea == 3 and np.array_equal(ha, hb) and np.array_equal(la, lb)


def test_ee_streak_resets_on_unstable_probe(monkeypatch):
    """Scripted probe outcomes: stable, unstable, stable, stable with patience 2 ->
    the loop ends at the fourth probe, not the second."""
    m, fresh = _tiny_lane(L=8)
    script = iter([0.0, 1.0, 0.0, 0.0, 0.0, 0.0])
    monkeypatch.setattr(oracle.model, "relative_delta", lambda hp, h: next(script))
    b = fresh()
    _, _, _, E = oracle.decode_step_ee(m, b, 8, oracle.EarlyExit(patience=2, min_L=2, tau=0.5))
    assert E == 5   # probes at 2 (stable), 3 (unstable), 4, 5 (stable, stable)


# ---------------------------------------------------------------------------
# shared-prefix reuse: appending to a cache and forking a prefix


def _kv_close(a, b, tol=1e-12):
    assert set(a.kv) == set(b.kv)
    for key in a.kv:
        for x, y in zip(a.kv[key], b.kv[key]):
            assert x.shape == y.shape, key
            assert np.allclose(x, y, rtol=tol, atol=tol), key


@pytest.mark.parametrize("cuts", [[7], [3, 9, 10]])
def test_append_equals_prefill_of_concatenation(tiny, cuts):
    """Cached chunks (any split of the prompt) == one uncached prefill of it."""
    w, m = tiny
    toks = synth.tokens(0, synth.STREAM_TOKENS, 16, 256)
    full, h_full, lg_full = oracle.prefill(m, toks, 4, want_logits="all")
    edges = [0] + cuts + [16]
    lane, h0, _ = oracle.prefill(m, toks[:edges[1]], 4, want_logits="none")
    hs = [h0]
    for a, b in zip(edges[1:-1], edges[2:]):
        h, lg = oracle.append(m, lane, toks[a:b], 4, want_logits="all")
        hs.append(h)
        assert np.allclose(lg, lg_full[a:b], rtol=1e-10, atol=1e-12)
    assert np.allclose(np.concatenate(hs), h_full, rtol=1e-11, atol=1e-13)
    _kv_close(lane, full)
    assert lane.pending == full.pending and lane.tokens == full.tokens and lane.ceiling == 4


def test_append_equals_teacher_forced_decode_steps(tiny):
    """T tokens appended at once == T single-token cached steps (multi-row causal
    masking against the one-row path), including a clamped depth."""
    w, m = tiny
    toks = synth.tokens(0, synth.STREAM_TOKENS, 12, 256)
    new = synth.tokens(0, 3100, 5, 256)
    a = oracle.prefill(m, toks, 5)[0]
    b = oracle.prefill(m, toks, 5)[0]
    h, lg = oracle.append(m, a, new, 7, want_logits="all")   # requested 7 > ceiling 5 -> 5
    assert a.ceiling == 5
    for t, tok in enumerate(new):
        hb, lb, nb, Lb = oracle.decode_step(m, b, 7, token=int(tok))
        assert Lb == 5
        assert np.allclose(h[t], hb, rtol=1e-11, atol=1e-13)
        assert np.allclose(lg[t], lb, rtol=1e-10, atol=1e-12)
    _kv_close(a, b)
    assert a.pending == b.pending
    h2, _ = oracle.append(m, a, new[:2], 3, want_logits="none")   # lower depth: ceiling drops
    assert a.ceiling == 3
    for t in range(2):
        hb, _, _, Lb = oracle.decode_step(m, b, 3, token=int(new[t]))
        assert Lb == 3 and np.allclose(h2[t], hb, rtol=1e-11, atol=1e-13)


def test_fork_then_append_equals_full_prefill(tiny):
    """A request built from a forked prefix == the same request prefilled alone
    (the shared and uncached modes must agree), and the source is left intact."""
    w, m = tiny
    prefix = synth.tokens(0, synth.STREAM_TOKENS, 10, 256)
    src = oracle.prefill(m, prefix, 4)[0]
    ref_src = oracle.prefill(m, prefix, 4)[0]
    for P, seed in [(10, 3200), (6, 3201), (1, 3202)]:
        suffix = synth.tokens(0, seed, 4, 256)
        child = oracle.fork(src, P)
        assert child.ceiling == 4 and child.tokens == list(map(int, prefix[:P]))
        assert child.pending == (src.pending if P == 10 else -1)
        h, lg = oracle.append(m, child, suffix, 4)
        want, h_want, lg_want = oracle.prefill(m, np.concatenate([prefix[:P], suffix]), 4)
        assert np.allclose(h, h_want[P:], rtol=1e-11, atol=1e-13)
        assert np.allclose(lg, lg_want, rtol=1e-10, atol=1e-12)
        _kv_close(child, want)
        assert child.pending == want.pending
        for _ in range(2):
            hc, _, nc, _ = oracle.decode_step(m, child, 4)
            hw, _, nw, _ = oracle.decode_step(m, want, 4)
            assert np.allclose(hc, hw, rtol=1e-11, atol=1e-13) and nc == nw
    _kv_close(src, ref_src, tol=0.0)
    assert src.tokens == ref_src.tokens and src.pending == ref_src.pending


# ---------------------------------------------------------------------------
# self-speculative decoding: the output is greedy decoding at the verify depth


def _plain_greedy(m, lane, L, n):
    out = []
    for _ in range(n):
        out.append(oracle.decode_step(m, lane, L)[2])
    return out


@pytest.mark.parametrize("Ld,k", [(2, 4), (4, 3), (6, 1), (1, 5)])
def test_speculative_equals_greedy_at_verify_depth(tiny, Ld, k):
    w, m = tiny
    toks = synth.tokens(0, 3300, 11, 256)
    a = oracle.prefill(m, toks, 8)[0]
    b = oracle.prefill(m, toks, 8)[0]
    got, acc = oracle.speculative_decode(m, a, Ld, 8, k, 17)
    want = _plain_greedy(m, b, 8, 17)
    assert got == want
    assert sum(x + 1 for x in acc) == 17 and all(0 <= x <= k for x in acc)
    assert a.tokens == b.tokens and a.pending == b.pending and a.ceiling == b.ceiling == 8
    for key in b.kv:
        if key[0] == "loop" and key[1] > 8:
            continue
        for x, y in zip(a.kv[key], b.kv[key]):
            assert x.shape == y.shape and np.allclose(x, y, rtol=1e-11, atol=1e-13), key


def test_speculative_equal_depths_accepts_every_draft(tiny):
    w, m = tiny
    toks = synth.tokens(0, 3301, 9, 256)
    lane = oracle.prefill(m, toks, 5)[0]
    got, acc = oracle.speculative_decode(m, lane, 5, 5, 3, 14)
    assert acc == [3, 3, 3, 1]                    # 4 + 4 + 4 + 2 tokens, the last round capped
    assert got == _plain_greedy(m, oracle.prefill(m, toks, 5)[0], 5, 14)


def test_speculative_without_drafts_is_plain_decode(tiny):
    w, m = tiny
    toks = synth.tokens(0, 3302, 7, 256)
    got, acc = oracle.speculative_decode(m, oracle.prefill(m, toks, 6)[0], 2, 6, 0, 6)
    assert acc == [0] * 6 and got == _plain_greedy(m, oracle.prefill(m, toks, 6)[0], 6, 6)


def test_speculative_wrong_drafts_change_nothing(tiny, monkeypatch):
    """A planted draft that always proposes a wrong token: nothing is accepted and
    the output is still greedy decoding at the verify depth."""
    w, m = tiny
    toks = synth.tokens(0, 3303, 10, 256)
    want = _plain_greedy(m, oracle.prefill(m, toks, 7)[0], 7, 9)
    real = oracle.model.decode_step
    lane = oracle.prefill(m, toks, 7)[0]
    seen = {"n": 0}

    def bad(m_, lane_, L, token=None):
        h, lg, nxt, Le = real(m_, lane_, L, token=token)
        seen["n"] += 1
        p = len(lane_.tokens)                      # position of the next token
        return h, lg, (want[min(p - 10, 8)] + 1) % 256, Le

    monkeypatch.setattr(oracle.model, "decode_step", bad)
    got, acc = oracle.speculative_decode(m, lane, 3, 7, 2, 9)
    monkeypatch.undo()
    assert seen["n"] > 0 and got == want and acc == [0] * 9


# ---------------------------------------------------------------------------
# store-h cache modes (iteration-axis KV compression)


def test_store_h_bytes_match_the_pages(golden_dir):
    for row in _read_lines(os.path.join(golden_dir, "store_h_bytes.txt")):
        mode, d, H, nbytes = row.split()
        assert oracle.h_bytes_per_position(int(d), int(H), mode) == int(nbytes), mode


def test_round_to_operand_against_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 4, 4000),
                        [0.0, -0.0, 1.0, 65504.0, 1e-8, 3.0e38]])
    t = torch.from_numpy(x.astype(np.float32))
    assert np.array_equal(oracle.round_to_operand(x, "bf16"), t.to(torch.bfloat16).to(torch.float64).numpy())
    small = x[np.abs(x) < 6e4]
    ts = torch.from_numpy(small.astype(np.float32))
    assert np.array_equal(oracle.round_to_operand(small, "f16"), ts.to(torch.float16).to(torch.float64).numpy())


def test_quantize_h_hand_example_and_bounds():
    # one row, two heads of 4: head 0 max 2.54 -> s = fp16(0.02) , head 1 all zero
    x = np.array([[2.54, -1.27, 0.01, 0.03, 0.0, 0.0, 0.0, 0.0]], np.float32)
    q, s = oracle.quantize_h(x, 2, 127)
    s0 = np.float32(np.float16(np.float32(2.54) / np.float32(127)))
    assert s[0, 0] == np.float16(s0) and s[0, 1] == 0
    assert q[0, :4].tolist() == [int(np.rint(np.float32(v) / s0)) for v in x[0, :4]]
    assert q[0, 4:].tolist() == [0, 0, 0, 0]
    # ties go to even: x / s = 2.5 and 3.5 exactly (s a power of two)
    xt = np.array([[0.625, 0.875, 31.75, -31.75]], np.float32)     # max 31.75 -> s = 0.25
    qt, st = oracle.quantize_h(xt, 1, 127)
    assert float(st[0, 0]) == 0.25 and qt[0].tolist() == [2, 4, 127, -127]
    rng = np.random.default_rng(9)
    for levels in (127, 7):
        xr = (rng.standard_normal((64, 96)) * rng.uniform(0.01, 3, (64, 1))).astype(np.float32)
        q, s = oracle.quantize_h(xr, 3, levels)
        back = oracle.dequant_h(q, s)
        s_el = np.repeat(s.astype(np.float64), 32, axis=1)
        assert np.all(np.abs(back - xr) <= 0.5 * s_el * (1 + 1e-3) + 1e-12)
        assert np.all(np.abs(q).reshape(64, 3, 32).max(axis=-1) == levels)


@pytest.mark.parametrize("mode", ["h", "h8", "h4"])
def test_store_h_identity_store_equals_kv_mode(tiny, mode, monkeypatch):
    """With a store that keeps x unchanged, rebuilding K/V from the slot's rows
    reproduces the K/V cache mode (positions and projection of the rebuild)."""
    import copy
    w, m = tiny
    mh = copy.copy(m)
    mh.kv_mode = mode
    monkeypatch.setattr(oracle.model, "h_store", lambda x, act, H, md: np.array(x, dtype=np.float64))
    toks = synth.tokens(0, 3400, 12, 256)
    a, ha, la = oracle.prefill(m, toks, 4, want_logits="all")
    b, hb, lb = oracle.prefill(mh, toks, 4, want_logits="all")
    assert np.allclose(ha, hb, rtol=1e-11, atol=1e-13) and np.allclose(la, lb, rtol=1e-10, atol=1e-12)
    for _ in range(3):
        xa = oracle.decode_step(m, a, 4)
        xb = oracle.decode_step(mh, b, 4)
        assert np.allclose(xa[0], xb[0], rtol=1e-11, atol=1e-13) and xa[2] == xb[2]


@pytest.mark.parametrize("mode", ["h", "h8", "h4"])
def test_store_h_cached_equals_uncached(mode):
    """Compression is per position, so cached decode == a prefill of the extended
    sequence in the same mode (bf16 model: operand rounding and both code widths)."""
    import copy
    spec = synth.ModelSpec("tiny-bf16", 320, 192, 2, 96, 384, 1, 1, 1, "bf16", "bf16")
    w = synth.make_weights(spec, 4)
    m = copy.copy(oracle.OracleModel.from_weights(w))
    m.kv_mode = mode
    toks = list(synth.tokens(0, 3401, 10, 320))
    lane, _, _ = oracle.prefill(m, toks, 3)
    seq = list(toks)
    for _ in range(3):
        seq.append(lane.pending)
        h, logits, _, _ = oracle.decode_step(m, lane, 3)
        _, h_full, lg_full = oracle.prefill(m, seq, 3, want_logits="last")
        assert np.allclose(h, h_full[-1], rtol=1e-10, atol=1e-12)
        assert np.allclose(logits, lg_full, rtol=1e-9, atol=1e-11)
    # and the compression is visible: the modes differ from each other and from K/V
    m_kv = oracle.OracleModel.from_weights(w)
    _, h_kv, _ = oracle.prefill(m_kv, toks, 3)
    _, h_m, _ = oracle.prefill(m, toks, 3)
    err = np.linalg.norm(h_m - h_kv) / np.linalg.norm(h_kv)
    assert 1e-7 < err < {"h": 5e-3, "h8": 2e-2, "h4": 2e-1}[mode], err


# ---------------------------------------------------------------------------
# delta-KV along the iteration axis


def _bf16_model(mode, seed=4):
    import copy
    spec = synth.ModelSpec("tiny-bf16", 320, 192, 2, 96, 384, 1, 2, 1, "bf16", "bf16")
    w = synth.make_weights(spec, seed)
    m = copy.copy(oracle.OracleModel.from_weights(w))
    m.kv_mode = mode
    return w, m


def test_delta_exact_differences_equal_store_h(monkeypatch):
    """With differences kept exactly, the delta chain reproduces the operand-type
    store-h mode: the anchor, the chaining of each loop layer's slots and the
    rebuild are right."""
    w, md = _bf16_model("d8")
    _, mh = _bf16_model("h")
    monkeypatch.setattr(oracle.model, "delta_store",
                        lambda x, prev, act, H: oracle.round_to_operand(x, act))
    toks = list(synth.tokens(0, 3500, 9, 320))
    a, ha, _ = oracle.prefill(md, toks, 4)
    b, hb, _ = oracle.prefill(mh, toks, 4)
    assert np.array_equal(ha, hb)
    for _ in range(2):
        xa, xb = oracle.decode_step(md, a, 4), oracle.decode_step(mh, b, 4)
        assert np.array_equal(xa[0], xb[0]) and xa[2] == xb[2]


def test_delta_reconstruction_within_one_step(monkeypatch):
    """Each delta slot's reconstruction is within half a code step (plus fp32
    rounding) of its own x: errors do not add up along the iterations; the first
    iteration keeps x exactly in the operand type."""
    w, md = _bf16_model("d8")
    seen = []
    real = oracle.model.delta_store

    def rec(x, prev, act, H):
        out = real(x, prev, act, H)
        seen.append((oracle.round_to_operand(x, act), np.asarray(prev, np.float64), out, H))
        return out

    monkeypatch.setattr(oracle.model, "delta_store", rec)
    toks = list(synth.tokens(0, 3501, 11, 320))
    oracle.prefill(md, toks, 6)
    monkeypatch.undo()
    assert len(seen) == 2 * 5                      # 2 loop layers x iterations 2..6
    for x_op, prev, out, H in seen:
        T, d = x_op.shape
        diff = (x_op.astype(np.float32) - prev.astype(np.float32)).astype(np.float64)
        step = np.abs(diff).reshape(T, H, d // H).max(axis=-1) / 127.0
        tol = np.repeat(step, d // H, axis=1) * 0.5 * (1 + 2e-3) + np.abs(x_op) * 2.0 ** -22
        assert np.all(np.abs(out - x_op) <= tol)


def test_delta_cached_equals_uncached():
    w, md = _bf16_model("d8")
    toks = list(synth.tokens(0, 3502, 10, 320))
    lane, _, _ = oracle.prefill(md, toks, 3)
    seq = list(toks)
    for _ in range(3):
        seq.append(lane.pending)
        h, logits, _, _ = oracle.decode_step(md, lane, 3)
        _, h_full, lg_full = oracle.prefill(md, seq, 3, want_logits="last")
        assert np.allclose(h, h_full[-1], rtol=1e-10, atol=1e-12)
        assert np.allclose(logits, lg_full, rtol=1e-9, atol=1e-11)
    _, mk = _bf16_model("kv")
    _, h_kv, _ = oracle.prefill(mk, toks, 3)
    _, h_d, _ = oracle.prefill(md, toks, 3)
    err = np.linalg.norm(h_d - h_kv) / np.linalg.norm(h_kv)
    assert 1e-7 < err < 2e-2, err
