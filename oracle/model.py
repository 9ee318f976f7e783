"""Plain CPU oracle of the looped transformer's hot path (test infrastructure only).

Pages cited (titles as printed on each page):
  [DYN]  "Dynamic-L Inference" (tinyloop docs, architecture)
  [BENCH] "Benchmark Comparison" (tinyloop docs, measured benchmarks)
  [CLI]  "CLI Reference" (tinyloop docs, framework)
  [VSG]  "Benchmark Comparison" (tinyloop docs, vs generic runtimes)
  [CDB]  "Depth-adaptive Inference of Looped Language Models via Continuous Depth
         Batching" (summary page)

What is computed (where the pages leave a point open, the function that depends
on it states the reading it takes):
  * pipeline embed -> pre blocks -> shared loop block (stack) x L -> post blocks ->
    head, [VSG] "Where Generic Runtimes Lose On Looped Checkpoints";
  * L is a call argument, never part of the weights, [DYN] "The Core Idea";
  * pre-norm blocks, one K/V cache per block application ([CLI], environment
    variable table, TINYLOOP_KV_H_MODE: the norm output feeds attn_qkv and the
    runtime keeps per-layer K/V buffers);
  * cached decode is the default and must agree with the uncached path ([CLI]
    "Current Behavior" and "Debugging The Reference Path");
  * symmetric per-group min-max INT4 without calibration ([BENCH] section 7),
    groups of 128 along K ([BENCH] section 5, 16 groups at K = 2048), two's
    complement nibbles in [-7, 7], even element in the low nibble ([CLI],
    TINYLOOP_KV_INT4);
  * FP16 body = the INT4 body dequantised once to fp16 ([CLI],
    TINYLOOP_EXPERIMENTAL_FP16_BODY);
  * per-token depth is clamped so it never rises within a generation ([CLI]
    "generate", --early-exit-patience);
  * greedy decoding is temperature 0 ([CLI] "generate", --temperature);
  * lanes of a batch run at their own depth ([DYN] "L-Aware Batching"), tokens
    leave the batch after their last loop iteration ([CDB] summary bullets).

Parity pins (tests/test_oracle_*.py): every function here is pinned by a closed
form, an invariant, a brute force or an independent library routine; none is
"parity unpinned" except absolute output values of the synthetic models, for
which the pages print no numbers.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rmsnorm", "rope_angles", "apply_rope", "silu", "causal_attention",
    "quantize_w4g128", "pack_nibbles", "unpack_nibbles", "dequant_w4g128", "fp16_body",
    "OracleModel", "Lane", "prefill", "decode_step", "forward_batch", "forward_ragged",
    "greedy_argmax", "clamp_depths", "active_lists", "bf16_bits_to_float",
    "EarlyExit", "probe_iteration", "relative_delta", "logit_margin", "decode_step_ee",
    "append", "fork", "truncate", "speculative_decode",
    "H_MODES", "round_to_operand", "quantize_h", "dequant_h", "h_store", "delta_store", "h_bytes_per_position",
]


# ---------------------------------------------------------------------------
# elementary steps


def rmsnorm(h: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x = h / sqrt(mean(h^2) + eps) * g over the last axis.

    Placement before QKV and before the MLP: [CLI] TINYLOOP_KV_H_MODE names the
    "pre-QKV" norm output as the input of attn_qkv.
    """
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * g


def rope_angles(positions: np.ndarray, head_dim: int, base: float, dt=np.float64):
    """cos and sin of p * theta_i, theta_i = base^(-2i/head_dim), i < head_dim/2.

    Rotary position embedding with base 10000 (model definition of the workloads);
    the rotate-half pairing (i, i + head_dim/2) is a reading: the pages name RoPE
    but not its pairing.
    """
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(dt), np.sin(ang).astype(dt)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x: [T, H, dh]; rotate each pair (x_i, x_{i+dh/2}) by its angle at the row's position."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def causal_attention(q: np.ndarray, k_all: np.ndarray, v_all: np.ndarray, q_pos: np.ndarray) -> np.ndarray:
    """Softmax attention of queries at positions q_pos over keys 0..q_pos (inclusive).

    q: [T, H, dh]; k_all, v_all: [S, H, dh] hold positions 0..S-1 of one lane in one
    cache slot.  Scale 1/sqrt(dh), max subtraction, no bias, one K/V head per query
    head.  Returns [T, H*dh].
    """
    T, H, dh = q.shape
    S = k_all.shape[0]
    scores = np.einsum("thd,shd->hts", q, k_all) / math.sqrt(dh)
    mask = np.arange(S)[None, :] > np.asarray(q_pos)[:, None]          # [T, S]
    scores = np.where(mask[None, :, :], -np.inf, scores)
    scores = scores - scores.max(axis=-1, keepdims=True)
    p = np.exp(scores)
    p = p / p.sum(axis=-1, keepdims=True)
    o = np.einsum("hts,shd->thd", p, v_all)
    return o.reshape(T, H * dh)


# ---------------------------------------------------------------------------
# INT4 group quantisation ([BENCH] sections 5 and 7; [CLI] TINYLOOP_KV_INT4)

GROUP = 128


def quantize_w4g128(w32: np.ndarray):
    """Symmetric per-group min-max INT4 of fp32 weights [N, K], groups of 128 along K.

    s = fp16(max|w| / 7) with the division in fp32, q = clamp(rint(w / s), -7, 7)
    with round-half-to-even and the division in fp32; a group whose fp16 scale is 0
    gets q = 0.  The fp32 arithmetic is the precision in which the GPU library takes
    the same integer decisions.  Returns (q int8 [N, K], s float16 [N, K/128]).
    """
    w32 = np.asarray(w32, dtype=np.float32)
    N, K = w32.shape
    assert K % GROUP == 0
    g = w32.reshape(N, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s32 > 0, np.rint(g / np.where(s32 > 0, s32, np.float32(1))), np.float32(0))
    q = np.clip(r, -7, 7).astype(np.int8).reshape(N, K)
    return q, s16


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Two's complement nibbles, element 2i in the low nibble of byte i, 2i+1 in the high."""
    q = np.asarray(q, dtype=np.int8)
    lo = q[..., 0::2].astype(np.uint8) & 0xF
    hi = q[..., 1::2].astype(np.uint8) & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: every nibble n maps to n if n < 8 else n - 16."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = (packed & 0xF).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant_w4g128(q: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """w[n, k] = q[n, k] * s[n, k // 128]; exact in fp32 (a 4-bit integer times an fp16)."""
    N, K = q.shape
    s = np.repeat(s16.astype(np.float32), GROUP, axis=1)
    return q.astype(np.float32) * s


def fp16_body(q: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """FP16 body: fp16(q * s), the dequantised cache built once at load ([CLI] FP16_BODY)."""
    return dequant_w4g128(q, s16).astype(np.float16)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# iteration-axis KV compression: store-h ([CLI] environment variables
# TINYLOOP_KV_H_MODE, with TINYLOOP_KV_INT8 / TINYLOOP_KV_INT4; [BENCH] section 9)
#
# Instead of K and V, a cache slot keeps the block's pre-QKV norm output x (one
# row of d values per position); at attention time K and V of every cached
# position are rebuilt by the block's own QKV projection.  "h" keeps x in the
# operand type, "h8" / "h4" as symmetric codes in [-127, 127] / [-7, 7] with one
# fp16 scale per (position, head).

H_MODES = ("kv", "h", "h8", "h4", "d8")
H_LEVELS = {"h8": 127, "h4": 7}


def round_to_operand(x: np.ndarray, act: str) -> np.ndarray:
    """x rounded to the operand type (fp32 / fp16 / bf16 with round-to-nearest-even)."""
    x32 = np.asarray(x, dtype=np.float32)
    if act == "f16":
        return x32.astype(np.float16).astype(np.float64)
    if act == "bf16":
        b = x32.view(np.uint32).astype(np.uint64)
        b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
        return b.astype(np.uint32).view(np.float32).astype(np.float64)
    return x32.astype(np.float64)


def quantize_h(x_op: np.ndarray, n_heads: int, levels: int):
    """Symmetric codes of operand-type rows [T, d], one scale per (row, head).

    s = fp16(max|x| / levels) with the division in fp32; q = clamp(rint(x / s),
    -levels, levels) with round-half-to-even and the division in fp32; a head whose
    scale is 0 gets q = 0.  Returns (q int8 [T, d], s float16 [T, H]).
    """
    x = np.asarray(x_op, dtype=np.float32)
    T, d = x.shape
    xh = x.reshape(T, n_heads, d // n_heads)
    a = np.abs(xh).max(axis=-1)
    sc = (a / np.float32(levels)).astype(np.float16)
    s32 = sc.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s32 > 0, np.rint(xh / s32), 0.0)
    q = np.clip(q, -levels, levels).astype(np.int8)
    return q.reshape(T, d), sc


def dequant_h(q: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """q * s per head, exact in float64."""
    T, d = q.shape
    H = sc.shape[1]
    return (q.reshape(T, H, d // H).astype(np.float64) * sc.astype(np.float64)[..., None]).reshape(T, d)


def h_store(x: np.ndarray, act: str, n_heads: int, mode: str) -> np.ndarray:
    """The values a store-h slot holds for rows x (what K and V are rebuilt from)."""
    x_op = round_to_operand(x, act)
    if mode == "h":
        return x_op
    q, sc = quantize_h(x_op, n_heads, H_LEVELS[mode])
    return dequant_h(q, sc)


def delta_store(x: np.ndarray, prev_hat: np.ndarray, act: str, n_heads: int) -> np.ndarray:
    """Iteration-axis delta-KV ([BENCH] section 9): a loop layer's slot at
    iteration j >= 2 codes the difference between its x (operand type) and the
    previous iteration's reconstruction prev_hat as int8 with one fp16 scale per
    (row, head); the slot's reconstruction is prev_hat + q * s.  The difference
    and the sum are taken in fp32, in iteration order (anchor first), so the
    reconstruction error stays one code step at every depth.
    """
    x_op = round_to_operand(x, act).astype(np.float32)
    p32 = np.asarray(prev_hat, dtype=np.float64).astype(np.float32)
    q, sc = quantize_h(x_op - p32, n_heads, 127)
    T, d = q.shape
    step = (q.reshape(T, n_heads, d // n_heads).astype(np.float32)
            * sc.astype(np.float32)[..., None]).reshape(T, d)
    return (p32 + step).astype(np.float64)


def h_bytes_per_position(d: int, n_heads: int, mode: str, operand_bytes: int = 2) -> int:
    """Bytes one position takes in one slot: K and V, x in the operand type, or
    codes (one byte, or half a byte packed two to a byte) plus fp16 scales."""
    if mode == "kv":
        return 2 * d * operand_bytes
    if mode == "h":
        return d * operand_bytes
    if mode in ("h8", "d8"):       # d8: a delta slot; its anchor slot takes the "h" size
        return d + 2 * n_heads
    return d // 2 + 2 * n_heads


# ---------------------------------------------------------------------------
# model


BLOCK_MATS = ("wqkv", "wo", "wgate", "wup", "wdown")


def _stored_to_float(a: np.ndarray, kind: str, dt) -> np.ndarray:
    if kind == "bf16":
        return bf16_bits_to_float(a).astype(dt)
    return np.asarray(a).astype(dt)


@dataclass
class OracleModel:
    """Weights of one looped model converted to the oracle's float type ``dt``.

    blocks are ordered pre blocks, loop-stack layers, post blocks.  For an INT4 loop
    block the oracle quantises the fp32 draws itself (quantize_w4g128) and keeps q
    and s for the bit-exact comparison; an FP16-body loop block is fp16(q*s) of the
    same q and s.
    """
    spec: object
    dt: type
    embed: np.ndarray
    head: np.ndarray
    final_norm: np.ndarray
    blocks: list
    w4: dict = field(default_factory=dict)   # (block, name) -> (q int8, s fp16)
    embed_kind: str = "f32"
    kv_mode: str = "kv"                      # one of H_MODES: what a cache slot keeps

    @classmethod
    def from_weights(cls, w, dt=np.float64):
        spec = w.spec
        bkind = spec.boundary_dtype
        blocks, w4 = [], {}
        for b, blk in enumerate(w.blocks):
            kind = spec.block_kind(b)
            out = {"norm1": blk["norm1"].astype(dt), "norm2": blk["norm2"].astype(dt)}
            for name in BLOCK_MATS:
                a = blk[name]
                if kind == "loop" and spec.loop_dtype in ("w4g128", "f16body"):
                    q, s = quantize_w4g128(a)
                    w4[(b, name)] = (q, s)
                    mat = dequant_w4g128(q, s) if spec.loop_dtype == "w4g128" else fp16_body(q, s)
                    out[name] = mat.astype(dt)
                else:
                    k = spec.loop_dtype if kind == "loop" else bkind
                    out[name] = _stored_to_float(a, k, dt)
            blocks.append(out)
        return cls(spec=spec, dt=dt, embed=w.embed, head=_stored_to_float(w.head, bkind, dt),
                   final_norm=w.final_norm.astype(dt), blocks=blocks, w4=w4, embed_kind=bkind)

    # -- pieces of the pipeline

    def embed_rows(self, tokens: np.ndarray) -> np.ndarray:
        return _stored_to_float(self.embed[np.asarray(tokens)], self.embed_kind, self.dt)

    def block(self, b: int, h: np.ndarray, pos: np.ndarray, past_k: np.ndarray, past_v: np.ndarray,
              prev: np.ndarray | None = None):
        """One pre-norm block on rows h at positions pos of ONE lane.

        past_k/past_v hold the lane's earlier positions in this block application's
        own cache slot ([CLI] TINYLOOP_KV_H_MODE: per-layer K/V buffers).  Returns the
        new residual rows and the k, v rows to append to that slot.  In a store-h
        mode the slot keeps h_store(x) rows instead (returned as k, with v empty),
        and K, V of every position are rebuilt from them by this block's wqkv.  In
        the delta mode ("d8") prev holds the previous iteration's reconstruction of
        these rows for a loop slot at iteration >= 2 (delta_store), else None (the
        slot keeps x in the operand type: boundary blocks and the anchor).
        """
        sp, W = self.spec, self.blocks[b]
        H, dh, d = sp.n_heads, sp.head_dim, sp.d_model
        T = h.shape[0]
        x = rmsnorm(h, W["norm1"], sp.rms_eps)
        qkv = x @ W["wqkv"].T
        q = qkv[:, :d].reshape(T, H, dh)
        k = qkv[:, d:2 * d].reshape(T, H, dh)
        v = qkv[:, 2 * d:].reshape(T, H, dh)
        cos, sin = rope_angles(pos, dh, sp.rope_base, self.dt)
        q = apply_rope(q, cos, sin)
        if self.kv_mode == "kv":
            k = apply_rope(k, cos, sin)
            k_all = np.concatenate([past_k, k], axis=0)
            v_all = np.concatenate([past_v, v], axis=0)
        else:
            if self.kv_mode == "d8":
                k = (delta_store(x, prev, sp.act_dtype, H) if prev is not None
                     else h_store(x, sp.act_dtype, H, "h"))
            else:
                k = h_store(x, sp.act_dtype, H, self.kv_mode)      # the rows this slot keeps
            v = np.zeros((T, 0), dtype=self.dt)
            x_all = np.concatenate([past_k, k], axis=0)
            S = x_all.shape[0]
            kv_all = x_all @ W["wqkv"][d:].T
            c_all, s_all = rope_angles(np.arange(S), dh, sp.rope_base, self.dt)
            k_all = apply_rope(kv_all[:, :d].reshape(S, H, dh), c_all, s_all)
            v_all = kv_all[:, d:].reshape(S, H, dh)
        o = causal_attention(q, k_all, v_all, pos)
        h = h + o @ W["wo"].T
        x2 = rmsnorm(h, W["norm2"], sp.rms_eps)
        u = silu(x2 @ W["wgate"].T) * (x2 @ W["wup"].T)
        h = h + u @ W["wdown"].T
        return h, k, v

    def logits(self, h: np.ndarray) -> np.ndarray:
        """Final RMSNorm then the head projection (head readable at any state: [CLI] logit margin)."""
        return rmsnorm(h, self.final_norm, self.spec.rms_eps) @ self.head.T

    def empty_kv(self):
        sp = self.spec
        if self.kv_mode != "kv":
            return np.zeros((0, sp.d_model), dtype=self.dt), np.zeros((0, 0), dtype=self.dt)
        z = np.zeros((0, sp.n_heads, sp.head_dim), dtype=self.dt)
        return z, z

    def delta_prev(self, kv: dict, key, pos: np.ndarray):
        """Delta mode: the previous iteration's reconstruction of rows pos for a loop
        slot at iteration >= 2 (that slot already holds them), else None."""
        if self.kv_mode != "d8" or key[0] != "loop" or key[1] < 2:
            return None
        return kv[("loop", key[1] - 1, key[2])][0][np.asarray(pos)]

    def slots(self, L: int):
        """Block applications in pipeline order for depth L: (block index, cache-slot key)."""
        sp = self.spec
        seq = [(b, ("pre", b)) for b in range(sp.n_pre)]
        for j in range(1, L + 1):
            seq += [(sp.n_pre + l, ("loop", j, l)) for l in range(sp.n_loop)]
        seq += [(sp.n_pre + sp.n_loop + b, ("post", b)) for b in range(sp.n_post)]
        return seq


def greedy_argmax(logits: np.ndarray) -> np.ndarray:
    """Greedy token ([CLI] temperature 0): argmax over fp32 logits, lowest index on ties.

    The comparison is taken in fp32, the precision in which the GPU library takes it.
    """
    l32 = np.asarray(logits, dtype=np.float32)
    return np.argmax(l32, axis=-1).astype(np.int32)   # numpy returns the first maximum


# ---------------------------------------------------------------------------
# lanes: prefill, cached decode, monotone depth


@dataclass
class Lane:
    """One generation: its tokens, per-slot K/V caches, current length and depth ceiling."""
    tokens: list
    kv: dict
    ceiling: int
    pending: int = -1
    hidden_last: np.ndarray | None = None


def prefill(m: OracleModel, tokens, L: int, want_logits: str = "last"):
    """Full causal forward of one sequence at depth L, filling every slot's cache.

    Returns (lane, hidden [T, d], logits).  want_logits: "last" -> [V] at the last
    position, "all" -> [T, V], "none" -> None.  The lane's pending token is the
    greedy token at the last position; its depth ceiling is L.
    """
    assert L >= 1
    tokens = np.asarray(tokens, dtype=np.int64)
    T = len(tokens)
    pos = np.arange(T)
    h = m.embed_rows(tokens)
    kv = {}
    for b, key in m.slots(L):
        pk, pv = m.empty_kv()
        h, k, v = m.block(b, h, pos, pk, pv, prev=m.delta_prev(kv, key, pos))
        kv[key] = (k, v)
    lane = Lane(tokens=list(map(int, tokens)), kv=kv, ceiling=L, hidden_last=h[-1].copy())
    logits = None
    if want_logits == "all":
        logits = m.logits(h)
        lane.pending = int(greedy_argmax(logits[-1]))
    elif want_logits == "last":
        logits = m.logits(h[-1:])[0]
        lane.pending = int(greedy_argmax(logits))
    return lane, h, logits


def decode_step(m: OracleModel, lane: Lane, L_req: int, token: int | None = None):
    """One cached decode step of one lane.

    The effective depth is min(L_req, ceiling) and becomes the new ceiling, so depth
    never rises within a generation ([CLI] --early-exit-patience).  Every slot used
    at this depth already holds all earlier positions of the lane.  ``token``
    defaults to the lane's pending greedy token.  Returns (hidden [d], logits [V],
    next token, effective depth).
    """
    assert L_req >= 1
    L = min(int(L_req), lane.ceiling)
    tok = lane.pending if token is None else int(token)
    p = len(lane.tokens)
    pos = np.array([p])
    h = m.embed_rows(np.array([tok]))
    for b, key in m.slots(L):
        pk, pv = lane.kv[key]
        assert pk.shape[0] == p, "cache slot misses earlier positions"
        h, k, v = m.block(b, h, pos, pk, pv, prev=m.delta_prev(lane.kv, key, pos))
        lane.kv[key] = (np.concatenate([pk, k]), np.concatenate([pv, v]))
    lane.tokens.append(tok)
    lane.ceiling = L
    logits = m.logits(h)[0]
    nxt = int(greedy_argmax(logits))
    lane.pending = nxt
    lane.hidden_last = h[0].copy()
    return h[0], logits, nxt, L


# ---------------------------------------------------------------------------
# shared-prefix reuse ([BENCH] section 2, shared-prefix throughput: a prefix's
# cache is computed once and reused by many requests, across every loop
# iteration's slot)


def append(m: OracleModel, lane: Lane, tokens, L_req: int, want_logits: str = "last"):
    """Cached forward of several new tokens of one lane.

    The tokens take the next positions of the lane at depth L = min(L_req, ceiling)
    (monotone clamping as for a decode step); every block application attends to
    the lane's earlier positions in its own cache slot and, causally, to the new
    rows.  Returns (hidden [T, d], logits: [V] of the last row, [T, V] or None);
    the lane's pending token is the greedy token of the last row.
    """
    assert L_req >= 1
    tokens = np.asarray(tokens, dtype=np.int64)
    assert len(tokens) >= 1
    L = min(int(L_req), lane.ceiling)
    p0 = len(lane.tokens)
    pos = p0 + np.arange(len(tokens))
    h = m.embed_rows(tokens)
    for b, key in m.slots(L):
        pk, pv = lane.kv[key]
        assert pk.shape[0] == p0, "cache slot misses earlier positions"
        h, k, v = m.block(b, h, pos, pk, pv, prev=m.delta_prev(lane.kv, key, pos))
        lane.kv[key] = (np.concatenate([pk, k]), np.concatenate([pv, v]))
    lane.tokens.extend(map(int, tokens))
    lane.ceiling = L
    lane.hidden_last = h[-1].copy()
    logits = None
    if want_logits == "all":
        logits = m.logits(h)
        lane.pending = int(greedy_argmax(logits[-1]))
    elif want_logits == "last":
        logits = m.logits(h[-1:])[0]
        lane.pending = int(greedy_argmax(logits))
    return h, logits


def fork(lane: Lane, prefix_len: int) -> Lane:
    """A new lane holding the first prefix_len positions of ``lane``.

    Every cache slot keeps those positions (each loop iteration's slot included),
    the depth ceiling is the source's, and the pending token is the source's when
    the whole lane is taken (otherwise the next call appends tokens).  The source
    is left unchanged.
    """
    P = int(prefix_len)
    assert 1 <= P <= len(lane.tokens)
    kv = {key: (k[:P].copy(), v[:P].copy()) for key, (k, v) in lane.kv.items()}
    whole = P == len(lane.tokens)
    return Lane(tokens=list(lane.tokens[:P]), kv=kv, ceiling=lane.ceiling,
                pending=lane.pending if whole else -1,
                hidden_last=lane.hidden_last.copy() if whole and lane.hidden_last is not None else None)


# ---------------------------------------------------------------------------
# self-speculative decoding ([DYN] "Self-Speculative Decoding": draft at a low L,
# verify at a high L with the same weights; [CLI] "speculate": --draft-loops,
# --verify-loops, --draft-ahead, greedy at temperature 0)


def truncate(lane: Lane, n: int) -> None:
    """Drop every position from n on, in every cache slot (a rejected draft)."""
    assert 0 <= n <= len(lane.tokens)
    lane.tokens = lane.tokens[:n]
    lane.kv = {key: (k[:n], v[:n]) for key, (k, v) in lane.kv.items()}


def speculative_decode(m: OracleModel, lane: Lane, L_draft: int, L_verify: int, draft_ahead: int, n_tokens: int):
    """n_tokens greedy tokens at depth L_verify, proposed draft_ahead at a time at depth L_draft.

    A round starts from the lane's pending token t at position p (the lane's
    length).  Draft: draft_ahead cached greedy steps at depth min(L_draft, L) on
    the lane's own cache, t first, each step's token fed to the next; the lane's
    ceiling is not lowered.  Verify: the lane is cut back to p and
    [t, d_1 .. d_k] are appended at depth L = min(L_verify, ceiling) in one cached
    pass, which rewrites every slot at those positions; g_i is the greedy token
    after row i.  The drafts are accepted while d_i == g_(i-1); with a accepted
    (at most the tokens still wanted minus one), the round emits g_0 .. g_a, the
    lane keeps t, d_1 .. d_a and g_a becomes its pending token.  The emitted
    sequence is the one greedy decoding at depth L produces.
    Returns (tokens [n_tokens], accepted drafts per round).
    """
    assert draft_ahead >= 0 and n_tokens >= 1
    Lv = min(int(L_verify), lane.ceiling)
    Ld = min(int(L_draft), Lv)
    out, accepted = [], []
    while len(out) < n_tokens:
        want = n_tokens - len(out)
        p, t = len(lane.tokens), lane.pending
        drafts, tok = [], t
        for _ in range(draft_ahead):
            _, _, tok, _ = decode_step(m, lane, Ld, token=tok)
            lane.ceiling = Lv                      # a draft does not lower the depth bound
            drafts.append(tok)
        truncate(lane, p)
        _, logits = append(m, lane, [t] + drafts, Lv, want_logits="all")
        g = [int(greedy_argmax(row)) for row in logits]
        a = 0
        while a < len(drafts) and drafts[a] == g[a]:
            a += 1
        a = min(a, want - 1)
        truncate(lane, p + a + 1)
        lane.pending = g[a]
        out.extend(g[:a + 1])
        accepted.append(a)
    return out, accepted


# ---------------------------------------------------------------------------
# confidence-based early exit of cached decode ([CLI] "generate": the options
# --early-exit-patience, --early-exit-min-L, --early-exit-tau,
# --early-exit-peek-every and --early-exit-logit-margin)


@dataclass
class EarlyExit:
    """Early-exit rule of one decode call.

    patience: consecutive stable probes that end the token's loop (0 disables);
    min_L: first loop iteration that is probed; peek_every: probe every this many
    iterations from min_L on; tau: hidden-state rule, stable when the relative L2
    change of the residual over one iteration is below tau; logit_margin > 0
    switches to the logit rule, stable when top-1 minus top-2 of the full head
    projection at the current state exceeds it.
    """
    patience: int
    min_L: int = 2
    tau: float = 1e-3
    peek_every: int = 1
    logit_margin: float = 0.0


def probe_iteration(ee: EarlyExit, j: int, L: int) -> bool:
    """Iteration j of a token running at most L iterations is probed.

    Probes start at min_L and repeat every peek_every iterations; a probe after the
    last iteration (j = L) could not shorten the loop and is not taken.
    """
    return ee.patience > 0 and j < L and j >= ee.min_L and (j - ee.min_L) % ee.peek_every == 0


def relative_delta(h_prev: np.ndarray, h: np.ndarray) -> float:
    """||h - h_prev||_2 / ||h||_2 of one token's residual across one loop iteration."""
    return float(np.linalg.norm(h - h_prev) / np.linalg.norm(h))


def logit_margin(logits: np.ndarray) -> float:
    """Top-1 minus top-2 logit (the two largest values of the row; equal values give 0)."""
    top = np.sort(np.asarray(logits, dtype=np.float64).ravel())[-2:]
    return float(top[1] - top[0])


def decode_step_ee(m: OracleModel, lane: Lane, L_req: int, ee: EarlyExit, token: int | None = None):
    """decode_step with the early-exit rule applied after every probed iteration.

    The token starts with depth L = min(L_req, ceiling).  After probed iteration j
    the rule looks at the state h_j; a stable probe extends the streak, an unstable
    one resets it; when the streak reaches patience the loop stops at j (its later
    cache slots are not written) and j becomes the effective depth and the lane's
    new ceiling (monotone clamping keeps the cache consistent for later tokens).
    Returns (hidden [d], logits [V], next token, effective depth).
    """
    assert L_req >= 1
    L = min(int(L_req), lane.ceiling)
    tok = lane.pending if token is None else int(token)
    p = len(lane.tokens)
    pos = np.array([p])
    sp = m.spec
    h = m.embed_rows(np.array([tok]))

    def run(b, key, h):
        pk, pv = lane.kv[key]
        assert pk.shape[0] == p, "cache slot misses earlier positions"
        h, k, v = m.block(b, h, pos, pk, pv, prev=m.delta_prev(lane.kv, key, pos))
        lane.kv[key] = (np.concatenate([pk, k]), np.concatenate([pv, v]))
        return h

    for b in range(sp.n_pre):
        h = run(b, ("pre", b), h)
    eff, streak = L, 0
    for j in range(1, L + 1):
        h_prev = h
        for l in range(sp.n_loop):
            h = run(sp.n_pre + l, ("loop", j, l), h)
        if probe_iteration(ee, j, L):
            if ee.logit_margin > 0:
                stable = logit_margin(m.logits(h)[0]) > ee.logit_margin
            else:
                stable = relative_delta(h_prev[0], h[0]) < ee.tau
            streak = streak + 1 if stable else 0
            if streak >= ee.patience:
                eff = j
                break
    for b in range(sp.n_post):
        h = run(sp.n_pre + sp.n_loop + b, ("post", b), h)
    lane.tokens.append(tok)
    lane.ceiling = eff
    logits = m.logits(h)[0]
    nxt = int(greedy_argmax(logits))
    lane.pending = nxt
    lane.hidden_last = h[0].copy()
    return h[0], logits, nxt, eff


def clamp_depths(requests, first_ceiling: int) -> np.ndarray:
    """Non-increasing depths: L_i = min(request_i, L_{i-1}), L_0 = first_ceiling ([CLI])."""
    out, c = [], int(first_ceiling)
    for r in requests:
        c = min(int(r), c)
        out.append(c)
    return np.asarray(out, dtype=np.int32)


# ---------------------------------------------------------------------------
# batches at iteration granularity ([DYN] L-Aware Batching; [CDB] summary)


def active_lists(depths: np.ndarray, max_L: int | None = None):
    """active_1 = all rows; active_{j+1} = [r in active_j, in order, if depth[r] > j]."""
    depths = np.asarray(depths)
    if max_L is None:
        max_L = int(depths.max()) if len(depths) else 0
    lists = []
    cur = list(range(len(depths)))
    for j in range(1, max_L + 1):
        lists.append(np.asarray(cur, dtype=np.int32))
        cur = [r for r in cur if depths[r] > j]
    return lists


def forward_batch(m: OracleModel, seqs, Ls, want_logits: str = "last"):
    """Several sequences in one pass, scheduled one loop iteration at a time.

    Rows of all sequences go through each block application together; at iteration
    j only rows whose sequence depth is >= j are active (rows leave after their last
    iteration).  Attention stays within a sequence and its own cache slot.  Returns
    (hidden rows in input order [sum T, d], per-sequence last logits or None,
    active row lists per iteration).
    """
    sp = m.spec
    assert m.kv_mode != "d8", "the delta cache mode chains a lane's slots: use prefill / append / decode_step"
    seqs = [np.asarray(s, dtype=np.int64) for s in seqs]
    lens = [len(s) for s in seqs]
    starts = np.cumsum([0] + lens)
    row_seq = np.concatenate([np.full(n, i) for i, n in enumerate(lens)])
    row_pos = np.concatenate([np.arange(n) for n in lens])
    row_L = np.asarray(Ls)[row_seq]
    h = m.embed_rows(np.concatenate(seqs))

    def apply(b, rows):
        sub = h[rows]
        out = np.empty_like(sub)
        for i in np.unique(row_seq[rows]):
            sel = np.nonzero(row_seq[rows] == i)[0]
            pk, pv = m.empty_kv()
            out[sel], _, _ = m.block(b, sub[sel], row_pos[rows][sel], pk, pv)
        h[rows] = out

    all_rows = np.arange(len(row_seq))
    for b in range(sp.n_pre):
        apply(b, all_rows)
    lists = active_lists(row_L)
    for act in lists:
        for l in range(sp.n_loop):
            apply(sp.n_pre + l, act)
    for b in range(sp.n_post):
        apply(sp.n_pre + sp.n_loop + b, all_rows)
    logits = None
    if want_logits == "last":
        logits = m.logits(h[starts[1:] - 1])
    return h, logits, lists


def forward_ragged(m: OracleModel, tokens, depth_per_pos, want_logits: str = "all"):
    """One sequence whose position p runs depth_per_pos[p] loop iterations.

    With non-increasing depths the rows active at iteration j are a prefix of the
    sequence, so iteration j is a causal pass over that prefix in slot j.  This is
    the uncached counterpart of prompt prefill followed by cached steps at clamped
    per-token depths.  Returns (hidden [T, d], logits [T, V] or None).
    """
    sp = m.spec
    assert m.kv_mode != "d8", "the delta cache mode chains a lane's slots: use prefill / append / decode_step"
    tokens = np.asarray(tokens, dtype=np.int64)
    dep = np.asarray(depth_per_pos)
    assert np.all(np.diff(dep) <= 0) and dep.min() >= 1
    T = len(tokens)
    pos = np.arange(T)
    h = m.embed_rows(tokens)
    for b in range(sp.n_pre):
        pk, pv = m.empty_kv()
        h, _, _ = m.block(b, h, pos, pk, pv)
    for j in range(1, int(dep.max()) + 1):
        n = int(np.sum(dep >= j))
        for l in range(sp.n_loop):
            pk, pv = m.empty_kv()
            h[:n], _, _ = m.block(sp.n_pre + l, h[:n], pos[:n], pk, pv)
    for b in range(sp.n_post):
        pk, pv = m.empty_kv()
        h, _, _ = m.block(sp.n_pre + sp.n_loop + b, h, pos, pk, pv)
    logits = m.logits(h) if want_logits == "all" else None
    return h, logits
