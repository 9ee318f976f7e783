"""Test and benchmark helpers: map synthetic model specs onto the C ABI structs,
and compare device outputs with the oracle's.

Marshalling and comparison only; no model arithmetic happens here.
"""
from __future__ import annotations

import os

import numpy as np

import looped_transformer_amd as tl
import synth

DT = {"f32": tl.TL_DT_F32, "f16": tl.TL_DT_F16, "bf16": tl.TL_DT_BF16}
ESZ = {"f32": 4, "f16": 2, "bf16": 2}


def ensure_built():
    """Build the HIP library and the input generator if they are missing."""
    if not os.path.exists(tl.LIB_PATH):
        from looped_transformer_amd import build as _b
        _b.build()
    synth.build()


def make_config(spec: synth.ModelSpec, max_lanes: int = 0, max_L: int = 32, max_pos: int = 1024,
                kv_arena_bytes: int = 0, kv_mode: int = 0, batch_invariant: int = 0) -> tl.tl_config:
    c = tl.tl_config()
    c.vocab, c.d_model, c.n_heads, c.head_dim, c.ffn = spec.vocab, spec.d_model, spec.n_heads, spec.head_dim, spec.ffn
    c.n_pre, c.n_loop, c.n_post = spec.n_pre, spec.n_loop, spec.n_post
    c.rms_eps, c.rope_base = spec.rms_eps, spec.rope_base
    c.boundary_dtype = DT[spec.boundary_dtype]
    c.act_dtype = DT[spec.act_dtype]
    if spec.loop_dtype in ("w4g128", "f16body"):
        c.loop_dtype = tl.TL_DT_W4G128
        c.loop_fp16_body = 1 if spec.loop_dtype == "f16body" else 0
    else:
        c.loop_dtype = DT[spec.loop_dtype]
    c.max_lanes, c.max_L, c.max_pos, c.kv_arena_bytes = max_lanes, max_L, max_pos, kv_arena_bytes
    c.kv_mode = kv_mode
    c.batch_invariant = batch_invariant
    return c


def kv_bytes(spec: synth.ModelSpec, ceilings, caps) -> int:
    """Bytes a set of lanes needs: one slot per block application, K and V, cap positions."""
    tot = 0
    for L, cap in zip(ceilings, caps):
        slots = spec.n_pre + spec.n_post + spec.n_loop * int(L)
        e = slots * 2 * spec.d_model * int(cap)
        tot += (e + 63) // 64 * 64
    return tot * ESZ[spec.act_dtype] + (1 << 20)


def load_model(w: synth.Weights, **cfg_kw) -> tl.Model:
    cfg = make_config(w.spec, **cfg_kw)
    return tl.tl_load_weights(cfg, w.embed, w.head, w.final_norm, w.blocks)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def row_rel_max(a, b) -> float:
    """Largest per-row relative L2 error over the rows of [rows, d] arrays."""
    a = np.asarray(a, dtype=np.float64).reshape(-1, np.shape(b)[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, np.shape(b)[-1])
    return float(np.max(np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)))


def near_tie_gaps(got_tokens, ref_logits) -> list:
    """For each token where the device's greedy choice differs from the oracle's,
    the oracle's own logit gap between its best token and the device's token, in
    units of the row's rms logit.  An empty list means every token agreed."""
    lg = np.asarray(ref_logits, dtype=np.float64).reshape(len(got_tokens), -1)
    got = np.asarray(got_tokens, dtype=np.int64)
    import oracle
    top = oracle.greedy_argmax(lg)
    gaps = []
    for t in np.nonzero(top != got)[0]:
        row = lg[t]
        gaps.append(float((row[top[t]] - row[got[t]]) / np.sqrt(np.mean(row * row))))
    return gaps
