"""Seeded synthetic inputs for the looped transformer (weights, ids, loop counts).

This package is shared by the CPU oracle (``oracle/``) and the GPU library's tests
and benchmark.  It generates random numbers and rounds them to their storage type;
it holds none of the model's arithmetic (no quantisation, no depth clamping, no
norms or products).  The generator is defined in ``synth.c``.

Model shapes follow the five workloads of the looped-transformer study: a tiny fp32
model, a 2048-wide model with an INT4 (or FP16-body) shared loop block, and a
5280-wide bf16 model with a 4-layer shared loop stack.  The pipeline itself
(embed -> pre blocks -> shared loop block x L -> head) is described on the
"vs generic runtimes" page, section "Where Generic Runtimes Lose On Looped
Checkpoints".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libtlsynth.so")
_lib = None

# stream ids: one independent counter stream per tensor / draw kind
STREAM_EMBED = 1
STREAM_HEAD = 2
STREAM_TOKENS = 1000
STREAM_PROMPT_TOKENS = 1001
STREAM_PROMPT_LENS = 1002
STREAM_LANE_L = 2000
STREAM_TOKEN_L = 2001
BLOCK_TENSORS = ("wqkv", "wo", "wgate", "wup", "wdown")


def block_stream(block_index: int, tensor: str) -> int:
    return 16 + 8 * block_index + BLOCK_TENSORS.index(tensor)


def build(force: bool = False) -> str:
    """Compile the generator with gcc (OpenMP, F16C)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-mf16c", "-msse4.1",
               _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, vp = ctypes.c_uint64, ctypes.c_void_p
        lib.syn_draw.restype = u64
        lib.syn_draw.argtypes = [u64, u64, u64]
        lib.syn_normal.argtypes = [u64, u64, u64, ctypes.c_double, ctypes.c_int, vp]
        lib.syn_uniform_int.argtypes = [u64, u64, u64, ctypes.c_int32, ctypes.c_uint32, vp]
        lib.syn_poisson.argtypes = [u64, u64, u64, ctypes.c_double, vp]
        lib.syn_f32_to_f16.argtypes = [vp, u64, vp]
        lib.syn_f32_to_bf16.argtypes = [vp, u64, vp]
        _lib = lib
    return _lib


def draw(seed: int, stream: int, i: int) -> int:
    return int(_get().syn_draw(seed, stream, i))


_KIND = {"f32": 0, "f16": 1, "bf16": 2}


def normal(seed: int, stream: int, shape, std: float = 0.02, dtype: str = "f32") -> np.ndarray:
    """N(0, std) draws rounded to fp32 and then to ``dtype``.

    fp16 comes back as numpy float16; bf16 comes back as its raw uint16 bits
    (numpy has no bf16), see :func:`bf16_to_f32`.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype={"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype])
    if n:
        _get().syn_normal(seed, stream, n, float(std), _KIND[dtype], out.ctypes.data)
    return out.reshape(shape)


def uniform_int(seed: int, stream: int, n: int, lo: int, n_range: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if n:
        _get().syn_uniform_int(seed, stream, n, lo, n_range, out.ctypes.data)
    return out


def poisson(seed: int, stream: int, n: int, lam: float) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if n:
        _get().syn_poisson(seed, stream, n, float(lam), out.ctypes.data)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _get().syn_f32_to_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# model and workload shapes


@dataclass
class ModelSpec:
    name: str
    vocab: int
    d_model: int
    n_heads: int
    head_dim: int
    ffn: int
    n_pre: int
    n_loop: int          # layers in the shared loop stack
    n_post: int
    boundary_dtype: str  # storage of embed, head, pre and post blocks: f32 | f16 | bf16
    loop_dtype: str      # f32 | f16 | bf16 | w4g128 | f16body (fp16 of the dequantised INT4 weights)
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    std: float = 0.02
    act: str = ""        # GEMM operand type on the GPU path ("" = boundary_dtype)

    @property
    def n_blocks(self) -> int:
        return self.n_pre + self.n_loop + self.n_post

    def block_kind(self, b: int) -> str:
        if b < self.n_pre:
            return "pre"
        if b < self.n_pre + self.n_loop:
            return "loop"
        return "post"

    @property
    def act_dtype(self) -> str:
        """Element type of the GEMM operands on the GPU path."""
        return self.act or self.boundary_dtype

    def block_params(self) -> int:
        d, f = self.d_model, self.ffn
        return 4 * d * d + 3 * d * f


SPECS = {
    1: ModelSpec("tiny-fp32", 256, 64, 4, 16, 256, 1, 1, 0, "f32", "f32"),
    2: ModelSpec("d2048-int4loop", 50304, 2048, 16, 128, 5632, 1, 1, 0, "f16", "w4g128"),
    3: ModelSpec("d2048-fp16body", 50304, 2048, 16, 128, 5632, 1, 1, 0, "f16", "f16body"),
    4: ModelSpec("d2048-int4loop", 50304, 2048, 16, 128, 5632, 1, 1, 0, "f16", "w4g128"),
    5: ModelSpec("d5280-bf16-stack4", 65536, 5280, 55, 96, 17920, 2, 4, 2, "bf16", "bf16", act="f32"),
}


@dataclass
class Weights:
    """Canonical host weights.  Linear weights are [out, in] row-major (y = x W^T).

    wqkv rows: q (head 0..H-1, head_dim rows each), then k, then v.
    Loop blocks of an INT4 model come as fp32 draws (each side quantises them);
    bf16 tensors are raw uint16 bits.
    """
    spec: ModelSpec
    embed: np.ndarray
    head: np.ndarray
    final_norm: np.ndarray
    blocks: list = field(default_factory=list)   # dicts: norm1, wqkv, wo, norm2, wgate, wup, wdown


def _draw_dtype(spec: ModelSpec, kind: str) -> str:
    if kind == "loop":
        if spec.loop_dtype in ("w4g128", "f16body"):
            return "f32"
        return spec.loop_dtype
    return spec.boundary_dtype


def make_weights(spec: ModelSpec, seed: int = 0) -> Weights:
    d, f, v = spec.d_model, spec.ffn, spec.vocab
    w = Weights(spec,
                embed=normal(seed, STREAM_EMBED, (v, d), spec.std, spec.boundary_dtype),
                head=normal(seed, STREAM_HEAD, (v, d), spec.std, spec.boundary_dtype),
                final_norm=np.ones(d, np.float32))
    shapes = {"wqkv": (3 * d, d), "wo": (d, d), "wgate": (f, d), "wup": (f, d), "wdown": (d, f)}
    for b in range(spec.n_blocks):
        dt = _draw_dtype(spec, spec.block_kind(b))
        blk = {"norm1": np.ones(d, np.float32), "norm2": np.ones(d, np.float32)}
        for t in BLOCK_TENSORS:
            blk[t] = normal(seed, block_stream(b, t), shapes[t], spec.std, dt)
        w.blocks.append(blk)
    return w


# ---------------------------------------------------------------------------
# workloads (token ids and loop counts); every id is uniform in [0, vocab)


def tokens(seed: int, stream: int, n: int, vocab: int) -> np.ndarray:
    return uniform_int(seed, stream, n, 0, vocab)


def lane_loops(seed: int, n_lanes: int, choices=(2, 4, 8, 16, 32)) -> np.ndarray:
    """Per-lane loop count drawn uniformly from ``choices`` (held for the whole generation)."""
    idx = uniform_int(seed, STREAM_LANE_L, n_lanes, 0, len(choices))
    return np.asarray(choices, dtype=np.int32)[idx]


def token_loop_draws(seed: int, n_seqs: int, n_tokens: int, lam: float = 7.0, cap: int = 32) -> np.ndarray:
    """Raw per-token draws min(cap, 1 + Poisson(lam)), shape [n_seqs, n_tokens].

    These are requests; the non-increasing clamp along each sequence is applied by
    whoever runs the model, not here.
    """
    p = poisson(seed, STREAM_TOKEN_L, n_seqs * n_tokens, lam)
    return np.minimum(cap, 1 + p).astype(np.int32).reshape(n_seqs, n_tokens)


def prompt_lengths(seed: int, n_seqs: int, lo: int = 32, hi: int = 512) -> np.ndarray:
    return uniform_int(seed, STREAM_PROMPT_LENS, n_seqs, lo, hi - lo + 1)
