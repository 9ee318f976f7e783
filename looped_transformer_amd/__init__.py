"""Python binding of libtl.so, the MI355X (gfx950) looped-transformer runtime.

Argument marshalling only: every step of the hot path runs in the library's HIP
kernels.  Functions carry the C ABI's names (include/tl.h) and take numpy arrays
for host buffers and torch tensors (or raw integer addresses) for device buffers.
torch is used for device memory (through the allocator callback) and streams.
Loading fails loudly when the library has not been built; there is no CPU path.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# TL_LIBRARY names another build of the same library (the host-sanitizer build
# libtl_asan.so); by default the in-tree libtl.so
LIB_PATH = os.environ.get("TL_LIBRARY") or os.path.join(_HERE, "libtl.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "tl.h")

TL_OK, TL_E_ARG, TL_E_OOM, TL_E_HIP, TL_E_STATE, TL_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5
TL_DT_F32, TL_DT_F16, TL_DT_BF16, TL_DT_W4G128 = 0, 1, 2, 3
TL_KV_KV, TL_KV_H, TL_KV_H8, TL_KV_H4, TL_KV_D8 = 0, 1, 2, 3, 4
_STATUS = {0: "TL_OK", -1: "TL_E_ARG", -2: "TL_E_OOM", -3: "TL_E_HIP", -4: "TL_E_STATE", -5: "TL_E_UNSUPPORTED"}


class TLError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), message))
        self.status = status
        self.message = message


class tl_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("vocab", "d_model", "n_heads", "head_dim", "ffn",
                                              "n_pre", "n_loop", "n_post")] + [
        ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
        ("act_dtype", ctypes.c_int32), ("boundary_dtype", ctypes.c_int32), ("loop_dtype", ctypes.c_int32),
        ("loop_fp16_body", ctypes.c_int32), ("max_lanes", ctypes.c_int32), ("max_L", ctypes.c_int32),
        ("max_pos", ctypes.c_int32), ("kv_arena_bytes", ctypes.c_uint64), ("kv_mode", ctypes.c_int32),
        ("batch_invariant", ctypes.c_int32)]


class tl_block_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("norm1", "norm2", "wqkv", "wo", "wgate", "wup", "wdown")]


class tl_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("blocks", ctypes.POINTER(tl_block_weights))]


class tl_early_exit(ctypes.Structure):
    _fields_ = [("patience", ctypes.c_int32), ("min_L", ctypes.c_int32), ("peek_every", ctypes.c_int32),
                ("tau", ctypes.c_float), ("logit_margin", ctypes.c_float)]


ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)
DEALLOC_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p)

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def lib():
    """Load libtl.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("%s is not built (run __graft_entry__.build()); there is no fallback path" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "tl_load_weights": [ctypes.POINTER(tl_config), ctypes.POINTER(tl_weights), ALLOC_FN, DEALLOC_FN, _P, _P,
                            ctypes.POINTER(_P)],
        "tl_forward": [_P, _I, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P],
        "tl_append": [_P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "tl_lane_fork": [_P, _I, _I, _I, _I, _P],
        "tl_speculate": [_P, _I, _P, _I, _I, _I, _I, _P, _P, _P],
        "tl_decode_step": [_P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "tl_decode_step_noalloc": [_P, _I, _P, _P, _P, _P, _P, _P, _P, _P],
        "tl_decode_step_ee": [_P, _I, _P, _P, ctypes.POINTER(tl_early_exit), _P, _P, _P, _P, _P, _P],
        "tl_decode_run": [_P, _I, _P, _I, _P, _P, _P, _P, _P, _I, _P],
        "tl_export_w4": [_P, _I, _I, _P, _P],
        "tl_lane_release": [_P, _I],
        "tl_memory_info": [_P, _P, _P, _P],
        "tl_sync_errors": [_P, _P],
        "tl_timing_enable": [_P, _I],
        "tl_timing_read": [_P, _P, _P],
        "tl_timing_read_kernels": [_P, _P, _P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.tl_free.argtypes = [_P]
    L.tl_free.restype = None
    L.tl_last_error.argtypes = []
    L.tl_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def header_symbols(path: str = HEADER):
    """Names of the functions include/tl.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:tl_status|void|const char\*)\s+(tl_\w+)\s*\(", text, re.M)))


def tl_last_error() -> str:
    return lib().tl_last_error().decode()


def _check(status: int):
    if status != TL_OK:
        raise TLError(status, tl_last_error())


def _ptr(x):
    """Device or host address of a torch tensor / numpy array / int; None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data
    if hasattr(x, "data_ptr"):
        assert x.is_contiguous()
        return x.data_ptr()
    raise TypeError(type(x))


def _i32(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


class TorchAllocator:
    """Device memory from torch's caching allocator, held until the library frees it."""

    def __init__(self, device: int = 0):
        import torch
        self._torch = torch
        self.device = device
        self.live = {}
        self.alloc_cb = ALLOC_FN(self._alloc)
        self.free_cb = DEALLOC_FN(self._free)

    def _alloc(self, nbytes, user):
        try:
            t = self._torch.empty(int(nbytes), dtype=self._torch.uint8, device="cuda:%d" % self.device)
        except Exception:
            return None
        p = t.data_ptr()
        self.live[p] = t
        return p

    def _free(self, p, user):
        self.live.pop(p, None)


class Model:
    """Handle returned by tl_load_weights; keeps the allocator alive with the model."""

    def __init__(self, handle, allocator, cfg):
        self.handle = handle
        self.allocator = allocator
        self.cfg = cfg

    @property
    def _as_parameter_(self):
        return self.handle


def tl_load_weights(cfg: tl_config, embed, head, final_norm, blocks, stream=None, allocator="torch") -> Model:
    """blocks: list of dicts with numpy arrays norm1, norm2, wqkv, wo, wgate, wup, wdown (canonical layout)."""
    keep = [np.ascontiguousarray(embed), np.ascontiguousarray(head),
            np.ascontiguousarray(final_norm, dtype=np.float32)]
    arr = (tl_block_weights * len(blocks))()
    for i, b in enumerate(blocks):
        fields = {}
        for k in ("norm1", "norm2", "wqkv", "wo", "wgate", "wup", "wdown"):
            a = np.ascontiguousarray(b[k])
            keep.append(a)
            fields[k] = a.ctypes.data
        arr[i] = tl_block_weights(**fields)
    head_ptr = keep[0].ctypes.data if head is embed else keep[1].ctypes.data
    w = tl_weights(keep[0].ctypes.data, head_ptr, keep[2].ctypes.data, arr)
    # "torch": torch's caching allocator; None: hipMalloc; or an object with
    # alloc_cb / free_cb (e.g. a TorchAllocator subclass)
    alloc = TorchAllocator() if isinstance(allocator, str) and allocator == "torch" else allocator
    out = _P()
    st = lib().tl_load_weights(ctypes.byref(cfg), ctypes.byref(w),
                               alloc.alloc_cb if alloc else ALLOC_FN(0), alloc.free_cb if alloc else DEALLOC_FN(0),
                               None, _stream(stream), ctypes.byref(out))
    _check(st)
    return Model(out.value, alloc, cfg)


def tl_forward(model, cu_seqlens, tokens, L=1, seq_L=None, lanes=None, max_new_tokens=0, out_hidden=None,
               out_logits=None, out_next=None, out_active_log=None, stream=None):
    cu = _i32(cu_seqlens)
    sl = _i32(seq_L)
    ln = _i32(lanes)
    _check(lib().tl_forward(model.handle, len(cu) - 1, _ptr(cu), _ptr(tokens), int(L), _ptr(sl), _ptr(ln),
                            int(max_new_tokens), _ptr(out_hidden), _ptr(out_logits), _ptr(out_next),
                            _ptr(out_active_log), _stream(stream)))


def tl_append(model, cu_seqlens, tokens, lanes, per_seq_L, out_hidden=None, out_logits=None, out_next=None,
              stream=None):
    """Returns the effective depths (numpy int32)."""
    cu = _i32(cu_seqlens)
    ln = _i32(lanes)
    pl = _i32(per_seq_L)
    eff = np.zeros(len(ln), np.int32)
    _check(lib().tl_append(model.handle, len(cu) - 1, _ptr(cu), _ptr(tokens), _ptr(ln), _ptr(pl), _ptr(out_hidden),
                           _ptr(out_logits), _ptr(out_next), _ptr(eff), _stream(stream)))
    return eff


def tl_lane_fork(model, src_lane: int, dst_lane: int, prefix_len: int, max_new_tokens: int = 0, stream=None):
    _check(lib().tl_lane_fork(model.handle, int(src_lane), int(dst_lane), int(prefix_len), int(max_new_tokens),
                              _stream(stream)))


def tl_speculate(model, lanes, L_draft, L_verify, draft_ahead, n_tokens, out_tokens, stream=None):
    """Returns the accepted drafts per round, [n_lanes, n_tokens] int32 (-1 after the last round)."""
    ln = _i32(lanes)
    acc = np.zeros((len(ln), int(n_tokens)), np.int32)
    _check(lib().tl_speculate(model.handle, len(ln), _ptr(ln), int(L_draft), int(L_verify), int(draft_ahead),
                              int(n_tokens), _ptr(out_tokens), _ptr(acc), _stream(stream)))
    return acc


def tl_decode_step(model, lanes, per_lane_L, out_tokens, in_tokens=None, out_logits=None, out_hidden=None,
                   out_active_log=None, stream=None):
    """Returns the effective depths (numpy int32)."""
    ln = _i32(lanes)
    pl = _i32(per_lane_L)
    eff = np.zeros(len(ln), np.int32)
    _check(lib().tl_decode_step(model.handle, len(ln), _ptr(ln), _ptr(pl), _ptr(in_tokens), _ptr(out_tokens),
                                _ptr(out_logits), _ptr(out_hidden), _ptr(eff), _ptr(out_active_log),
                                _stream(stream)))
    return eff


def tl_decode_step_noalloc(model, lanes, per_lane_L, out_tokens, in_tokens=None, out_logits=None, out_hidden=None,
                           stream=None):
    """tl_decode_step on the library's per-device scratch (no allocation);
    returns the effective depths."""
    ln = _i32(lanes)
    pl = _i32(per_lane_L)
    eff = np.zeros(len(ln), np.int32)
    _check(lib().tl_decode_step_noalloc(model.handle, len(ln), _ptr(ln), _ptr(pl), _ptr(in_tokens),
                                        _ptr(out_tokens), _ptr(out_logits), _ptr(out_hidden), _ptr(eff),
                                        _stream(stream)))
    return eff


def tl_decode_step_ee(model, lanes, per_lane_L, out_tokens, patience, min_L=2, tau=1e-3, peek_every=1,
                      logit_margin=0.0, in_tokens=None, out_logits=None, out_hidden=None, stream=None):
    """Decode step with the device-side early-exit rule; returns the effective depths."""
    ln = _i32(lanes)
    pl = _i32(per_lane_L)
    eff = np.zeros(len(ln), np.int32)
    rule = tl_early_exit(int(patience), int(min_L), int(peek_every), float(tau), float(logit_margin))
    _check(lib().tl_decode_step_ee(model.handle, len(ln), _ptr(ln), _ptr(pl), ctypes.byref(rule), _ptr(in_tokens),
                                   _ptr(out_tokens), _ptr(out_logits), _ptr(out_hidden), _ptr(eff),
                                   _stream(stream)))
    return eff


def tl_decode_run(model, lanes, L_req, out_tokens, in_tokens=None, out_hidden=None, boundary_min=1, stream=None):
    """L_req: [n_lanes, n_steps]; returns the effective depths [n_lanes, n_steps]."""
    ln = _i32(lanes)
    req = _i32(L_req)
    n, steps = req.shape
    eff = np.zeros((n, steps), np.int32)
    _check(lib().tl_decode_run(model.handle, n, _ptr(ln), steps, _ptr(req), _ptr(in_tokens), _ptr(out_tokens),
                               _ptr(out_hidden), _ptr(eff), int(boundary_min), _stream(stream)))
    return eff


def tl_export_w4(model, block: int, matrix: int, N: int, K: int):
    q = np.empty((N, K), np.int8)
    s = np.empty((N, K // 128), np.uint16)
    _check(lib().tl_export_w4(model.handle, block, matrix, _ptr(q), _ptr(s)))
    return q, s


def tl_lane_release(model, lane: int):
    _check(lib().tl_lane_release(model.handle, int(lane)))


def tl_memory_info(model):
    vals = [ctypes.c_uint64() for _ in range(3)]
    _check(lib().tl_memory_info(model.handle, *[ctypes.addressof(v) for v in vals]))
    return tuple(v.value for v in vals)


def tl_sync_errors(model, stream=None):
    _check(lib().tl_sync_errors(model.handle, _stream(stream)))


TIMING_CLASSES = ("gemm_qkv_loop", "gemm_o_loop", "gemm_gu_loop", "gemm_down_loop", "gemm_qkv_boundary",
                  "gemm_o_boundary", "gemm_gu_boundary", "gemm_down_boundary", "attention", "rmsnorm", "head",
                  "compact", "embed", "hrebuild")


def tl_timing_enable(model, on: bool = True):
    _check(lib().tl_timing_enable(model.handle, 1 if on else 0))


def tl_timing_read(model):
    """{class name: (total ms, launches)} since the last read."""
    ms = np.zeros(len(TIMING_CLASSES), np.float64)
    n = np.zeros(len(TIMING_CLASSES), np.int64)
    _check(lib().tl_timing_read(model.handle, _ptr(ms), _ptr(n)))
    return {k: (float(ms[i]), int(n[i])) for i, k in enumerate(TIMING_CLASSES)}


def tl_timing_read_kernels(model):
    """{class name: (summed kernel ms, kernels)} since the last read: the product
    kernels' own durations, stamped by the runtime."""
    ms = np.zeros(len(TIMING_CLASSES), np.float64)
    n = np.zeros(len(TIMING_CLASSES), np.int64)
    _check(lib().tl_timing_read_kernels(model.handle, _ptr(ms), _ptr(n)))
    return {k: (float(ms[i]), int(n[i])) for i, k in enumerate(TIMING_CLASSES)}


def tl_free(model):
    if model.handle:
        lib().tl_free(model.handle)
        model.handle = None
