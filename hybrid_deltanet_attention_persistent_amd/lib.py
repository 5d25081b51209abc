"""Thin ctypes binding of the C ABI in include/mk.h (argument marshalling only).

Every step of the forward pass runs in the HIP library; this module only converts
Python/numpy/torch arguments to the C types, allocates the device arena with
torch (PyTorch is used for device memory and streams only), and raises on a
non-zero status.  The functions keep the C names: mk_required_bytes,
mk_load_weights, mk_reset_state, mk_prefill, mk_decode_step, mk_sync_status,
mk_free.  There is no fallback: if libmk.so is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmk.so")

MK_OK, MK_EINVAL, MK_EDTYPE, MK_ESHAPE, MK_ECTX, MK_ESTATE, MK_ELAUNCH, MK_EHIP, MK_EHANG, MK_ETOKEN, MK_ENAN = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10)
MK_LAYER_DELTANET, MK_LAYER_ATTENTION = 0, 1
MK_DTYPE_BF16, MK_DTYPE_F16, MK_DTYPE_F32 = 1, 2, 3

EXPORTED = ["mk_required_bytes", "mk_load_weights", "mk_reset_state", "mk_prefill", "mk_decode_step",
            "mk_decode_step_static", "mk_sync_status", "mk_free", "mk_status_string", "mk_last_error",
            "mk_lookup_draft", "mk_generate_lookup", "mk_select_seq", "mk_decode_batch", "mk_set_prefill_blocks"]
MK_STATIC_SCRATCH_BYTES = 16 << 20


class MkError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class MkConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("layer_kind", ctypes.POINTER(ctypes.c_uint8)),
        ("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("dn_heads", ctypes.c_int32), ("dn_dk", ctypes.c_int32), ("dn_dv", ctypes.c_int32), ("conv_k", ctypes.c_int32),
        ("at_q_heads", ctypes.c_int32), ("at_kv_heads", ctypes.c_int32), ("at_head_dim", ctypes.c_int32),
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("l2_eps", ctypes.c_float),
        ("tied_embedding", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("prefill_chunk", ctypes.c_int32),
        ("max_verify", ctypes.c_int32), ("kv_quant", ctypes.c_int32), ("n_seq", ctypes.c_int32),
    ]


class MkLookupStats(ctypes.Structure):
    _fields_ = [("forwards", ctypes.c_int32), ("drafted", ctypes.c_int32), ("accepted", ctypes.c_int32)]


class MkTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("data", ctypes.c_void_p), ("on_device", ctypes.c_int32)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libmk.so (built by build.py).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.mk_required_bytes.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(sz)]
    lib.mk_load_weights.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(MkTensor), i32, vp, sz, vp,
                                    ctypes.POINTER(vp)]
    lib.mk_reset_state.argtypes = [vp, vp]
    lib.mk_prefill.argtypes = [vp, vp, i32, vp, vp, vp]
    lib.mk_decode_step.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.mk_decode_step_static.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.mk_sync_status.argtypes = [vp, vp, ctypes.POINTER(i32)]
    lib.mk_lookup_draft.argtypes = [vp, i32, i32, i32, i32, vp]
    lib.mk_generate_lookup.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, ctypes.POINTER(MkLookupStats), vp]
    lib.mk_select_seq.argtypes = [vp, i32]
    lib.mk_decode_batch.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.mk_set_prefill_blocks.argtypes = [vp, i32]
    lib.mk_free.argtypes = [vp]
    lib.mk_free.restype = None
    lib.mk_status_string.argtypes = [ctypes.c_int]
    lib.mk_status_string.restype = ctypes.c_char_p
    lib.mk_last_error.argtypes = []
    lib.mk_last_error.restype = ctypes.c_char_p
    for f in ("mk_required_bytes", "mk_load_weights", "mk_reset_state", "mk_prefill", "mk_decode_step",
              "mk_decode_step_static", "mk_sync_status", "mk_lookup_draft", "mk_generate_lookup", "mk_select_seq",
              "mk_decode_batch", "mk_set_prefill_blocks"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != MK_OK:
        lib = load_library()
        raise MkError(status, where, f"{lib.mk_status_string(status).decode()} ({lib.mk_last_error().decode()})")


def make_config(cfg) -> tuple:
    """mk_config for a workloads.ModelConfig; returns (struct, keep-alive buffer)."""
    kinds = (ctypes.c_uint8 * cfg.n_layers)(*[MK_LAYER_DELTANET if k == "D" else MK_LAYER_ATTENTION
                                              for k in cfg.layer_kinds])
    c = MkConfig(cfg.n_layers, ctypes.cast(kinds, ctypes.POINTER(ctypes.c_uint8)), cfg.hidden, cfg.vocab, cfg.ffn,
                 cfg.dn_heads, cfg.dn_dk, cfg.dn_dv, cfg.conv_k, cfg.at_q_heads, cfg.at_kv_heads, cfg.at_head_dim,
                 cfg.rope_theta, cfg.rms_eps, cfg.l2_eps, 1 if cfg.tied_embedding else 0, cfg.max_ctx,
                 cfg.prefill_chunk, cfg.max_verify, int(getattr(cfg, "kv_quant", 0)), int(getattr(cfg, "n_seq", 1)))
    return c, kinds


def make_tensors(weights: Dict[str, np.ndarray], dtype: int = MK_DTYPE_BF16):
    """mk_tensor array over the weights (bf16 bit patterns as uint16: host numpy arrays, or contiguous
    torch tensors, which may live on the GPU); returns (array, keep-alive)."""
    keep = []
    arr = (MkTensor * len(weights))()
    for i, (name, a) in enumerate(weights.items()):
        if hasattr(a, "data_ptr"):           # torch tensor (host or device memory)
            a = a.contiguous()
            ptr, on_dev, shp = a.data_ptr(), 1 if a.is_cuda else 0, tuple(a.shape)
        else:
            a = np.ascontiguousarray(a)
            ptr, on_dev, shp = a.ctypes.data, 0, a.shape
        keep.append(a)
        nm = name.encode()
        keep.append(nm)
        shape = (ctypes.c_int64 * 4)(*(list(shp) + [0] * (4 - len(shp))))
        arr[i] = MkTensor(nm, dtype, len(shp), shape, ptr, on_dev)
    return arr, keep


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ---------------------------------------------------------------------------- C-named wrappers
def mk_required_bytes(cfg) -> int:
    lib = load_library()
    c, keep = make_config(cfg)
    n = ctypes.c_size_t(0)
    _check(lib.mk_required_bytes(ctypes.byref(c), ctypes.byref(n)), "mk_required_bytes")
    return n.value


def mk_load_weights(cfg, weights: Dict[str, np.ndarray], arena, stream=None, dtype: int = MK_DTYPE_BF16) -> int:
    """Returns the opaque model handle (int).  `arena`: a torch uint8 CUDA tensor of mk_required_bytes."""
    lib = load_library()
    c, keep_c = make_config(cfg)
    arr, keep_t = make_tensors(weights, dtype)
    out = ctypes.c_void_p(0)
    _check(lib.mk_load_weights(ctypes.byref(c), arr, len(weights), arena.data_ptr(), arena.numel(),
                               _stream(stream), ctypes.byref(out)), "mk_load_weights")
    return out.value


def mk_reset_state(handle: int, stream=None) -> None:
    _check(load_library().mk_reset_state(handle, _stream(stream)), "mk_reset_state")


def mk_prefill(handle: int, tokens, next_token, last_logits=None, stream=None) -> None:
    _check(load_library().mk_prefill(handle, _ptr(tokens), int(tokens.numel()), _ptr(next_token),
                                     _ptr(last_logits), _stream(stream)), "mk_prefill")


def mk_set_prefill_blocks(handle: int, max_blocks: int) -> None:
    _check(load_library().mk_set_prefill_blocks(handle, int(max_blocks)), "mk_set_prefill_blocks")


def mk_decode_step(handle: int, tokens, n_tokens: int, argmax, logits=None, n_accepted=None, stream=None) -> None:
    _check(load_library().mk_decode_step(handle, _ptr(tokens), int(n_tokens), _ptr(argmax), _ptr(logits),
                                         _ptr(n_accepted), _stream(stream)), "mk_decode_step")


def mk_decode_step_static(handle: int, tokens, n_tokens: int, argmax, logits=None, n_accepted=None,
                          stream=None) -> None:
    _check(load_library().mk_decode_step_static(handle, _ptr(tokens), int(n_tokens), _ptr(argmax), _ptr(logits),
                                                _ptr(n_accepted), _stream(stream)), "mk_decode_step_static")


def mk_sync_status(handle: int, stream=None) -> int:
    """Synchronise and return the position; raises MkError on a device-side error."""
    pos = ctypes.c_int32(0)
    _check(load_library().mk_sync_status(handle, _stream(stream), ctypes.byref(pos)), "mk_sync_status")
    return pos.value


def mk_lookup_draft(history, ngram_min: int, ngram_max: int, max_draft: int) -> list:
    """Lookup draft tokens for `history` (host ints); see include/mk.h."""
    h = np.ascontiguousarray(np.asarray(history, dtype=np.int32))
    out = np.zeros(max(int(max_draft), 1), dtype=np.int32)
    n = load_library().mk_lookup_draft(h.ctypes.data if h.size else None, int(h.size), int(ngram_min), int(ngram_max),
                                       int(max_draft), out.ctypes.data)
    if n < 0:
        _check(n, "mk_lookup_draft")
    return out[:n].tolist()


def mk_generate_lookup(handle: int, history, last_token: int, n_generate: int, ngram_min: int = 1,
                       ngram_max: int = 3, stream=None) -> tuple:
    """Greedy tokens generated with lookup drafts: (tokens, {"forwards", "drafted", "accepted"})."""
    h = np.ascontiguousarray(np.asarray(history, dtype=np.int32))
    out = np.zeros(max(int(n_generate), 1), dtype=np.int32)
    st = MkLookupStats()
    _check(load_library().mk_generate_lookup(handle, h.ctypes.data if h.size else None, int(h.size), int(last_token),
                                             int(n_generate), int(ngram_min), int(ngram_max), out.ctypes.data,
                                             ctypes.byref(st), _stream(stream)), "mk_generate_lookup")
    return out[:n_generate].tolist(), {"forwards": st.forwards, "drafted": st.drafted, "accepted": st.accepted}


def mk_select_seq(handle: int, seq: int) -> None:
    _check(load_library().mk_select_seq(handle, int(seq)), "mk_select_seq")


def mk_decode_batch(handle: int, seqs, tokens, argmax, logits=None, stream=None) -> None:
    """One decode step for each sequence in `seqs` (host ints); tokens / argmax / logits are device buffers."""
    sq = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
    _check(load_library().mk_decode_batch(handle, sq.ctypes.data if sq.size else None, int(sq.size), _ptr(tokens),
                                          _ptr(argmax), _ptr(logits), _stream(stream)), "mk_decode_batch")


def mk_free(handle: int) -> None:
    load_library().mk_free(handle)


class Model:
    """Convenience owner of one loaded model: the torch arena and the handle."""

    def __init__(self, cfg, weights: Dict[str, np.ndarray], device: str = "cuda:0"):
        import torch
        self.cfg = cfg
        self.device = torch.device(device)
        nbytes = mk_required_bytes(cfg)
        with torch.cuda.device(self.device):
            self.arena = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
            off = (-self.arena.data_ptr()) % 256
            self.arena_view = self.arena[off:off + nbytes]
            self.handle = mk_load_weights(cfg, weights, self.arena_view)

    def reset(self):
        mk_reset_state(self.handle)

    def prefill(self, tokens, next_token, last_logits=None):
        mk_prefill(self.handle, tokens, next_token, last_logits)

    def set_prefill_blocks(self, max_blocks: int):
        mk_set_prefill_blocks(self.handle, max_blocks)

    def decode_step(self, tokens, argmax, logits=None, n_accepted=None, n_tokens: Optional[int] = None):
        mk_decode_step(self.handle, tokens, int(tokens.numel() if n_tokens is None else n_tokens), argmax, logits,
                       n_accepted)

    def sync(self) -> int:
        return mk_sync_status(self.handle)

    def select(self, seq: int):
        mk_select_seq(self.handle, seq)

    def decode_batch(self, seqs, tokens, argmax, logits=None):
        mk_decode_batch(self.handle, seqs, tokens, argmax, logits)

    def generate_lookup(self, history, last_token: int, n_generate: int, ngram_min: int = 1, ngram_max: int = 3):
        return mk_generate_lookup(self.handle, history, last_token, n_generate, ngram_min, ngram_max)

    def close(self):
        if self.handle:
            mk_free(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
