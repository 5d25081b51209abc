"""C-ABI boundary tests that need no GPU: the library loads, exports every declared
symbol, and rejects bad calls before anything is enqueued (the loader checks the
type of every tensor, as on the page "업데이트: 단일 RTX 3090에서 Qwen 3.8 27B를 140 tok/s로
구동", section on the merged PRs)."""
import ctypes
import dataclasses
import os
import re

import numpy as np
import pytest

import workloads as W
from hybrid_deltanet_attention_persistent_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(L.LIB_PATH):
        from hybrid_deltanet_attention_persistent_amd import build
        build.build()
    return L.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_named_calls():
    names = declared_functions()
    for n in ("mk_load_weights", "mk_prefill", "mk_decode_step", "mk_reset_state"):
        assert n in names


def test_library_exports_every_declared_symbol(so):
    for name in declared_functions():
        assert hasattr(so, name), name
    assert set(declared_functions()) == set(L.EXPORTED)


def test_status_strings(so):
    for code in range(0, -11, -1):
        s = so.mk_status_string(code).decode()
        assert s and s != "unknown status"
    assert so.mk_status_string(-99).decode() == "unknown status"


@pytest.mark.parametrize("cfg", [W.TINY, W.HYBRID_24L])
def test_required_bytes(so, cfg):
    n = L.mk_required_bytes(cfg)
    weights = W.param_count(cfg) * 2
    assert n > weights
    assert n % 256 == 0


def test_required_bytes_scales_with_context(so):
    a = L.mk_required_bytes(W.HYBRID_24L)
    b = L.mk_required_bytes(dataclasses.replace(W.HYBRID_24L, max_ctx=1024))
    kv = 6 * 2 * (8448 - 1024) * 2 * 128 * 2      # 6 layers x K,V x positions x kv heads x hd x bf16
    rope = (8448 - 1024) * 64 * 2 * 4             # cos/sin table
    assert kv + rope <= a - b <= kv + rope + 65536


def test_required_bytes_with_8bit_cache(so):
    """The 8-bit cache holds one byte per element plus two exponent bytes (K, V) per position and
    kv head: half the bf16 cache's element bytes."""
    a = L.mk_required_bytes(W.HYBRID_24L)
    b = L.mk_required_bytes(W.HYBRID_24L_Q8)
    pos = 8448 * 2                                # positions x kv heads
    saved = 6 * 2 * pos * 128                     # 6 layers x K,V x one byte less per element
    exps = 6 * pos * 2                            # 6 layers x (K, V) exponent bytes
    assert saved - exps - 65536 <= a - b <= saved - exps + 65536


def test_required_bytes_per_sequence(so):
    """Each sequence past the first adds its own DeltaNet states, conv rings, pending buffers, KV
    cache, control block and layer table; the weights are shared."""
    cfg = W.HYBRID_24L
    a = L.mk_required_bytes(cfg)
    b = L.mk_required_bytes(dataclasses.replace(cfg, n_seq=3))
    assert L.mk_required_bytes(dataclasses.replace(cfg, n_seq=0)) == a == L.mk_required_bytes(dataclasses.replace(cfg, n_seq=1))
    n_dn, n_at = 18, 6
    S = 8 * 128 * 128 * 4
    ring = 8 * cfg.conv_channels * 4
    pend = 2 * 8 * 5 * (256 + 4 * 128) * 4
    kv = 2 * cfg.max_ctx * 2 * 128 * 2
    per_seq = n_dn * (S + ring + pend) + n_at * kv
    assert 2 * per_seq <= b - a <= 2 * per_seq + 2 * (cfg.n_layers * 3 + 2) * 256 + 2 * cfg.n_layers * 256


@pytest.mark.parametrize("change", [
    dict(kv_quant=2), dict(kv_quant=-1), dict(n_seq=6), dict(n_seq=-1),
    dict(hidden=300), dict(dn_heads=9), dict(dn_dk=96, dn_dv=96), dict(at_head_dim=32),
    dict(at_q_heads=6, at_kv_heads=4), dict(max_verify=6), dict(max_verify=0), dict(max_ctx=100),
    dict(max_ctx=20480), dict(prefill_chunk=32), dict(conv_k=3), dict(tied_embedding=False), dict(ffn=100),
    dict(vocab=0), dict(rms_eps=-1.0),
])
def test_bad_config_rejected(so, change):
    cfg = dataclasses.replace(W.TINY, **change)
    with pytest.raises(L.MkError) as e:
        L.mk_required_bytes(cfg)
    assert e.value.status == L.MK_EINVAL


def test_bad_layer_kind_rejected(so):
    c, keep = L.make_config(W.TINY)
    c.layer_kind[2] = 7
    n = ctypes.c_size_t(0)
    assert so.mk_required_bytes(ctypes.byref(c), ctypes.byref(n)) == L.MK_EINVAL
    assert so.mk_required_bytes(None, ctypes.byref(n)) == L.MK_EINVAL


def _load(so, cfg, weights, arena=None, nbytes=0, dtype=L.MK_DTYPE_BF16, tensors=None):
    c, keep_c = L.make_config(cfg)
    arr, keep_t = (tensors if tensors is not None else L.make_tensors(weights, dtype))
    out = ctypes.c_void_p(0)
    st = so.mk_load_weights(ctypes.byref(c), arr, len(arr), arena, nbytes, None, ctypes.byref(out))
    return st, out.value


@pytest.fixture(scope="module")
def tiny_weights():
    return W.make_weights(W.TINY, seed=0)


def test_loader_checks_every_tensor_type(so, tiny_weights):
    for name in ("embed", "layers.3.attn.wk", "layers.1.dn.conv", "lnf"):
        w = dict(tiny_weights)
        arr, keep = L.make_tensors(w)
        idx = list(w).index(name)
        arr[idx].dtype = L.MK_DTYPE_F32
        st, h = _load(so, W.TINY, w, tensors=(arr, keep))
        assert st == L.MK_EDTYPE and h is None
        assert name in so.mk_last_error().decode()


def test_loader_rejects_bad_on_device_flag(so, tiny_weights):
    arr, keep = L.make_tensors(tiny_weights)
    arr[3].on_device = 2
    st, h = _load(so, W.TINY, tiny_weights, tensors=(arr, keep))
    assert st == L.MK_EINVAL and h is None
    assert "on_device" in so.mk_last_error().decode()


def test_loader_rejects_shape_missing_unknown_duplicate(so, tiny_weights):
    w = dict(tiny_weights)
    w["layers.0.dn.wq"] = w["layers.0.dn.wq"][:, :128]
    assert _load(so, W.TINY, w)[0] == L.MK_ESHAPE
    w = dict(tiny_weights)
    del w["layers.2.ffn.wd"]
    assert _load(so, W.TINY, w)[0] == L.MK_ESHAPE
    w = dict(tiny_weights)
    w["layers.0.bogus"] = w["lnf"]
    assert _load(so, W.TINY, w)[0] == L.MK_ESHAPE
    arr, keep = L.make_tensors(tiny_weights)
    arr2 = (L.MkTensor * (len(arr) + 1))(*arr, arr[5])
    assert _load(so, W.TINY, None, tensors=(arr2, keep))[0] == L.MK_ESHAPE
    # attention tensors in a DeltaNet layer are unknown
    w = dict(tiny_weights)
    w["layers.0.attn.wq"] = w["layers.3.attn.wq"]
    assert _load(so, W.TINY, w)[0] == L.MK_ESHAPE


def test_loader_rejects_bad_arena_before_touching_the_device(so, tiny_weights):
    need = L.mk_required_bytes(W.TINY)
    assert _load(so, W.TINY, tiny_weights, arena=None, nbytes=need)[0] == L.MK_EINVAL
    assert _load(so, W.TINY, tiny_weights, arena=4096 + 8, nbytes=need)[0] == L.MK_EINVAL      # misaligned
    assert _load(so, W.TINY, tiny_weights, arena=4096, nbytes=need - 256)[0] == L.MK_EINVAL     # too small
    st = so.mk_load_weights(None, None, 0, None, 0, None, None)
    assert st == L.MK_EINVAL


def test_calls_on_unloaded_model_are_rejected(so):
    buf = ctypes.c_void_p(4096)
    assert so.mk_prefill(None, buf, 4, buf, None, None) == L.MK_ESTATE
    assert so.mk_decode_step(None, buf, 1, buf, None, None, None) == L.MK_ESTATE
    assert so.mk_decode_step_static(None, buf, 1, buf, None, None, None) == L.MK_ESTATE
    assert so.mk_reset_state(None, None) == L.MK_ESTATE
    assert so.mk_select_seq(None, 0) == L.MK_ESTATE
    assert so.mk_set_prefill_blocks(None, 2) == L.MK_ESTATE
    seqs = (ctypes.c_int32 * 2)(0, 1)
    assert so.mk_decode_batch(None, seqs, 2, buf, buf, None, None) == L.MK_ESTATE
    pos = ctypes.c_int32(0)
    assert so.mk_sync_status(None, None, ctypes.byref(pos)) == L.MK_ESTATE
    so.mk_free(None)  # no-op


def test_static_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    m = re.search(r"MK_STATIC_SCRATCH_BYTES\s*=\s*(\d+)\s*<<\s*(\d+)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == L.MK_STATIC_SCRATCH_BYTES
