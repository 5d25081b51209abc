"""Persistent single-launch forward pass of a hybrid Gated-DeltaNet + attention decoder
on AMD Instinct MI355X (gfx950).

The computation lives in the HIP library libmk.so (C ABI: include/mk.h); ``lib``
is its thin ctypes binding.  Build it with ``python -m
hybrid_deltanet_attention_persistent_amd.build``.  Nothing here computes the
model on the host: without the library every entry point raises ImportError.
"""
from .lib import (  # noqa: F401
    Model, MkError, load_library, mk_required_bytes, mk_load_weights, mk_reset_state, mk_prefill,
    mk_decode_step, mk_decode_step_static, mk_sync_status, mk_free, mk_lookup_draft, mk_generate_lookup,
    mk_select_seq, mk_decode_batch, mk_set_prefill_blocks, make_config, make_tensors, LIB_PATH, EXPORTED,
)
