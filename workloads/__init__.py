"""Seeded synthetic inputs for the hybrid Gated-DeltaNet + attention decoder.

This module is the only code that both the CPU oracle and the GPU path use.  It
holds model shapes, workload shapes and seeded random draws (weights, prompts,
draft tokens), and nothing of the forward pass itself.

Model shapes follow the launch page "OS Megakernel that match M5 Max Tok/w at 2x
the Throughput on RTX 3090" (section "Why nobody had done this yet?": 24 layers,
18 DeltaNet layers and 6 full-attention layers, interleaved).  The pages name no
head counts or widths; the two shapes below are the tiny 4-layer hybrid and a
0.8B-class 24-layer hybrid with the [D, D, D, A] x 6 pattern.

Random draws: every tensor is drawn from its own numpy PCG64 stream seeded with
``SeedSequence([seed, tensor_index])`` over the canonical tensor list, so a
tensor's values do not depend on which other tensors exist.  Matrices, the
embedding and the conv taps are N(0, std) float32 draws rounded to bfloat16
(round to nearest even).  Norm gains are 1 unless ``gain_std`` > 0, in which
case they are 1 + N(0, gain_std).  No biases exist.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

DELTANET = "D"
ATTENTION = "A"


@dataclass(frozen=True)
class ModelConfig:
    name: str
    layer_kinds: Tuple[str, ...]
    hidden: int
    vocab: int
    ffn: int
    dn_heads: int
    dn_dk: int
    dn_dv: int
    conv_k: int
    at_q_heads: int
    at_kv_heads: int
    at_head_dim: int
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    l2_eps: float = 1e-6
    tied_embedding: bool = True
    max_ctx: int = 8448
    prefill_chunk: int = 64
    max_verify: int = 5
    kv_quant: int = 0          # 0: K/V cache in bfloat16; 1: 8-bit codes with a power-of-two scale per row
    n_seq: int = 1             # sequences held at once (batch decode serves up to this many per launch)

    @property
    def n_layers(self) -> int:
        return len(self.layer_kinds)

    @property
    def dn_qk(self) -> int:  # width of the q (and k) projection of a DeltaNet layer
        return self.dn_heads * self.dn_dk

    @property
    def dn_v(self) -> int:  # width of the v (and z) projection of a DeltaNet layer
        return self.dn_heads * self.dn_dv

    @property
    def conv_channels(self) -> int:  # q, k and v channels pass through the short conv
        return 2 * self.dn_qk + self.dn_v


def _pattern(n_groups: int) -> Tuple[str, ...]:
    return (DELTANET, DELTANET, DELTANET, ATTENTION) * n_groups


TINY = ModelConfig(
    name="tiny-hybrid-4L", layer_kinds=_pattern(1), hidden=256, vocab=4096, ffn=768,
    dn_heads=4, dn_dk=64, dn_dv=64, conv_k=4,
    at_q_heads=4, at_kv_heads=2, at_head_dim=64, max_ctx=64)

HYBRID_24L = ModelConfig(
    name="hybrid-24L-h1024", layer_kinds=_pattern(6), hidden=1024, vocab=151936, ffn=3584,
    dn_heads=8, dn_dk=128, dn_dv=128, conv_k=4,
    at_q_heads=8, at_kv_heads=2, at_head_dim=128, max_ctx=8448)

# the same models with the 8-bit K/V cache (codes + a power-of-two scale per cached row)
TINY_Q8 = dataclasses.replace(TINY, name="tiny-hybrid-4L-q8", kv_quant=1)
HYBRID_24L_Q8 = dataclasses.replace(HYBRID_24L, name="hybrid-24L-h1024-q8", kv_quant=1)

MODELS = {m.name: m for m in (TINY, HYBRID_24L, TINY_Q8, HYBRID_24L_Q8)}


@dataclass(frozen=True)
class Workload:
    """One run shape: a prompt, then greedy decode steps (or verify forwards)."""
    name: str
    model: ModelConfig
    prompt_len: int
    decode_steps: int
    verify_width: int = 1  # 1 = plain decode; 5 = 1 accepted + 4 draft tokens per forward
    weight_seed: int = 0
    prompt_seed: int = 1
    draft_seed: int = 2


WORKLOADS = {
    "tiny-pp16-tg16": Workload("tiny-pp16-tg16", TINY, 16, 16),
    "24L-pp520-tg128": Workload("24L-pp520-tg128", HYBRID_24L, 520, 128),
    "24L-pp520": Workload("24L-pp520", HYBRID_24L, 520, 0),
    "24L-pp8192-tg128": Workload("24L-pp8192-tg128", HYBRID_24L, 8192, 128),
    "24L-pp520-verify5": Workload("24L-pp520-verify5", HYBRID_24L, 520, 128, verify_width=5),
    # 8-bit KV cache: a context long enough that decode reads cached rows past the prefetched ones
    "24L-q8-pp8192-tg32": Workload("24L-q8-pp8192-tg32", HYBRID_24L_Q8, 8192, 32),
}


def tensor_specs(cfg: ModelConfig) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Canonical tensor list: (name, shape, kind) with kind 'mat' or 'gain'.

    Matrices are stored [out, in] (row-major, one output per row)."""
    H, V, I = cfg.hidden, cfg.vocab, cfg.ffn
    specs: List[Tuple[str, Tuple[int, ...], str]] = [("embed", (V, H), "mat")]
    for i, kind in enumerate(cfg.layer_kinds):
        p = f"layers.{i}."
        specs.append((p + "ln1", (H,), "gain"))
        if kind == DELTANET:
            specs += [
                (p + "dn.wq", (cfg.dn_qk, H), "mat"),
                (p + "dn.wk", (cfg.dn_qk, H), "mat"),
                (p + "dn.wv", (cfg.dn_v, H), "mat"),
                (p + "dn.wz", (cfg.dn_v, H), "mat"),
                (p + "dn.wa", (cfg.dn_heads, H), "mat"),
                (p + "dn.wb", (cfg.dn_heads, H), "mat"),
                (p + "dn.conv", (cfg.conv_channels, cfg.conv_k), "mat"),
                (p + "dn.gnorm", (cfg.dn_dv,), "gain"),
                (p + "dn.wo", (H, cfg.dn_v), "mat"),
            ]
        else:
            specs += [
                (p + "attn.wq", (cfg.at_q_heads * cfg.at_head_dim, H), "mat"),
                (p + "attn.wk", (cfg.at_kv_heads * cfg.at_head_dim, H), "mat"),
                (p + "attn.wv", (cfg.at_kv_heads * cfg.at_head_dim, H), "mat"),
                (p + "attn.wo", (H, cfg.at_q_heads * cfg.at_head_dim), "mat"),
            ]
        specs += [
            (p + "ln2", (H,), "gain"),
            (p + "ffn.wg", (I, H), "mat"),
            (p + "ffn.wu", (I, H), "mat"),
            (p + "ffn.wd", (H, I), "mat"),
        ]
    specs.append(("lnf", (H,), "gain"))
    return specs


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_weights(cfg: ModelConfig, seed: int = 0, std: float = 0.02,
                 gain_std: float = 0.0) -> Dict[str, np.ndarray]:
    """All weights as bfloat16 bit patterns (uint16 arrays), keyed by canonical name."""
    out: Dict[str, np.ndarray] = {}
    for idx, (name, shape, kind) in enumerate(tensor_specs(cfg)):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, idx])))
        if kind == "mat":
            vals = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
        elif gain_std > 0:
            vals = np.float32(1.0) + rng.standard_normal(shape, dtype=np.float32) * np.float32(gain_std)
        else:
            vals = np.ones(shape, dtype=np.float32)
        out[name] = f32_to_bf16_bits(vals)
    return out


def make_prompt(cfg: ModelConfig, n: int, seed: int = 1) -> np.ndarray:
    """n token ids drawn uniformly from [0, vocab)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed])))
    return rng.integers(0, cfg.vocab, size=n, dtype=np.int64).astype(np.int32)


def make_drafts(cfg: ModelConfig, n_forwards: int, width: int = 5, seed: int = 2) -> np.ndarray:
    """Draft token ids for verify forwards: [n_forwards, width - 1], uniform in [0, vocab)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed])))
    return rng.integers(0, cfg.vocab, size=(n_forwards, width - 1), dtype=np.int64).astype(np.int32)


def param_count(cfg: ModelConfig) -> int:
    return int(sum(int(np.prod(s)) for _, s, _ in tensor_specs(cfg)))


__all__ = [
    "ModelConfig", "Workload", "TINY", "HYBRID_24L", "TINY_Q8", "HYBRID_24L_Q8", "MODELS", "WORKLOADS", "DELTANET", "ATTENTION",
    "tensor_specs", "make_weights", "make_prompt", "make_drafts", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "param_count",
]
