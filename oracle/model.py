"""Whole-model CPU oracle: prefill, decode and multi-token verify of the hybrid decoder.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Structure (launch page "OS Megakernel that match M5 Max Tok/w at 2x the
Throughput on RTX 3090", section "Why nobody had done this yet?": DeltaNet
layers interleaved with full-attention layers).  Readings where the pages are
silent: every layer is pre-norm with a residual stream, x += mixer(RMSNorm(x))
then x += FFN(RMSNorm(x)); a final RMSNorm feeds an LM head tied to the token
embedding; the greedy token is the lowest index among the maximal logits.

Every token is processed in order.  For speed the loops run layer by layer
over a block of tokens, which changes nothing: the projections act on each
token separately, and the sequence mixers (short conv, delta rule, causal
attention) walk the tokens in order.

Precision.  ``EXACT`` rounds nothing beyond the bfloat16 weights.  ``C2`` (the
contract the GPU path implements) also stores the attention K and V cache in
bfloat16, and keeps every activation in full precision in every mode: the
weights and the KV cache are what the forward pass streams from memory, the
activations are a few kilobytes per token.  ``C1`` additionally rounds, during
prefill, the activation operand of every projection, the attention queries and
the attention probabilities (normalised to the row maximum, rounded before they
weight V; the denominator sums the unrounded values) to bfloat16.  On the
seeded random-init models C1 is not a usable parity contract: a relative
perturbation of 1e-7 at the input changes its prefill logits by about 1%
(each perturbation flips some bfloat16 roundings, which cascade), while under
C2 the same perturbation changes them by about 2e-5.  The LM head input is
never rounded.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Tuple

import numpy as np

from workloads import ModelConfig, DELTANET
from .ops import (round_bf16, kv_q8_rows, bf16_bits_to_f64, rmsnorm, silu, l2norm, gates, causal_conv,
                  delta_rule_step, rope, gated_rmsnorm, swiglu, argmax_lowest)


@dataclass(frozen=True)
class Contract:
    kv_bf16: bool       # K and V are stored in the cache as bfloat16
    prefill_bf16: bool  # prefill rounds projection operands, attention queries and probabilities


EXACT = Contract(kv_bf16=False, prefill_bf16=False)
C1 = Contract(kv_bf16=True, prefill_bf16=True)
C2 = Contract(kv_bf16=True, prefill_bf16=False)


def attention_causal(Q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, q_pos: np.ndarray,
                     round_p: bool, block: int = 256) -> np.ndarray:
    """Causal softmax attention of the queries Q at positions q_pos over the cache.

    Q: [T, n_q, d]; Kc, Vc: [>= max(q_pos)+1, n_kv, d].  Query head i reads kv head
    i*n_kv//n_q.  Each query attends to keys 0..q_pos[t]; probabilities are
    exp(s - max s), optionally rounded to bfloat16 before weighting V, divided by
    the sum of the unrounded values.  Queries are taken in blocks only so that the
    scores of a block come from one matrix product."""
    T, n_q, d = Q.shape
    n_kv = Kc.shape[1]
    out = np.zeros_like(Q)
    scale = 1.0 / np.sqrt(d)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        end = int(q_pos[t1 - 1]) + 1
        keys = np.arange(end)
        mask = keys[None, :] <= q_pos[t0:t1, None]
        for i in range(n_q):
            j = i * n_kv // n_q
            s = (Q[t0:t1, i, :] @ Kc[:end, j, :].T) * scale
            s = np.where(mask, s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            w = round_bf16(e) if round_p else e
            out[t0:t1, i, :] = (w @ Vc[:end, j, :]) / e.sum(axis=1, keepdims=True)
    return out


class OracleModel:
    """Float64 forward pass of the synthetic hybrid decoder with its recurrent state."""

    def __init__(self, cfg: ModelConfig, weight_bits: Dict[str, np.ndarray], contract: Contract = C2):
        self.cfg = cfg
        self.contract = contract
        self.w = {name: bf16_bits_to_f64(bits) for name, bits in weight_bits.items()}
        self.reset()

    # ------------------------------------------------------------------ state
    def reset(self) -> None:
        c = self.cfg
        self.pos = 0
        self.S: Dict[int, np.ndarray] = {}
        self.conv: Dict[int, np.ndarray] = {}
        self.Kc: Dict[int, np.ndarray] = {}
        self.Vc: Dict[int, np.ndarray] = {}
        for i, kind in enumerate(c.layer_kinds):
            if kind == DELTANET:
                self.S[i] = np.zeros((c.dn_heads, c.dn_dv, c.dn_dk))
                self.conv[i] = np.zeros((c.conv_k - 1, c.conv_channels))
            else:
                self.Kc[i] = np.zeros((c.max_ctx, c.at_kv_heads, c.at_head_dim))
                self.Vc[i] = np.zeros((c.max_ctx, c.at_kv_heads, c.at_head_dim))

    def snapshot(self):
        return (self.pos, {i: s.copy() for i, s in self.S.items()}, {i: h.copy() for i, h in self.conv.items()})

    def restore(self, snap) -> None:
        # Cache rows at positions >= pos are never read before they are rewritten.
        self.pos, S, conv = snap
        self.S = {i: s.copy() for i, s in S.items()}
        self.conv = {i: h.copy() for i, h in conv.items()}

    # ------------------------------------------------------------------ layers
    def _deltanet(self, li: int, h: np.ndarray, rnd) -> np.ndarray:
        c, w, p = self.cfg, self.w, f"layers.{li}.dn."
        T = h.shape[0]
        nh, dk, dv = c.dn_heads, c.dn_dk, c.dn_dv
        qkv = np.concatenate([h @ w[p + "wq"].T, h @ w[p + "wk"].T, h @ w[p + "wv"].T], axis=1)
        z = (h @ w[p + "wz"].T).reshape(T, nh, dv)
        alpha, beta = gates(h @ w[p + "wa"].T, h @ w[p + "wb"].T)          # [T, nh]
        pre, self.conv[li] = causal_conv(self.conv[li], qkv, w[p + "conv"])
        act = silu(pre)
        q = l2norm(act[:, :c.dn_qk].reshape(T, nh, dk), c.l2_eps)
        k = l2norm(act[:, c.dn_qk:2 * c.dn_qk].reshape(T, nh, dk), c.l2_eps)
        v = act[:, 2 * c.dn_qk:].reshape(T, nh, dv)
        S = self.S[li]
        o = np.zeros((T, nh, dv))
        for t in range(T):
            for hd in range(nh):
                S[hd], o[t, hd] = delta_rule_step(S[hd], k[t, hd], v[t, hd], q[t, hd],
                                                  alpha[t, hd], beta[t, hd])
        y = gated_rmsnorm(o, z, w[p + "gnorm"], c.rms_eps).reshape(T, nh * dv)
        return rnd(y) @ w[p + "wo"].T

    def _attention(self, li: int, h: np.ndarray, prefill: bool, rnd) -> np.ndarray:
        c, w, p = self.cfg, self.w, f"layers.{li}.attn."
        T = h.shape[0]
        d = c.at_head_dim
        pos = self.pos + np.arange(T)
        q = rope((h @ w[p + "wq"].T).reshape(T, c.at_q_heads, d), pos[:, None], c.rope_theta)
        k = rope((h @ w[p + "wk"].T).reshape(T, c.at_kv_heads, d), pos[:, None], c.rope_theta)
        v = (h @ w[p + "wv"].T).reshape(T, c.at_kv_heads, d)
        if c.kv_quant:                  # 8-bit codes, power-of-two scale per cached row
            k, v = kv_q8_rows(k)[2], kv_q8_rows(v)[2]
        elif self.contract.kv_bf16:
            k, v = round_bf16(k), round_bf16(v)
        self.Kc[li][self.pos:self.pos + T] = k
        self.Vc[li][self.pos:self.pos + T] = v
        round_mm = prefill and self.contract.prefill_bf16
        if round_mm:
            q = round_bf16(q)
        o = attention_causal(q, self.Kc[li], self.Vc[li], pos, round_p=round_mm)
        return rnd(o.reshape(T, c.at_q_heads * d)) @ w[p + "wo"].T

    # ------------------------------------------------------------------ forward
    def forward(self, tokens, prefill: bool, logits_for: str = "last") -> np.ndarray:
        """Run tokens through all layers from the current state and advance it.

        logits_for: 'last' -> [V] logits of the last token, 'all' -> [T, V], 'none' -> None."""
        c, w = self.cfg, self.w
        tokens = np.asarray(tokens, dtype=np.int64)
        T = tokens.shape[0]
        if T == 0:
            raise ValueError("no tokens")
        if self.pos + T > c.max_ctx:
            raise ValueError("context overflow")
        if np.any(tokens < 0) or np.any(tokens >= c.vocab):
            raise ValueError("token id out of range")
        rnd = round_bf16 if (prefill and self.contract.prefill_bf16) else (lambda a: a)
        x = w["embed"][tokens].copy()
        for li, kind in enumerate(c.layer_kinds):
            p = f"layers.{li}."
            h = rnd(rmsnorm(x, w[p + "ln1"], c.rms_eps))
            if kind == DELTANET:
                x = x + self._deltanet(li, h, rnd)
            else:
                x = x + self._attention(li, h, prefill, rnd)
            h2 = rnd(rmsnorm(x, w[p + "ln2"], c.rms_eps))
            m = rnd(swiglu(h2 @ w[p + "ffn.wg"].T, h2 @ w[p + "ffn.wu"].T))
            x = x + m @ w[p + "ffn.wd"].T
        self.pos += T
        if logits_for == "none":
            return None
        rows = x[-1:] if logits_for == "last" else x
        logits = rmsnorm(rows, w["lnf"], c.rms_eps) @ w["embed"].T
        return logits[0] if logits_for == "last" else logits

    def prefill(self, tokens) -> np.ndarray:
        """Process a prompt; returns the logits of its last position."""
        return self.forward(tokens, prefill=True, logits_for="last")

    def decode(self, token: int) -> np.ndarray:
        """One greedy decode step consuming ``token``; returns its logits."""
        return self.forward([int(token)], prefill=False, logits_for="last")

    def verify(self, tokens) -> Tuple[List[int], int, np.ndarray]:
        """Verify forward: tokens = [t0 (last accepted), d1..d_{n-1} (drafts)].

        Returns (greedy token after each position, n_accepted, logits [n, V]).
        n_accepted = 1 + the length of the longest draft prefix that equals the
        greedy choices; the state is left after exactly the accepted tokens
        t0, d1, ..., d_{n_accepted-1}, so the next forward starts from
        greedy[n_accepted-1]."""
        snap = self.snapshot()
        logits = self.forward(tokens, prefill=False, logits_for="all")
        greedy = [argmax_lowest(row) for row in logits]
        n_acc = 1
        while n_acc < len(tokens) and int(tokens[n_acc]) == greedy[n_acc - 1]:
            n_acc += 1
        self.restore(snap)
        self.forward(list(tokens[:n_acc]), prefill=False, logits_for="none")
        return greedy, n_acc, logits

    def generate(self, prompt, steps: int):
        """Prefill then ``steps`` greedy decode steps.  Returns (tokens [steps+1], logits [steps+1, V])."""
        logits = [self.prefill(prompt)]
        toks = [argmax_lowest(logits[0])]
        for _ in range(steps):
            logits.append(self.decode(toks[-1]))
            toks.append(argmax_lowest(logits[-1]))
        return np.array(toks, dtype=np.int64), np.stack(logits)
