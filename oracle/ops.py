"""Elementary operations of the hybrid decoder, written from their definitions in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Readings of the pages used here (the launch page "OS Megakernel that match M5
Max Tok/w at 2x the Throughput on RTX 3090" names the blocks but prints no
equation):

* RMSNorm: x / sqrt(mean(x^2) + eps) * gain, eps inside the square root.
* DeltaNet recurrence ("linear attention with a learned recurrence", section
  "Why nobody had done this yet?"): the gated delta rule
  S <- alpha * S (I - beta k k^T) + beta v k^T with S of shape [d_v, d_k]; the
  state is updated first and then read out as o = S q.  With this orientation a
  unit key k written with alpha = beta = 1 reads back its value v.
* Gates: beta = sigmoid(b), alpha = exp(-softplus(a)).
* Short causal conv: depthwise over time, the last tap multiplies the current
  token, zero history before the first token, SiLU after the conv.
* q and k are L2-normalised per head after the conv: x / sqrt(sum(x^2) + eps).
* Gated RMSNorm of the DeltaNet output per head: RMSNorm(o) * gain * SiLU(z).
* Attention ("full attention fuses QKV, RoPE, causal softmax, and output
  projection", section "We wrote a single CUDA kernel ..."): grouped-query
  attention with contiguous groups, rotate-half RoPE over the full head
  dimension with inverse frequencies theta^(-2i/d), positions from 0, softmax
  scale 1/sqrt(d).
* SwiGLU feed-forward: W_d (SiLU(W_g h) * (W_u h)).
* Greedy decoding takes the lowest index among equal maxima.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_bf16", "bf16_bits_to_f64", "rmsnorm", "sigmoid", "silu", "softplus", "l2norm",
    "gates", "causal_conv", "delta_rule_step", "delta_rule_step_literal", "delta_rule_chunked",
    "rope", "rope_inv_freq", "attention_masked_dense", "attention_one_query", "gated_rmsnorm",
    "swiglu", "argmax_lowest", "kv_q8_rows",
]


# ----------------------------------------------------------------------------- rounding
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 the way an FP32 datapath does.

    The value is first rounded to float32 (nearest, ties to even), then its low
    16 mantissa bits are dropped with round-to-nearest-even on the dropped half.
    Returned as float64 holding the bfloat16 value."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    hi = bits >> np.uint64(16)
    lo = bits & np.uint64(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint64(1)) == 1))
    hi = hi + up.astype(np.uint64)
    out = (hi << np.uint64(16)).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)


def kv_q8_rows(x: np.ndarray):
    """8-bit KV-cache quantisation with one power-of-two scale per row (the last axis).

    The pages name an 8-bit KV cache ("q8" on the Korean update page, limits section; block-quantised
    KV caches on the RTX 3090 tag page) without defining its format; the reading used here: per
    cached row (one position of one KV head), in float32, a = max |x_i|, e = the smallest integer
    >= -126 with a <= 127 * 2^e (so e = -126 for an all-zero or tiny row, and every nonzero stored
    value is a normal number; e fits one signed byte), codes q_i = round-half-even(x_i * 2^-e) in
    [-127, 127], stored value q_i * 2^e.  A power-of-two scale keeps every stored value exactly a
    bfloat16 number (|q| <= 127 needs 7 significant bits).

    Returns (codes int8 [..., d], exponents int32 [...], values float64 [..., d])."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    a = np.max(np.abs(x32), axis=-1)
    _, E = np.frexp(a.astype(np.float64))                   # a in [2^(E-1), 2^E), E = 0 for a == 0
    E = E.astype(np.int64)
    e = np.where(a.astype(np.float64) <= np.ldexp(127.0, E - 7), E - 7, E - 6)
    e = np.maximum(np.where(a == 0, -126, e), -126)
    scaled = np.ldexp(x32.astype(np.float64), -e[..., None])  # exact: a power-of-two rescaling
    q = np.clip(np.rint(scaled), -127, 127).astype(np.int64)  # rint: ties to even
    return q.astype(np.int8), e.astype(np.int32), np.ldexp(q.astype(np.float64), e[..., None])


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- pointwise
def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square norm over the last axis, eps inside the square root."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def sigmoid(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(x: np.ndarray) -> np.ndarray:
    return x * sigmoid(x)


def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def l2norm(x: np.ndarray, eps: float) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gates(a: np.ndarray, b: np.ndarray):
    """Decay alpha = exp(-softplus(a)) in (0, 1) and write strength beta = sigmoid(b)."""
    return np.exp(-softplus(a)), sigmoid(b)


# ----------------------------------------------------------------------------- short conv
def causal_conv(history: np.ndarray, inputs: np.ndarray, taps: np.ndarray):
    """Depthwise causal conv over time, one output per input row.

    history: [K-1, C] previous pre-conv inputs, oldest first (zeros at the start).
    inputs:  [T, C] pre-conv inputs of the new tokens.
    taps:    [C, K]; tap K-1 multiplies the current token, tap 0 the token K-1 steps back.
    Returns (outputs [T, C] before the SiLU, new history [K-1, C])."""
    K = taps.shape[1]
    full = np.concatenate([history, inputs], axis=0)  # [K-1+T, C]
    T = inputs.shape[0]
    out = np.zeros_like(inputs)
    for i in range(K):
        out += taps[:, i][None, :] * full[i:i + T]
    return out, full[T:].copy()


# ----------------------------------------------------------------------------- delta rule
def delta_rule_step(S: np.ndarray, k: np.ndarray, v: np.ndarray, q: np.ndarray,
                    alpha: float, beta: float):
    """One gated delta-rule step and its read-out, in the factored form.

    alpha*S*(I - beta*k*k^T) + beta*v*k^T equals alpha*S + (beta*(v - alpha*S k)) k^T.
    S: [d_v, d_k].  Returns (new S, o = S_new q)."""
    u = beta * (v - alpha * (S @ k))
    S_new = alpha * S + np.outer(u, k)
    return S_new, S_new @ q


def delta_rule_step_literal(S: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: float, beta: float):
    """The same update multiplied out as written: alpha*S*(I - beta*k*k^T) + beta*v*k^T."""
    d_k = k.shape[0]
    return alpha * S @ (np.eye(d_k) - beta * np.outer(k, k)) + beta * np.outer(v, k)


def delta_rule_chunked(S0: np.ndarray, K: np.ndarray, V: np.ndarray, Q: np.ndarray,
                       log_alpha: np.ndarray, beta: np.ndarray, chunk: int):
    """The delta rule over T tokens processed in chunks, unrolled in closed form.

    Within a chunk starting from state S0, with G_i the cumulative sum of log
    alpha over the chunk, the recurrence unrolls to
        S_i = e^{G_i} S0 + sum_{j<=i} e^{G_i - G_j} u_j k_j^T,
        u_i = beta_i (v_i - e^{G_i} S0 k_i) - beta_i sum_{j<i} e^{G_i - G_j} (k_i . k_j) u_j,
    i.e. (I + A) U = B with A strictly lower triangular, solved by forward
    substitution; the outputs are o_i = S_i q_i.
    K, Q: [T, d_k]; V: [T, d_v]; log_alpha, beta: [T].  Returns (O [T, d_v], S_T)."""
    T = K.shape[0]
    S = S0.copy()
    O = np.zeros((T, V.shape[1]))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        k, v, q = K[c0:c1], V[c0:c1], Q[c0:c1]
        b = beta[c0:c1]
        G = np.cumsum(log_alpha[c0:c1])
        n = c1 - c0
        incl_mask = np.tril(np.ones((n, n), dtype=bool))
        decay = np.exp(np.where(incl_mask, G[:, None] - G[None, :], -np.inf))  # e^{G_i-G_j}, j <= i
        lower = np.tril(np.ones((n, n)), -1)
        A = (b[:, None] * decay * (k @ k.T)) * lower
        B = b[:, None] * (v - np.exp(G)[:, None] * (k @ S.T))
        U = np.zeros_like(B)
        for i in range(n):                                 # forward substitution of (I + A) U = B
            U[i] = B[i] - A[i, :i] @ U[:i]
        O[c0:c1] = np.exp(G)[:, None] * (q @ S.T) + (decay * (q @ k.T)) @ U
        S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * U).T @ k
    return O, S


# ----------------------------------------------------------------------------- attention
def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    return theta ** (-np.arange(0, d // 2, dtype=np.float64) * 2.0 / d)


def rope(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding.  x: [..., d]; pos: scalar or array broadcastable to x[..., 0]."""
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention_one_query(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, round_p: bool = False) -> np.ndarray:
    """Causal softmax attention of one position over the keys 0..p of the cache.

    q: [n_q, d]; Kc, Vc: [p+1, n_kv, d]; query head i reads kv head i*n_kv//n_q.
    With round_p, the normalised-to-max probabilities exp(s - max s) are rounded to
    bfloat16 before weighting V, while the denominator sums the unrounded values."""
    n_q, d = q.shape
    n_kv = Kc.shape[1]
    o = np.zeros_like(q)
    for i in range(n_q):
        j = i * n_kv // n_q
        s = (Kc[:, j, :] @ q[i]) / np.sqrt(d)
        e = np.exp(s - np.max(s))
        w = round_bf16(e) if round_p else e
        o[i] = (w @ Vc[:, j, :]) / np.sum(e)
    return o


def attention_masked_dense(Q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Brute-force causal attention over a whole sequence: full T x T scores, masked softmax.

    Q: [T, n_q, d]; K, V: [T, n_kv, d]."""
    T, n_q, d = Q.shape
    n_kv = K.shape[1]
    out = np.zeros_like(Q)
    mask = np.tril(np.ones((T, T), dtype=bool))
    for i in range(n_q):
        j = i * n_kv // n_q
        s = (Q[:, i, :] @ K[:, j, :].T) / np.sqrt(d)
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        out[:, i, :] = p @ V[:, j, :]
    return out


# ----------------------------------------------------------------------------- misc
def gated_rmsnorm(o: np.ndarray, z: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm of o, times a gain shared by the heads, times SiLU(z).  o, z: [..., d_v]."""
    return rmsnorm(o, gain, eps) * silu(z)


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    return silu(g) * u


def argmax_lowest(logits: np.ndarray) -> int:
    """Greedy token: the lowest index among the maxima.  Non-finite logits are an error."""
    if not np.all(np.isfinite(logits)):
        raise FloatingPointError("non-finite logits")
    return int(np.argmax(logits))
