"""Benchmark: batch-1 greedy decode (tg128 after a pp520 prompt) of the 24-layer hybrid
Gated-DeltaNet + attention decoder on one MI355X, through the C ABI.

One step = reset the state, prefill the 520-token synthetic prompt (one launch),
then 128 greedy decode steps chained on the device (one launch each).  Prints one
JSON line: decode tok/s (the headline), prefill tok/s, the roofline of the decode
kernel measured with HIP events on the launch stream, and the CPU oracle timed on
this host as a reported baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
BASELINE_DECODE_TOKS = 413.0    # the pages' megakernel decode figure (tg128, RTX 3090)
WORKLOAD_CHOICES = ["24L-pp520-tg128", "24L-pp8192-tg128", "tiny-pp16-tg16"]


def decode_bytes_per_token(cfg: W.ModelConfig, ctx: float) -> dict:
    """Algorithmic HBM bytes of one decode step at context length ctx (before the new token).

    Weights: every matrix once (the tied embedding once, as the LM head; plus one
    embedding row), conv taps and gains.  State: each DeltaNet state read and
    written once, the conv history read, the KV cache read once per layer and the
    new K, V written."""
    n_dn = sum(1 for k in cfg.layer_kinds if k == "D")
    n_at = cfg.n_layers - n_dn
    H, I = cfg.hidden, cfg.ffn
    dn_mat = (2 * cfg.dn_qk + 2 * cfg.dn_v + 2 * cfg.dn_heads) * H + H * cfg.dn_v
    at_mat = (cfg.at_q_heads + 2 * cfg.at_kv_heads) * cfg.at_head_dim * H + H * cfg.at_q_heads * cfg.at_head_dim
    ffn = 3 * H * I
    weights = 2 * (n_dn * dn_mat + n_at * at_mat + cfg.n_layers * ffn + cfg.vocab * H + H)
    small = 4 * (n_dn * (cfg.conv_channels * cfg.conv_k + cfg.dn_dv) + 2 * cfg.n_layers * H + H)
    state = n_dn * cfg.dn_heads * cfg.dn_dv * cfg.dn_dk * 4 * 2
    conv = n_dn * cfg.conv_channels * 4 * (cfg.conv_k - 1 + 1)
    kv_row = cfg.at_kv_heads * cfg.at_head_dim * 2 * 2      # K and V of one position, bf16
    kv = n_at * kv_row * (ctx + 1)
    return dict(weights=weights, all=weights + small + state + conv + kv)


def prefill_flops(cfg: W.ModelConfig, T: int, p0: int = 0) -> dict:
    """Algorithmic FLOPs of one prefill of T tokens starting at position p0.

    Projections: 2 T x (every weight matrix but the embedding); causal attention: QK^T and
    P.V over keys 0..p for each query (4 hd (p + 1) per query and head); delta rule:
    6 dk dv per token and head (decay, S k, rank-1 update, S q); LM head of the last row."""
    n_dn = sum(1 for k in cfg.layer_kinds if k == "D")
    n_at = cfg.n_layers - n_dn
    H, I = cfg.hidden, cfg.ffn
    dn_mat = (2 * cfg.dn_qk + 2 * cfg.dn_v + 2 * cfg.dn_heads) * H + H * cfg.dn_v
    at_mat = (cfg.at_q_heads + 2 * cfg.at_kv_heads) * cfg.at_head_dim * H + H * cfg.at_q_heads * cfg.at_head_dim
    proj = 2.0 * T * (n_dn * dn_mat + n_at * at_mat + cfg.n_layers * 3 * H * I)
    keys = sum(p0 + t + 1 for t in range(T))
    att = 4.0 * cfg.at_head_dim * keys * cfg.at_q_heads * n_at
    delta = 6.0 * cfg.dn_dk * cfg.dn_dv * cfg.dn_heads * T * n_dn
    lm = 2.0 * cfg.vocab * H
    return dict(projections=proj, attention=att, delta_rule=delta, lm_head=lm, all=proj + att + delta + lm)


def source_hash() -> str:
    h = hashlib.sha256()
    for f in ("mk_forward_kernel.h", "mk_forward.hip", "mk_layout.h"):
        h.update(open(os.path.join(ROOT, "hybrid_deltanet_attention_persistent_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("source_hash") != source_hash() or d.get("kernel") != kernel:
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(seconds: float = 15.0) -> dict:
    """The oracle as it stands, single-threaded, on a bounded sample of the decode workload."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    from oracle import OracleModel, C2, argmax_lowest
    cfg = W.HYBRID_24L
    weights = W.make_weights(cfg, seed=0)
    prompt = W.make_prompt(cfg, 8, seed=1)
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        m = OracleModel(cfg, weights, C2)
        del weights
        t = argmax_lowest(m.prefill(prompt))
        n, t0 = 0, time.perf_counter()
        while True:
            t = argmax_lowest(m.decode(t))
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds or n >= 200:
                break
    finally:
        if ctx is not None:
            ctx.unregister() if hasattr(ctx, "unregister") else None
    return {"value": n / el, "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} greedy decode steps of the 24-layer model after an 8-token prompt, float64, "
                      f"one thread ({el:.1f} s)"}


def extras(model, cfg, stream) -> dict:
    """Secondary measurements on the same model: multi-token verify forwards after the pp520
    prompt (1 accepted + 4 seeded random drafts each, state rolled back to the accepted prefix),
    and decode at long context after an 8192-token prompt."""
    import torch
    dev = stream.device
    out = {}
    # verify: 64 forwards of [last accepted, 4 drafts]
    prompt = torch.tensor(W.make_prompt(cfg, 520, seed=1), dtype=torch.int32, device=dev)
    drafts = torch.tensor(W.make_drafts(cfg, 64, 5, seed=2), dtype=torch.int32, device=dev)
    am = torch.zeros((64, 5), dtype=torch.int32, device=dev)
    nacc = torch.zeros(64, dtype=torch.int32, device=dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    model.reset()
    model.prefill(prompt, tok)
    model.sync()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for f in range(64):
        model.decode_step(drafts[f], am[f], None, nacc[f:f + 1])
    e1.record(stream)
    model.sync()
    ms = e0.elapsed_time(e1)
    acc = int(nacc.sum().item())
    out["verify"] = {"forwards": 64, "tokens_per_forward": 5, "us_per_forward": round(ms * 1e3 / 64, 1),
                     "forwards_per_s": round(64 / (ms * 1e-3), 1), "positions_per_s": round(5 * 64 / (ms * 1e-3), 1),
                     "committed_tok_per_s_random_drafts": round(acc / (ms * 1e-3), 1),
                     "accepted_per_forward_random_drafts": round(acc / 64, 3)}
    # long context: 8192-token prompt, 128 decode steps
    prompt = torch.tensor(W.make_prompt(cfg, 8192, seed=1), dtype=torch.int32, device=dev)
    toks = torch.zeros(129, dtype=torch.int32, device=dev)
    model.reset()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    model.prefill(prompt, toks[0:1])
    p1.record(stream)
    e0.record(stream)
    for i in range(128):
        model.decode_step(toks[i:i + 1], toks[i + 1:i + 2])
    e1.record(stream)
    model.sync()
    pf_ms, dec_ms = p0.elapsed_time(p1), e0.elapsed_time(e1)
    by = decode_bytes_per_token(cfg, 8192 + 63.5)
    us = dec_ms * 1e3 / 128
    pf = prefill_flops(cfg, 8192)
    out["long_context_8192"] = {"decode_tok_s": round(128 / (dec_ms * 1e-3), 1), "decode_us_per_token": round(us, 1),
                                "hbm_frac_all_bytes": round(by["all"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "hbm_frac_weights_only": round(by["weights"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "prefill_ms": round(pf_ms, 2), "prefill_tok_s": round(8192 / (pf_ms * 1e-3), 1),
                                "prefill_mfma_frac": round(pf["all"] / (pf_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="24L-pp520-tg128", choices=WORKLOAD_CHOICES)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the secondary measurements (verify forwards, 8192-token context)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build runs the forward pass on a single MI355X "
              "(no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import hybrid_deltanet_attention_persistent_amd as pkg
    wl = W.WORKLOADS[args.workload]
    cfg = wl.model
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    weights = W.make_weights(cfg, seed=wl.weight_seed)
    prompt = torch.tensor(W.make_prompt(cfg, wl.prompt_len, seed=wl.prompt_seed), dtype=torch.int32, device=dev)
    model = pkg.Model(cfg, weights, device="cuda:0")
    del weights
    T = wl.decode_steps
    tok = torch.zeros(T + 1, dtype=torch.int32, device=dev)

    def one_step(ev=None):
        model.reset()
        if ev is not None:
            ev[0].record(stream)
        model.prefill(prompt, tok[0:1])
        if ev is not None:
            ev[1].record(stream)
        for i in range(T):
            if ev is not None:
                ev[2 + 2 * i].record(stream)
            model.decode_step(tok[i:i + 1], tok[i + 1:i + 2])
            if ev is not None:
                ev[3 + 2 * i].record(stream)

    for _ in range(args.warmup):   # warm-up first, as a server warms up before taking requests
        one_step()
    model.sync()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + 2 * T)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    model.sync()
    pre_ms = [events[s][0].elapsed_time(events[s][1]) for s in range(args.steps)]
    dec_ms = [[events[s][2 + 2 * i].elapsed_time(events[s][3 + 2 * i]) for i in range(T)] for s in range(args.steps)]
    dec_total = [events[s][2].elapsed_time(events[s][1 + 2 * T]) for s in range(args.steps)]
    decode_tok_s = T * args.steps / (sum(dec_total) / 1e3)
    prefill_tok_s = wl.prompt_len * args.steps / (sum(pre_ms) / 1e3)
    launch_us = float(np.mean(dec_ms)) * 1e3
    ctx_mid = wl.prompt_len + (T - 1) / 2.0
    by = decode_bytes_per_token(cfg, ctx_mid)
    achieved = by["all"] / (launch_us * 1e-6) / 1e9
    pf = prefill_flops(cfg, wl.prompt_len)
    pf_s = float(np.median(pre_ms)) * 1e-3
    pf_tflops = pf["all"] / pf_s / 1e12
    kernel = "mk_forward<1, 1>"
    traffic = load_traffic(kernel)
    line = {
        "metric": "decode tok/s (batch 1, tg128 after pp520)" if wl.name != "tiny-pp16-tg16" else "decode tok/s",
        "value": round(decode_tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(decode_tok_s / BASELINE_DECODE_TOKS, 3) if wl.name == "24L-pp520-tg128" else None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} pp{wl.prompt_len} tg{T} batch 1 (seeded random weights and prompt)",
                   "prompt_tokens": wl.prompt_len, "decode_tokens": T, "batch": 1},
        "prefill_tok_s": round(prefill_tok_s, 1),
        "prefill_roofline": {"bound": "mfma", "achieved": round(pf_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(pf_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "flops_per_prefill": int(pf["all"]), "prefill_ms_median": round(pf_s * 1e3, 3),
                             "weights_hbm_frac": round(by["weights"] / pf_s / 1e9 / HBM_PEAK_GBS, 4)},
        "decode_us_per_token": round(launch_us, 2),
        "hbm_weights_only_frac": round(by["weights"] / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": kernel, "bytes_per_launch": int(by["all"]),
                     "launch_us": round(launch_us, 2)},
    }
    if not args.no_extras and wl.name == "24L-pp520-tg128":
        line["extras"] = extras(model, cfg, stream)
    del model
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = {"read": 1 << 30, "write": 1 << 30}
        del src, dst
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
