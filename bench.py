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
import dataclasses
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
CONTEXT_RTX3090_DECODE_TOKS = 413.0   # the pages' megakernel decode figure (tg128, another GPU): context only
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
    # K and V of one position: bf16, or (8-bit cache) one byte per element plus one exponent byte per row
    kv_row = cfg.at_kv_heads * 2 * ((cfg.at_head_dim + 1) if cfg.kv_quant else cfg.at_head_dim * 2)
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


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(decode_seconds: float = 10.0) -> dict:
    """The oracle as it stands, single-threaded, on a bounded sample of the headline workload:
    the whole 520-token prompt (timed: prefill tok/s), then greedy decode steps after it for
    about `decode_seconds` (timed: decode tok/s, the value)."""
    from threadpoolctl import threadpool_limits
    from oracle import OracleModel, C2, argmax_lowest
    cfg = W.HYBRID_24L
    weights = W.make_weights(cfg, seed=0)
    prompt = W.make_prompt(cfg, 520, seed=1)
    with threadpool_limits(limits=1):
        m = OracleModel(cfg, weights, C2)
        del weights
        t0 = time.perf_counter()
        t = argmax_lowest(m.prefill(prompt))
        pf_s = time.perf_counter() - t0
        n, t0 = 0, time.perf_counter()
        while True:
            t = argmax_lowest(m.decode(t))
            n += 1
            el = time.perf_counter() - t0
            if el >= decode_seconds or n >= 128:
                break
    return {"value": round(n / el, 3), "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"pp520 prompt of the 24-layer model ({pf_s:.1f} s), then {n} greedy decode steps after "
                      f"it ({el:.1f} s); float64 numpy, one BLAS thread",
            "prefill_tok_s": round(520 / pf_s, 2), "cpu_model": host_cpu_model(),
            "os_cpu_count": os.cpu_count()}


def long_context(model, cfg, stream, n_prompt: int = 8192, n_decode: int = 128) -> dict:
    """Prefill of an n_prompt-token seeded prompt, then n_decode chained greedy decode steps."""
    import torch
    dev = stream.device
    prompt = torch.tensor(W.make_prompt(cfg, n_prompt, seed=1), dtype=torch.int32, device=dev)
    toks = torch.zeros(n_decode + 1, dtype=torch.int32, device=dev)
    model.reset()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    model.prefill(prompt, toks[0:1])
    p1.record(stream)
    e0.record(stream)
    for i in range(n_decode):
        model.decode_step(toks[i:i + 1], toks[i + 1:i + 2])
    e1.record(stream)
    model.sync()
    pf_ms, dec_ms = p0.elapsed_time(p1), e0.elapsed_time(e1)
    by = decode_bytes_per_token(cfg, n_prompt + (n_decode - 1) / 2.0)
    us = dec_ms * 1e3 / n_decode
    pf = prefill_flops(cfg, n_prompt)
    return {"decode_tok_s": round(n_decode / (dec_ms * 1e-3), 1), "decode_us_per_token": round(us, 1),
            "hbm_frac_all_bytes": round(by["all"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "hbm_frac_weights_only": round(by["weights"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "prefill_ms": round(pf_ms, 2), "prefill_tok_s": round(n_prompt / (pf_ms * 1e-3), 1),
            "prefill_mfma_frac": round(pf["all"] / (pf_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def batch_decode(pkg, cfg, weights, stream, n_steps: int = 64) -> dict:
    """Batch decode: B sequences (B = 1..5), each after its own 520-token seeded prompt, share one
    weight pass per launch; n_steps launches chained on the device.  Aggregate tok/s counts every
    sequence's token."""
    import torch
    dev = stream.device
    nmax = 5
    cfgb = dataclasses.replace(cfg, n_seq=nmax)
    m = pkg.Model(cfgb, weights, device=str(dev))
    prompts = [torch.tensor(W.make_prompt(cfg, 520, seed=1 + s), dtype=torch.int32, device=dev) for s in range(nmax)]
    res = {}
    for B in range(1, nmax + 1):
        seqs = list(range(B))
        tok = torch.zeros((n_steps + 1, B), dtype=torch.int32, device=dev)
        for rep in range(2):          # the first pass warms the batch instantiation up
            m.reset()
            for s in seqs:
                m.select(s)
                m.prefill(prompts[s], tok[0, s:s + 1])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n_steps):
                m.decode_batch(seqs, tok[i], tok[i + 1])
            e1.record(stream)
            m.sync()
        us = e0.elapsed_time(e1) * 1e3 / n_steps
        by = decode_bytes_per_token(cfg, 520 + (n_steps - 1) / 2.0)
        kv_state = by["all"] - by["weights"]
        launch_bytes = by["weights"] + B * kv_state
        res[f"B{B}"] = {"us_per_launch": round(us, 1), "aggregate_tok_s": round(B * 1e6 / us, 1),
                        "hbm_frac": round(launch_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    m.close()
    res["note"] = ("mk_decode_batch over sequences 0..B-1 of one model (n_seq = 5), each after its own pp520 prompt; "
                   "B = 1 runs the one-column decode kernel, B >= 2 the five-column batch kernel")
    return res


def extras(model, cfg, stream, weights=None) -> dict:
    """Secondary measurements on the same model: multi-token verify forwards after the pp520
    prompt (1 accepted + 4 seeded random drafts each, state rolled back to the accepted prefix),
    greedy generation with lookup drafts after the same prompt, and decode at long context after
    an 8192-token prompt, with the bf16 KV cache and (given the weights) with the 8-bit one."""
    import torch
    dev = stream.device
    out = {}
    # verify: 64 forwards of [last accepted, 4 drafts], each started from the previous forward's
    # greedy token after its last accepted position (picked on the device: no host round trip)
    nf = 64
    prompt = torch.tensor(W.make_prompt(cfg, 520, seed=1), dtype=torch.int32, device=dev)
    # tokens [last accepted, 4 drafts] per forward (make_drafts gives the 4 drafts)
    toks = torch.zeros((nf, 5), dtype=torch.int32, device=dev)
    toks[:, 1:] = torch.tensor(W.make_drafts(cfg, nf, 5, seed=2), dtype=torch.int32, device=dev)
    am = torch.zeros((nf, 5), dtype=torch.int32, device=dev)
    nacc = torch.zeros((nf, 1), dtype=torch.int32, device=dev)
    model.reset()
    model.prefill(prompt, toks[0, 0:1])
    model.sync()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nf)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for f in range(nf):
        ev[f][0].record(stream)
        model.decode_step(toks[f], am[f], None, nacc[f])
        ev[f][1].record(stream)
        if f + 1 < nf:
            toks[f + 1, 0:1] = torch.gather(am[f], 0, (nacc[f] - 1).long())
    e1.record(stream)
    model.sync()
    ms = e0.elapsed_time(e1)
    launch_us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    acc = int(nacc.sum().item())
    out["verify"] = {"forwards": nf, "tokens_per_forward": 5, "us_per_forward": round(launch_us, 1),
                     "forwards_per_s": round(1e6 / launch_us, 1), "positions_per_s": round(5e6 / launch_us, 1),
                     "committed_tok_per_s_random_drafts": round(acc / (ms * 1e-3), 1),
                     "accepted_per_forward_random_drafts": round(acc / nf, 3)}
    # lookup drafts: 128 greedy tokens after the pp520 prompt, each launch verifying the last token
    # plus the n-gram drafts found in the prompt and the tokens generated so far (one host round
    # trip per launch), against 128 chained decode steps on the same state
    pnp = W.make_prompt(cfg, 520, seed=1)
    first = torch.zeros(1, dtype=torch.int32, device=dev)
    model.reset()
    model.prefill(prompt, first)
    model.sync()
    t_first = int(first.item())
    t0 = time.perf_counter()
    toks_lk, st = model.generate_lookup(pnp, t_first, 128, 1, 3)
    lk_s = time.perf_counter() - t0
    model.reset()
    model.prefill(prompt, first)
    model.sync()
    chain = torch.zeros(129, dtype=torch.int32, device=dev)
    chain[0:1] = first
    t0 = time.perf_counter()
    for i in range(128):
        model.decode_step(chain[i:i + 1], chain[i + 1:i + 2])
    model.sync()
    dec_s = time.perf_counter() - t0
    same = toks_lk == chain[1:].cpu().numpy().tolist()
    # the same 128 tokens with perfect drafts (the greedy continuation just computed, 4 per verify
    # forward, chained on the device): what verify commits when every draft is right
    model.reset()
    model.prefill(prompt, first)
    nfw = 128 // 5
    planted = torch.zeros((nfw, 5), dtype=torch.int32, device=dev)
    for f in range(nfw):
        planted[f] = chain[5 * f:5 * f + 5]
    pam = torch.zeros((nfw, 5), dtype=torch.int32, device=dev)
    pacc = torch.zeros((nfw, 1), dtype=torch.int32, device=dev)
    model.sync()
    e0.record(stream)
    for f in range(nfw):
        model.decode_step(planted[f], pam[f], None, pacc[f])
    e1.record(stream)
    model.sync()
    pl_ms = e0.elapsed_time(e1)
    pl_ok = bool(torch.equal(pam[:, :4], planted[:, 1:])) and int(pacc.min().item()) == 5
    out["lookup_decode"] = {"tokens": 128, "launches": st["forwards"], "drafted": st["drafted"],
                            "accepted_drafts": st["accepted"], "tokens_per_launch": round(128 / st["forwards"], 3),
                            "committed_tok_per_s": round(128 / lk_s, 1), "plain_decode_tok_per_s": round(128 / dec_s, 1),
                            "speedup": round(dec_s / lk_s, 3), "tokens_equal_plain_decode": bool(same),
                            "note": "host clock around each loop; the lookup loop synchronises once per launch",
                            "perfect_drafts": {"forwards": nfw, "accepted_per_forward": 5, "all_accepted": pl_ok,
                                               "committed_tok_per_s": round(5 * nfw / (pl_ms * 1e-3), 1)}}
    # long context: 8192-token prompt, 128 decode steps
    out["long_context_8192"] = long_context(model, cfg, stream)
    if weights is not None:
        import hybrid_deltanet_attention_persistent_amd as pkg
        out["batch_decode"] = batch_decode(pkg, cfg, weights, stream)
        cfg8 = dataclasses.replace(cfg, name=cfg.name + "-q8", kv_quant=1)
        m8 = pkg.Model(cfg8, weights, device=str(dev))
        long_context(m8, cfg8, stream, 1024, 8)      # warm-up of the 8-bit instantiations
        out["long_context_8192_kv8"] = long_context(m8, cfg8, stream)
        out["long_context_8192_kv8"]["kv_cache"] = "int8 codes + power-of-two scale per row"
        m8.close()
    return out


def energy(model, cfg, stream, seconds: float = 4.0) -> dict:
    """Energy per token from the GPU's own energy accumulator (amdsmi), accelerator socket only,
    like the launch page's method (section "Measurement:": NVML energy counters, accelerator power
    only), at the power cap the GPU runs with: the page's power-limit sweep (section "Then we
    turned the power down") needs privileges this run does not have.  The driver refreshes the
    accumulator only every so often, so energy is read around windows of several seconds (timed by
    the accumulator's own timestamp): window A repeats (reset, pp520 prompt, 128 chained decode
    steps), window B repeats (reset, pp520 prompt); decode energy per token = (A per round - B per
    round) / 128."""
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as e:  # noqa: BLE001 -- reported, not fatal
        return {"error": f"amdsmi unavailable: {e}"}
    try:
        h = amdsmi.amdsmi_get_processor_handles()[0]   # the one visible GPU

        def read():
            e = amdsmi.amdsmi_get_energy_count(h)
            return e["energy_accumulator"] * e["counter_resolution"] * 1e-6, e["timestamp"] * 1e-9

        cap = amdsmi.amdsmi_get_power_cap_info(h)
        dev = stream.device
        prompt = torch.tensor(W.make_prompt(cfg, 520, seed=1), dtype=torch.int32, device=dev)
        toks = torch.zeros(129, dtype=torch.int32, device=dev)

        def window(decode: bool):
            model.sync()
            j0, s0 = read()
            t0, n = time.perf_counter(), 0
            while time.perf_counter() - t0 < seconds:
                model.reset()
                model.prefill(prompt, toks[0:1])
                if decode:
                    for i in range(128):
                        model.decode_step(toks[i:i + 1], toks[i + 1:i + 2])
                model.sync()
                n += 1
            j1, s1 = read()
            return j1 - j0, s1 - s0, n

        ea, sa, na = window(True)
        eb, sb, nb = window(False)
        if ea <= 0 or eb <= 0 or sa <= 0 or sb <= 0:
            return {"error": f"energy accumulator did not advance (A {ea} J over {sa} s, B {eb} J over {sb} s)"}
        e_pf = eb / nb
        e_tok = (ea / na - e_pf) / 128
        t_tok = (sa / na - sb / nb) / 128
        w = lambda v: round(v * 1e-6, 1) if v > 1e5 else v   # caps are reported in microwatts
        return {"decode_tok_per_j": round(1 / e_tok, 3), "decode_j_per_tok": round(e_tok, 4),
                "decode_avg_power_w": round(e_tok / t_tok, 1), "decode_tok_s_in_window": round(1 / t_tok, 1),
                "prefill_pp520_j": round(e_pf, 3), "prefill_tok_per_j": round(520 / e_pf, 1),
                "prefill_avg_power_w": round(eb / sb, 1),
                "window_a": {"rounds": na, "seconds": round(sa, 3), "joules": round(ea, 1)},
                "window_b": {"rounds": nb, "seconds": round(sb, 3), "joules": round(eb, 1)},
                "power_cap_w": w(cap["power_cap"]),
                "note": "socket energy accumulator (15.3 uJ units) and its timestamp; the host synchronises "
                        "after every round, so idle gaps between launches are inside the windows"}
    except Exception as e:  # noqa: BLE001
        return {"error": f"energy read failed: {e}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:  # noqa: BLE001
            pass


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="24L-pp520-tg128", choices=WORKLOAD_CHOICES)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-energy", action="store_true", help="skip the energy-per-token windows of the extras")
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
        "vs_baseline": None,
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
        line["extras"] = extras(model, cfg, stream, weights)
        if not args.no_energy:
            line["extras"]["energy"] = energy(model, cfg, stream)
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
