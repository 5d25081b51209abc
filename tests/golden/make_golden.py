"""Write the stored expected values used by the GPU parity tests.

Every value here comes from the CPU oracle (``oracle/``) run on the seeded
synthetic inputs of ``workloads``; nothing is read from the GPU path.  Run from
the repository root:

    python tests/golden/make_golden.py 24L-pp520-tg128 [24L-pp520-verify5 24L-pp8192-tg128 ...]

Each workload writes tests/golden/<name>.npz with, per compared position: the
oracle's greedy token, its logits at a fixed seeded sample of vocabulary ids,
its top-8 ids and values, and the margin between its two largest logits.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from oracle import OracleModel, C2, argmax_lowest  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
N_SAMPLE = 512


def sample_ids(vocab: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([77])))
    return np.sort(rng.choice(vocab, size=min(N_SAMPLE, vocab), replace=False)).astype(np.int64)


def summarize(logits: np.ndarray, ids: np.ndarray):
    top = np.argsort(-logits, kind="stable")[:8]
    srt = np.sort(logits)
    return logits[ids], top, logits[top], srt[-1] - srt[-2]


def run_generate(wl: W.Workload):
    cfg = wl.model
    weights = W.make_weights(cfg, seed=wl.weight_seed)
    prompt = W.make_prompt(cfg, wl.prompt_len, seed=wl.prompt_seed)
    ids = sample_ids(cfg.vocab)
    m = OracleModel(cfg, weights, C2)
    del weights
    rows = []
    t0 = time.time()
    lg = m.prefill(prompt)
    print(f"{wl.name}: prefill {wl.prompt_len} in {time.time() - t0:.1f}s", flush=True)
    toks = [argmax_lowest(lg)]
    rows.append(summarize(lg, ids))
    for i in range(wl.decode_steps):
        lg = m.decode(toks[-1])
        toks.append(argmax_lowest(lg))
        rows.append(summarize(lg, ids))
        if i % 16 == 15:
            print(f"{wl.name}: decode {i + 1} ({time.time() - t0:.1f}s)", flush=True)
    return dict(prompt=prompt, tokens=np.array(toks, dtype=np.int64), sample_ids=ids,
                sample_logits=np.stack([r[0] for r in rows]).astype(np.float32),
                top_ids=np.stack([r[1] for r in rows]).astype(np.int64),
                top_vals=np.stack([r[2] for r in rows]).astype(np.float32),
                margin=np.array([r[3] for r in rows], dtype=np.float32))


def run_verify(wl: W.Workload, max_forwards: int = 160):
    """Commit loop of verify forwards [t0, d1..d4] with seeded random drafts until
    decode_steps tokens are committed after the prompt's greedy token."""
    cfg = wl.model
    weights = W.make_weights(cfg, seed=wl.weight_seed)
    prompt = W.make_prompt(cfg, wl.prompt_len, seed=wl.prompt_seed)
    drafts = W.make_drafts(cfg, max_forwards, wl.verify_width, seed=wl.draft_seed)
    ids = sample_ids(cfg.vocab)[::4]
    m = OracleModel(cfg, weights, C2)
    del weights
    t0 = time.time()
    g0 = argmax_lowest(m.prefill(prompt))
    committed = [g0]
    fwd_tokens, fwd_greedy, fwd_nacc, fwd_sample = [], [], [], []
    f = 0
    while len(committed) < wl.decode_steps + 1 and f < max_forwards:
        toks = [committed[-1]] + [int(d) for d in drafts[f]]
        greedy, n_acc, logits = m.verify(toks)
        fwd_tokens.append(toks)
        fwd_greedy.append(greedy)
        fwd_nacc.append(n_acc)
        fwd_sample.append(logits[:, ids])
        committed += greedy[:n_acc]
        f += 1
        if f % 16 == 0:
            print(f"{wl.name}: {f} forwards, {len(committed)} committed ({time.time() - t0:.1f}s)", flush=True)
    return dict(prompt=prompt, drafts=drafts[:f], sample_ids=ids, committed=np.array(committed, dtype=np.int64),
                fwd_tokens=np.array(fwd_tokens, dtype=np.int64), fwd_greedy=np.array(fwd_greedy, dtype=np.int64),
                fwd_nacc=np.array(fwd_nacc, dtype=np.int64),
                fwd_sample_logits=np.stack(fwd_sample).astype(np.float32))


def main(names):
    for name in names:
        wl = W.WORKLOADS[name]
        out = run_verify(wl) if wl.verify_width > 1 else run_generate(wl)
        path = os.path.join(HERE, name + ".npz")
        np.savez_compressed(path, **out)
        print(f"wrote {path}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["tiny-pp16-tg16"])
