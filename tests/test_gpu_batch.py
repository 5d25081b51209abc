"""Batch decode (mk_decode_batch): B sequences, each with its own state and KV cache, share one
weight pass per launch (the concurrency figures of the RTX 3090 tag page's Dflash2 item).

Bar: every sequence's greedy tokens and logits equal, bit for bit, those of single-sequence decode
steps on the same sequence (the batch kernel runs the decode arithmetic per column), and the
oracle's within max |error| 3e-2 / relative L2 1e-2 where the oracle is run.
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from oracle import OracleModel, C2, argmax_lowest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
MAX_ABS, REL_L2 = 3e-2, 1e-2


def close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.max(np.abs(gpu - ref))
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err < MAX_ABS and rel < REL_L2, f"{what}: max abs {err:.3e}, rel L2 {rel:.3e}"


@pytest.fixture(scope="module")
def dev():
    import hybrid_deltanet_attention_persistent_amd as pkg
    pkg.load_library()
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def i32(x, dev):
    return torch.tensor(np.asarray(x, dtype=np.int32).reshape(-1), dtype=torch.int32, device=dev)


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def single_run(cfg, weights, dev, prompt, steps):
    """Prefill + `steps` chained greedy decode steps on a one-sequence model: (tokens, logits)."""
    import hybrid_deltanet_attention_persistent_amd as pkg
    m = pkg.Model(dataclasses.replace(cfg, n_seq=1), weights, device=str(dev))
    tok = torch.zeros(steps + 1, dtype=torch.int32, device=dev)
    lg = torch.zeros((steps + 1, cfg.vocab), dtype=torch.float32, device=dev)
    m.prefill(i32(prompt, dev), tok[0:1], lg[0])
    for i in range(steps):
        m.decode_step(tok[i:i + 1], tok[i + 1:i + 2], lg[i + 1])
    m.sync()
    out = tok.cpu().numpy().tolist(), lg.cpu().numpy().copy()
    m.close()
    return out


def batch_run(m, dev, vocab, seqs, prompts, steps):
    """Prefill each of `seqs` with its prompt, then `steps` batch launches over all of them, chained on
    the device.  Returns per sequence (tokens, logits), position 0 from the prefill."""
    n = len(seqs)
    tok = torch.zeros((steps + 1, n), dtype=torch.int32, device=dev)
    lg = torch.zeros((steps + 1, n, vocab), dtype=torch.float32, device=dev)
    for c, (s, p) in enumerate(zip(seqs, prompts)):
        m.select(s)
        m.prefill(i32(p, dev), tok[0, c:c + 1], lg[0, c])
    for i in range(steps):
        m.decode_batch(seqs, tok[i], tok[i + 1], lg[i + 1])
    m.sync()
    t, l = tok.cpu().numpy(), lg.cpu().numpy()
    return [(t[:, c].tolist(), l[:, c].copy()) for c in range(n)]


# ---------------------------------------------------------------------------------- tiny model
@pytest.fixture(scope="module")
def tiny():
    return W.make_weights(W.TINY, seed=0)


def test_tiny_batch_of_three_equals_single_decode_and_oracle(dev, tiny):
    import hybrid_deltanet_attention_persistent_amd as pkg
    cfg = dataclasses.replace(W.TINY, n_seq=3)
    prompts = [W.make_prompt(cfg, n, seed=60 + n) for n in (5, 16, 9)]
    m = pkg.Model(cfg, tiny, device=str(dev))
    res = batch_run(m, dev, cfg.vocab, [0, 1, 2], prompts, 12)
    for c, p in enumerate(prompts):
        st, sl = single_run(cfg, tiny, dev, p, 12)
        assert res[c][0] == st, f"sequence {c}"
        assert np.array_equal(bits(res[c][1]), bits(sl)), f"sequence {c}"
        rt, rl = OracleModel(W.TINY, tiny, C2).generate(p, 12)
        assert res[c][0] == list(rt), f"sequence {c}"
        for i in range(13):
            close(res[c][1][i], rl[i], f"sequence {c} position {i}")
    for s in range(3):
        m.select(s)
        assert m.sync() == len(prompts[s]) + 12
    m.close()


def test_tiny_batch_subset_order_and_interleaving(dev, tiny):
    """Batches over a subset in any order, single decode steps of one sequence in between, and a
    sequence left out of a batch keeps its state."""
    import hybrid_deltanet_attention_persistent_amd as pkg
    cfg = dataclasses.replace(W.TINY, n_seq=3)
    prompts = [W.make_prompt(cfg, n, seed=70 + n) for n in (7, 3, 12)]
    m = pkg.Model(cfg, tiny, device=str(dev))
    refs = [OracleModel(W.TINY, tiny, C2) for _ in range(3)]
    nxt = [0, 0, 0]
    for s in range(3):
        m.select(s)
        o = torch.zeros(1, dtype=torch.int32, device=dev)
        m.prefill(i32(prompts[s], dev), o)
        m.sync()
        nxt[s] = int(o.item())
        assert nxt[s] == argmax_lowest(refs[s].prefill(prompts[s]))
    plan = [[2, 0], [1], "single 0", [0, 1, 2], [1, 2], "single 2", [2, 1, 0]]
    for step in plan:
        if isinstance(step, str):
            s = int(step.split()[1])
            m.select(s)
            o = torch.zeros(1, dtype=torch.int32, device=dev)
            lg = torch.zeros(cfg.vocab, dtype=torch.float32, device=dev)
            m.decode_step(i32([nxt[s]], dev), o, lg)
            m.sync()
            rl = refs[s].decode(nxt[s])
            close(lg.cpu().numpy(), rl, step)
            nxt[s] = int(o.item())
            assert nxt[s] == argmax_lowest(rl), step
            continue
        n = len(step)
        o = torch.zeros(n, dtype=torch.int32, device=dev)
        lg = torch.zeros((n, cfg.vocab), dtype=torch.float32, device=dev)
        m.decode_batch(step, i32([nxt[s] for s in step], dev), o, lg)
        m.sync()
        for c, s in enumerate(step):
            rl = refs[s].decode(nxt[s])
            close(lg[c].cpu().numpy(), rl, f"batch {step} sequence {s}")
            nxt[s] = int(o[c].item())
            assert nxt[s] == argmax_lowest(rl), f"batch {step} sequence {s}"
    for s in range(3):
        m.select(s)
        assert m.sync() == refs[s].pos
    m.close()


def test_tiny_batch_rejections(dev, tiny):
    import hybrid_deltanet_attention_persistent_amd as pkg
    from hybrid_deltanet_attention_persistent_amd import MkError
    from hybrid_deltanet_attention_persistent_amd.lib import MK_EINVAL, MK_ECTX
    cfg = dataclasses.replace(W.TINY, n_seq=2)
    m = pkg.Model(cfg, tiny, device=str(dev))
    t = i32([1, 2, 3, 4, 5], dev)
    o = torch.zeros(5, dtype=torch.int32, device=dev)
    for s in range(2):
        m.select(s)
        m.prefill(i32(W.make_prompt(cfg, 6, seed=80 + s), dev), o[:1])
    for seqs in ([0, 0], [0, 2], [-1], [0, 1, 1], []):
        with pytest.raises(MkError) as e:
            m.decode_batch(seqs, t, o)
        assert e.value.status == MK_EINVAL, seqs
    with pytest.raises(MkError) as e:
        m.select(2)
    assert e.value.status == MK_EINVAL
    # a verify forward on sequence 1 leaves it unsettled until its next decode step
    m.select(1)
    m.decode_step(t[:3], o[:3], None, torch.zeros(1, dtype=torch.int32, device=dev))
    with pytest.raises(MkError) as e:
        m.decode_batch([0, 1], t, o)
    assert e.value.status == MK_EINVAL
    m.decode_step(o[:1], o[3:4])
    m.decode_batch([0, 1], t, o)
    m.sync()
    # a sequence at max_ctx
    m.reset()
    m.select(0)
    m.prefill(i32(W.make_prompt(cfg, cfg.max_ctx, seed=3), dev), o[:1])
    with pytest.raises(MkError) as e:
        m.decode_batch([1, 0], t, o)
    assert e.value.status == MK_ECTX
    m.decode_batch([1], t, o)
    m.sync()
    m.close()
    m8 = pkg.Model(dataclasses.replace(W.TINY_Q8, n_seq=2), tiny, device=str(dev))
    with pytest.raises(MkError) as e:
        m8.decode_batch([0, 1], t, o)
    assert e.value.status == MK_EINVAL
    m8.close()


# ---------------------------------------------------------------------------------- 24 layers
@pytest.fixture(scope="module")
def big_weights():
    return W.make_weights(W.HYBRID_24L, seed=0)


def test_24L_batch_of_five_equals_single_decode(dev, big_weights):
    """Five sequences at different positions (prompts of 1, 67, 130, 200 and 520 tokens) through the
    hidden-1024 batch kernel: every token and logit bit-identical to single-sequence decode, and the
    520-token sequence's first tokens equal to the stored oracle continuation."""
    import hybrid_deltanet_attention_persistent_amd as pkg
    cfg = dataclasses.replace(W.HYBRID_24L, n_seq=5)
    lens = (1, 67, 130, 200, 520)
    prompts = [W.make_prompt(cfg, n, seed=90 + i) for i, n in enumerate(lens[:-1])] + [W.make_prompt(cfg, 520, seed=1)]
    m = pkg.Model(cfg, big_weights, device=str(dev))
    steps = 6
    res = batch_run(m, dev, cfg.vocab, [4, 3, 2, 1, 0], prompts, steps)
    m.close()
    for c, p in enumerate(prompts):
        st, sl = single_run(cfg, big_weights, dev, p, steps)
        assert res[c][0] == st, f"prompt of {len(p)}"
        assert np.array_equal(bits(res[c][1]), bits(sl)), f"prompt of {len(p)}"
    gd = dict(np.load(f"{__import__('os').path.dirname(__file__)}/golden/24L-pp520-tg128.npz", allow_pickle=False))
    assert res[-1][0] == gd["tokens"][:steps + 1].tolist()


def test_24L_batch_matches_live_oracle(dev, big_weights):
    """Two short prompts in one batch against the live oracle, every logit."""
    import hybrid_deltanet_attention_persistent_amd as pkg
    cfg = dataclasses.replace(W.HYBRID_24L, n_seq=2)
    prompts = [W.make_prompt(cfg, 3, seed=95), W.make_prompt(cfg, 66, seed=96)]
    m = pkg.Model(cfg, big_weights, device=str(dev))
    res = batch_run(m, dev, cfg.vocab, [1, 0], prompts, 2)
    m.close()
    for c, p in enumerate(prompts):
        rt, rl = OracleModel(W.HYBRID_24L, big_weights, C2).generate(p, 2)
        assert res[c][0] == list(rt)
        for i in range(3):
            close(res[c][1][i], rl[i], f"prompt {len(p)} position {i}")
