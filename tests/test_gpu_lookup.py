"""Greedy generation with weight-free lookup drafts (mk_generate_lookup) through the C ABI.

Speculative decoding must not change the output: every generated token equals the greedy
choice of plain decode (page "업데이트: 단일 RTX 3090에서 Qwen 3.8 27B를 140 tok/s로 구동", accuracy and
speed sections; the drafts are the "lookup-augmented draft" of the RTX 3090 tag page).  The tiny
model is checked against chained mk_decode_step calls and the live oracle, the 24-layer model
against the stored oracle continuation of the pp520 prompt.
"""
import os

import numpy as np
import pytest

import workloads as W
from oracle import OracleModel, C2, argmax_lowest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def dev():
    import hybrid_deltanet_attention_persistent_amd as pkg
    pkg.load_library()
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def i32(x, dev):
    return torch.tensor(np.asarray(x, dtype=np.int32).reshape(-1), dtype=torch.int32, device=dev)


def prefill(m, prompt, dev):
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    m.prefill(i32(prompt, dev), nxt)
    m.sync()
    return int(nxt.item())


def chained_decode(m, first, n, dev):
    outs = [torch.tensor([first], dtype=torch.int32, device=dev)]
    for _ in range(n):
        o = torch.zeros(1, dtype=torch.int32, device=dev)
        m.decode_step(outs[-1], o)
        outs.append(o)
    m.sync()
    return [int(o.item()) for o in outs[1:]]


def repetitive_prompt(cfg, seed, n):
    """A prompt built from a short seeded pattern repeated (so that suffixes recur and drafts exist)."""
    rng = np.random.default_rng(seed)
    pat = rng.integers(0, cfg.vocab, size=7)
    return np.resize(pat, n).astype(np.int64)


@pytest.mark.parametrize("kind", ["seeded", "repetitive"])
def test_tiny_lookup_generation_equals_greedy_decode(dev, kind):
    import hybrid_deltanet_attention_persistent_amd as pkg
    cfg = W.TINY
    weights = W.make_weights(cfg, seed=0)
    prompt = W.make_prompt(cfg, 16, seed=11) if kind == "seeded" else repetitive_prompt(cfg, 12, 21)
    n = 40                                      # prompt + n within the tiny model's 64 positions
    m = pkg.Model(cfg, weights, device=str(dev))
    t0 = prefill(m, prompt, dev)
    toks, st = m.generate_lookup(prompt, t0, n, ngram_min=1, ngram_max=3)
    pos = m.sync()
    assert pos == len(prompt) + n
    assert st["forwards"] + st["accepted"] == n and st["accepted"] <= st["drafted"]
    assert st["drafted"] > 0                    # the loop did run verify forwards
    m.reset()
    t0b = prefill(m, prompt, dev)
    assert t0b == t0
    ref = chained_decode(m, t0, n, dev)
    assert toks == ref, f"first difference at {next(i for i in range(n) if toks[i] != ref[i])}"
    # the oracle's greedy continuation (drafts cannot change it)
    o = OracleModel(cfg, weights, C2)
    t = argmax_lowest(o.prefill(prompt))
    assert t == t0
    want = []
    for _ in range(n):
        t = argmax_lowest(o.decode(t))
        want.append(t)
    assert toks == want
    # the state after the call continues like plain decode: one more step from the last token
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    m2 = pkg.Model(cfg, weights, device=str(dev))
    t0c = prefill(m2, prompt, dev)
    toks2, _ = m2.generate_lookup(prompt, t0c, n - 1)
    m2.decode_step(i32([toks2[-1]], dev), nxt)
    m2.sync()
    assert toks2 + [int(nxt.item())] == want
    m.close()
    m2.close()


def test_24L_lookup_generation_equals_stored_oracle_continuation(dev):
    import hybrid_deltanet_attention_persistent_amd as pkg
    path = os.path.join(GOLDEN, "24L-pp520-tg128.npz")
    if not os.path.exists(path):
        pytest.skip("stored oracle outputs 24L-pp520-tg128.npz not generated")
    gd = dict(np.load(path, allow_pickle=False))
    cfg = W.HYBRID_24L
    prompt = W.make_prompt(cfg, 520, seed=1)
    assert np.array_equal(prompt, gd["prompt"])
    m = pkg.Model(cfg, W.make_weights(cfg, seed=0), device=str(dev))
    t0 = prefill(m, prompt, dev)
    assert t0 == int(gd["tokens"][0])
    n = len(gd["tokens"]) - 1
    toks, st = m.generate_lookup(prompt, t0, n, ngram_min=1, ngram_max=3)
    assert m.sync() == 520 + n
    want = [int(x) for x in gd["tokens"][1:]]
    assert toks == want, f"first difference at {next(i for i in range(n) if toks[i] != want[i])}"
    assert st["forwards"] + st["accepted"] == n
    print(f"24L lookup decode: {n} tokens in {st['forwards']} launches, {st['accepted']} of {st['drafted']} drafts accepted")
    m.close()


def test_lookup_generation_rejects_bad_arguments(dev):
    import hybrid_deltanet_attention_persistent_amd as pkg
    cfg = W.TINY
    m = pkg.Model(cfg, W.make_weights(cfg, seed=0), device=str(dev))
    prompt = W.make_prompt(cfg, 10, seed=3)
    t0 = prefill(m, prompt, dev)
    for args in [(prompt, cfg.vocab, 4, 1, 3), (prompt, t0, 4, 0, 3), (prompt, t0, 4, 3, 2), (prompt, t0, -1, 1, 3)]:
        with pytest.raises(pkg.MkError) as e:
            m.generate_lookup(*args)
        assert e.value.status == pkg.lib.MK_EINVAL
    assert m.sync() == 10                      # nothing was launched
    toks, _ = m.generate_lookup(prompt, t0, 0)
    assert toks == [] and m.sync() == 10
    m.close()
