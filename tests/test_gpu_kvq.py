"""GPU parity of the 8-bit KV cache (mk_config.kv_quant = 1) against the oracle with the same
cache format (oracle.ops.kv_q8_rows: int8 codes and a power-of-two scale per cached row; the
8-bit cache of the pages' limits and tag pages).

Same bar as the bf16 cache: greedy tokens equal to the oracle's, logits within max |error| 3e-2
and relative L2 error 1e-2; verify forwards bit-identical to sequential decode steps.  The
quantiser's decisions are taken in FP32 on both sides; a code that lands on the other side of a
rounding boundary moves one cached element by one step, far inside the bar.
"""
import os

import numpy as np
import pytest

import workloads as W
from oracle import OracleModel, C2, argmax_lowest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MAX_ABS, REL_L2 = 3e-2, 1e-2


def close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.max(np.abs(gpu - ref))
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err < MAX_ABS and rel < REL_L2, f"{what}: max abs {err:.3e}, rel L2 {rel:.3e}"
    return err, rel


@pytest.fixture(scope="module")
def dev():
    import hybrid_deltanet_attention_persistent_amd as pkg
    pkg.load_library()
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def i32(x, dev):
    return torch.tensor(np.asarray(x, dtype=np.int32).reshape(-1), dtype=torch.int32, device=dev)


class Runner:
    def __init__(self, cfg, weights, dev):
        import hybrid_deltanet_attention_persistent_amd as pkg
        self.cfg, self.dev = cfg, dev
        self.m = pkg.Model(cfg, weights, device=str(dev))
        self.tok = torch.zeros(5, dtype=torch.int32, device=dev)
        self.lg = torch.zeros((5, cfg.vocab), dtype=torch.float32, device=dev)
        self.nacc = torch.zeros(1, dtype=torch.int32, device=dev)

    def prefill(self, prompt):
        self.m.prefill(i32(prompt, self.dev), self.tok[:1], self.lg[0])
        self.m.sync()
        return int(self.tok[0].item()), self.lg[0].cpu().numpy().copy()

    def decode(self, t):
        self.m.decode_step(i32([t], self.dev), self.tok[:1], self.lg[0])
        self.m.sync()
        return int(self.tok[0].item()), self.lg[0].cpu().numpy().copy()

    def verify(self, toks):
        n = len(toks)
        self.m.decode_step(i32(toks, self.dev), self.tok[:n], self.lg[:n], self.nacc)
        self.m.sync()
        return (self.tok[:n].cpu().numpy().tolist(), int(self.nacc.item()), self.lg[:n].cpu().numpy().copy())

    def close(self):
        self.m.close()


# ---------------------------------------------------------------------------------- tiny model
@pytest.fixture(scope="module")
def tiny():
    return W.make_weights(W.TINY_Q8, seed=0)


def test_tiny_q8_generate_matches_oracle(dev, tiny):
    cfg = W.TINY_Q8
    prompt = W.make_prompt(cfg, 16, seed=1)
    ref_toks, ref_logits = OracleModel(cfg, tiny, C2).generate(prompt, 16)
    r = Runner(cfg, tiny, dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros((17, cfg.vocab), dtype=torch.float32, device=dev)
    r.m.prefill(i32(prompt, dev), nxt, logits[0])
    outs = [nxt]
    for i in range(16):
        o = torch.zeros(1, dtype=torch.int32, device=dev)
        r.m.decode_step(outs[-1], o, logits[i + 1])
        outs.append(o)
    assert r.m.sync() == 32
    assert [int(o.item()) for o in outs] == list(ref_toks)
    for i in range(17):
        close(logits[i].cpu().numpy(), ref_logits[i], f"position {i}")
    r.close()


def test_tiny_q8_teacher_forced_to_a_full_context(dev, tiny):
    """Prompt of 5, then 59 forced tokens: every position of the 64-token context, both appends
    (prefill and decode) and both reads (prefill attention and decode split-KV)."""
    cfg = W.TINY_Q8
    prompt = W.make_prompt(cfg, 5, seed=21)
    feed = W.make_prompt(cfg, cfg.max_ctx - 5, seed=22)
    ref = OracleModel(cfg, tiny, C2)
    r = Runner(cfg, tiny, dev)
    g, lg = r.prefill(prompt)
    rl = ref.prefill(prompt)
    close(lg, rl, "prefill")
    assert g == argmax_lowest(rl)
    for i, t in enumerate(feed):
        g, lg = r.decode(int(t))
        rl = ref.decode(int(t))
        close(lg, rl, f"step {i}")
        assert g == argmax_lowest(rl), f"step {i}"
    r.close()


def test_tiny_q8_prompt_after_decode(dev, tiny):
    """A second prompt after decode steps: prefill attention reads rows that decode appended."""
    cfg = W.TINY_Q8
    p1, p2 = W.make_prompt(cfg, 9, seed=51), W.make_prompt(cfg, 23, seed=52)
    ref = OracleModel(cfg, tiny, C2)
    r = Runner(cfg, tiny, dev)
    checks = [(r.prefill(p1), ref.prefill(p1))]
    t = checks[-1][0][0]
    for _ in range(3):
        checks.append((r.decode(t), ref.decode(t)))
        t = checks[-1][0][0]
    checks.append((r.prefill(p2), ref.prefill(p2)))
    t = checks[-1][0][0]
    checks.append((r.decode(t), ref.decode(t)))
    for i, ((g, lg), rl) in enumerate(checks):
        assert g == argmax_lowest(rl), f"call {i}"
        close(lg, rl, f"call {i}")
    r.close()


@pytest.mark.parametrize("n_good", [0, 2, 4])
def test_tiny_q8_verify_is_bit_identical_to_sequential_decode(dev, tiny, n_good):
    cfg = W.TINY_Q8
    prompt = W.make_prompt(cfg, 11, seed=8)
    seq = Runner(cfg, tiny, dev)
    g0, _ = seq.prefill(prompt)
    ref = OracleModel(cfg, tiny, C2)
    ref.prefill(prompt)
    greedy_ref, t = [], g0
    for _ in range(4):
        t = argmax_lowest(ref.decode(t))
        greedy_ref.append(t)
    drafts = list(greedy_ref)
    if n_good < 4:
        drafts[n_good] = (drafts[n_good] + 1) % cfg.vocab
    toks = [g0] + drafts
    seq_out = [seq.decode(t) for t in toks]
    ver = Runner(cfg, tiny, dev)
    ver.prefill(prompt)
    vg, n_acc, vl = ver.verify(toks)
    assert vg == [s[0] for s in seq_out]
    assert np.array_equal(vl.view(np.uint32), np.stack([s[1] for s in seq_out]).view(np.uint32))
    assert n_acc == n_good + 1
    # the next decode reads the verify's appended (8-bit) rows of the accepted positions
    seq2 = Runner(cfg, tiny, dev)
    seq2.prefill(prompt)
    for t in toks[:n_acc]:
        seq2.decode(t)
    a, b = ver.decode(vg[n_acc - 1]), seq2.decode(vg[n_acc - 1])
    assert a[0] == b[0] and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    for x in (seq, ver, seq2):
        x.close()


# ---------------------------------------------------------------------------------- 24 layers
@pytest.fixture(scope="module")
def big_weights():
    return W.make_weights(W.HYBRID_24L_Q8, seed=0)


def test_24L_q8_ragged_prompt_matches_live_oracle(dev, big_weights):
    """The hidden-1024 kernels with the 8-bit cache against the live oracle: a prompt of two
    chunks + 2 tokens, then three chained greedy steps."""
    cfg = W.HYBRID_24L_Q8
    prompt = W.make_prompt(cfg, 130, seed=41)
    ref_toks, ref_logits = OracleModel(cfg, big_weights, C2).generate(prompt, 3)
    r = Runner(cfg, big_weights, dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros((4, cfg.vocab), dtype=torch.float32, device=dev)
    r.m.prefill(i32(prompt, dev), nxt, logits[0])
    outs = [nxt]
    for i in range(3):
        o = torch.zeros(1, dtype=torch.int32, device=dev)
        r.m.decode_step(outs[-1], o, logits[i + 1])
        outs.append(o)
    assert r.m.sync() == 133
    assert [int(o.item()) for o in outs] == list(ref_toks)
    for i in range(4):
        close(logits[i].cpu().numpy(), ref_logits[i], f"position {i}")
    r.close()


def test_24L_q8_cache_changes_the_result_but_little(dev, big_weights):
    """The 8-bit model is not silently run with the bf16 cache: its logits differ from the bf16
    model's, by quantisation noise only."""
    prompt = W.make_prompt(W.HYBRID_24L, 130, seed=41)
    a = Runner(W.HYBRID_24L_Q8, big_weights, dev)
    b = Runner(W.HYBRID_24L, big_weights, dev)
    (ga, la), (gb, lb) = a.prefill(prompt), b.prefill(prompt)
    (ga2, la2), (gb2, lb2) = a.decode(ga), b.decode(ga)
    for x, y in ((la, lb), (la2, lb2)):
        assert not np.array_equal(x.view(np.uint32), y.view(np.uint32))
        assert np.linalg.norm(x - y) / np.linalg.norm(y) < 5e-2
    a.close()
    b.close()


def test_24L_q8_verify_bit_identical_to_decode(dev, big_weights):
    cfg = W.HYBRID_24L_Q8
    prompt = W.make_prompt(cfg, 70, seed=31)
    drafts = W.make_drafts(cfg, 3, 5, seed=32)
    a = Runner(cfg, big_weights, dev)
    b = Runner(cfg, big_weights, dev)
    ga, _ = a.prefill(prompt)
    gb, _ = b.prefill(prompt)
    assert ga == gb
    t, consumed = ga, []
    for f in range(3):
        toks = [t] + drafts[f].tolist()
        vg, n_acc, vl = a.verify(toks)
        seq = [b.decode(x) for x in toks]
        assert vg == [s[0] for s in seq], f"forward {f}"
        assert np.array_equal(vl.view(np.uint32), np.stack([s[1] for s in seq]).view(np.uint32)), f"forward {f}"
        consumed += toks[:n_acc]
        b.m.reset()
        b.prefill(prompt)
        for x in consumed:
            b.decode(x)
        t = vg[n_acc - 1]
    a.close()
    b.close()


def golden(name):
    path = os.path.join(GOLDEN, name + ".npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_golden.py {name})")
    return dict(np.load(path, allow_pickle=False))


def test_24L_q8_long_context(dev, big_weights):
    """8192-token prompt with the 8-bit cache and 32 greedy steps against the stored oracle run:
    decode reads cached rows both from the prefetched registers and in the later grouped loads."""
    gd = golden("24L-q8-pp8192-tg32")
    cfg = W.HYBRID_24L_Q8
    prompt = W.make_prompt(cfg, 8192, seed=1)
    assert np.array_equal(prompt, gd["prompt"])
    n = len(gd["tokens"])
    r = Runner(cfg, big_weights, dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros((n, cfg.vocab), dtype=torch.float32, device=dev)
    r.m.prefill(i32(prompt, dev), nxt, logits[0])
    outs = [nxt]
    for i in range(n - 1):
        o = torch.zeros(1, dtype=torch.int32, device=dev)
        r.m.decode_step(outs[-1], o, logits[i + 1])
        outs.append(o)
    assert r.m.sync() == 8192 + n - 1
    toks = np.array([int(o.item()) for o in outs])
    lg = logits.cpu().numpy()
    mism = np.nonzero(toks != gd["tokens"])[0]
    if len(mism):
        i = int(mism[0])
        pytest.fail(f"greedy token mismatch at position {i}: gpu {toks[i]} oracle {gd['tokens'][i]}, "
                    f"oracle top-2 margin {gd['margin'][i]:.3e}")
    for i in range(n):
        close(lg[i][gd["sample_ids"]], gd["sample_logits"][i], f"position {i} (sampled ids)")
        close(lg[i][gd["top_ids"][i]], gd["top_vals"][i], f"position {i} (oracle top-8)")
    r.close()
