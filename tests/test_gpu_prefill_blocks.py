"""Prefill in two row blocks (the second on a side stream, one step behind the first) against the
one-block prefill, through the C ABI.

The split is at a 64-token chunk boundary, so the delta rule's chunks, every projection's
accumulation order and attention's key blocks are those of the one-block form: the logits, the
greedy token and the state left for decode must agree bit for bit.  The cases cover prompts at
position 0 and at unaligned positions (the conv history and RoPE positions of the second block),
a prompt spanning two passes, a prefill right after a partial verify (the pending delta-rule
updates are replayed by the first block only), the 8-bit KV cache, and the 24-layer model at the
pp520 prompt against the live oracle.
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


class Runner:
    def __init__(self, cfg, weights, dev, blocks):
        import hybrid_deltanet_attention_persistent_amd as pkg
        self.cfg, self.dev = cfg, dev
        self.m = pkg.Model(cfg, weights, device=str(dev))
        self.m.set_prefill_blocks(blocks)
        self.tok = torch.zeros(5, dtype=torch.int32, device=dev)
        self.lg = torch.zeros((5, cfg.vocab), dtype=torch.float32, device=dev)
        self.nacc = torch.zeros(1, dtype=torch.int32, device=dev)

    def prefill(self, prompt):
        self.m.prefill(i32(prompt, self.dev), self.tok[:1], self.lg[0])
        assert self.m.sync() >= len(prompt)
        return int(self.tok[0].item()), self.lg[0].cpu().numpy().copy()

    def decode(self, t):
        self.m.decode_step(i32([t], self.dev), self.tok[:1], self.lg[0])
        self.m.sync()
        return int(self.tok[0].item()), self.lg[0].cpu().numpy().copy()

    def verify(self, toks):
        n = len(toks)
        self.m.decode_step(i32(toks, self.dev), self.tok[:n], self.lg[:n], self.nacc)
        self.m.sync()
        return self.tok[:n].cpu().numpy().tolist(), int(self.nacc.item()), self.lg[:n].cpu().numpy().copy()

    def close(self):
        self.m.close()


def same(a, b, what):
    assert a[0] == b[0], f"{what}: token {a[0]} != {b[0]}"
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32)), \
        f"{what}: logits differ, max |d| {np.max(np.abs(a[1] - b[1])):.3e}"


def run_pair(cfg, weights, dev, prompts, steps=3):
    """The same prompts (in successive calls) and greedy steps on a one-block and a two-block model."""
    one, two = Runner(cfg, weights, dev, 1), Runner(cfg, weights, dev, 2)
    outs = []
    for j, p in enumerate(prompts):
        a, b = one.prefill(p), two.prefill(p)
        same(a, b, f"prefill {j} ({len(p)} tokens)")
        outs.append(a)
    t = outs[-1][0]
    for i in range(steps):
        a, b = one.decode(t), two.decode(t)
        same(a, b, f"decode {i}")
        t = a[0]
    one.close()
    two.close()
    return outs


@pytest.fixture(scope="module")
def tiny():
    return W.make_weights(W.TINY, seed=0)


@pytest.mark.parametrize("lens", [[256], [300], [37, 300], [5, 1100], [100, 256, 513]])
def test_tiny_two_blocks_bit_identical(dev, tiny, lens):
    cfg = dataclasses.replace(W.TINY, max_ctx=2048)
    prompts = [W.make_prompt(cfg, n, seed=70 + j) for j, n in enumerate(lens)]
    run_pair(cfg, tiny, dev, prompts)


def test_tiny_two_blocks_match_oracle(dev, tiny):
    cfg = dataclasses.replace(W.TINY, max_ctx=1024)
    prompts = [W.make_prompt(cfg, 21, seed=80), W.make_prompt(cfg, 389, seed=81)]
    ref = OracleModel(cfg, tiny, C2)
    r = Runner(cfg, tiny, dev, 2)
    for j, p in enumerate(prompts):
        g, lg = r.prefill(p)
        rl = ref.prefill(p)
        close(lg, rl, f"prefill {j}")
        assert g == argmax_lowest(rl)
    for i in range(3):
        g2, lg = r.decode(g)
        rl = ref.decode(g)
        close(lg, rl, f"decode {i}")
        g = g2
        assert g == argmax_lowest(rl)
    r.close()


def test_tiny_two_blocks_after_partial_verify(dev, tiny):
    """A 300-token prefill right after a verify with 2 pending updates: the first block replays
    them, the second must not; bit-identical to one block and equal to the oracle."""
    cfg = dataclasses.replace(W.TINY, max_ctx=1024)
    prompt = W.make_prompt(cfg, 13, seed=31)
    probe = OracleModel(cfg, tiny, C2)
    t = argmax_lowest(probe.prefill(prompt))
    d1 = argmax_lowest(probe.decode(t))
    d2 = argmax_lowest(probe.decode(d1))
    toks = [t, d1, d2, (d2 + 7) % cfg.vocab, 11]
    more = W.make_prompt(cfg, 300, seed=32)
    ref = OracleModel(cfg, tiny, C2)
    ref.prefill(prompt)
    rg, rn, _ = ref.verify(toks)
    rl = ref.prefill(more)
    res = []
    for blocks in (1, 2):
        r = Runner(cfg, tiny, dev, blocks)
        r.prefill(prompt)
        vg, n_acc, _ = r.verify(toks)
        assert n_acc == rn == 3 and vg == rg
        res.append(r.prefill(more))
        res.append(r.decode(res[-1][0]))
        r.close()
    same(res[0], res[2], "prefill after verify")
    same(res[1], res[3], "decode after it")
    close(res[2][1], rl, "prefill after verify (oracle)")
    assert res[2][0] == argmax_lowest(rl)


def test_tiny_q8_two_blocks_bit_identical(dev):
    cfg = dataclasses.replace(W.TINY_Q8, max_ctx=1024)
    weights = W.make_weights(W.TINY_Q8, seed=0)
    run_pair(cfg, weights, dev, [W.make_prompt(cfg, 19, seed=90), W.make_prompt(cfg, 333, seed=91)])


def test_rejects_bad_block_count(dev, tiny):
    import hybrid_deltanet_attention_persistent_amd as pkg
    m = pkg.Model(W.TINY, tiny, device=str(dev))
    for bad in (0, 3, -1):
        with pytest.raises(pkg.MkError):
            m.set_prefill_blocks(bad)
    m.close()


def test_24L_pp520_two_blocks_bit_identical_and_match_oracle(dev):
    cfg = W.HYBRID_24L
    weights = W.make_weights(cfg, seed=0)
    prompt = W.make_prompt(cfg, 520, seed=1)
    outs = run_pair(cfg, weights, dev, [prompt], steps=2)
    ref = OracleModel(cfg, weights, C2)
    rl = ref.prefill(prompt)
    close(outs[0][1], rl, "pp520 prefill logits (every one of the vocabulary)")
    assert outs[0][0] == argmax_lowest(rl)


def test_decode_after_kernels_on_another_stream(dev, tiny):
    """Kernels on a second hardware queue move the XCD the dispatcher starts its round-robin
    placement from (measured: workgroup 0 no longer lands on XCD 0).  The persistent kernel reads
    its XCD from the hardware, so decode and verify after such work still match the oracle."""
    cfg = W.TINY
    s2 = torch.cuda.Stream()
    a = torch.ones(1 << 16, device=dev)
    with torch.cuda.stream(s2):
        for _ in range(3):
            a.add_(1.0)
    ev = torch.cuda.Event()
    ev.record(s2)
    torch.cuda.current_stream().wait_event(ev)
    prompt = W.make_prompt(cfg, 16, seed=1)
    ref_toks, ref_logits = OracleModel(cfg, tiny, C2).generate(prompt, 6)
    r = Runner(cfg, tiny, dev, 2)
    g, lg = r.prefill(prompt)
    got = [g]
    close(lg, ref_logits[0], "prefill")
    for i in range(6):
        g, lg = r.decode(g)
        got.append(g)
        close(lg, ref_logits[i + 1], f"decode {i}")
    assert got == list(ref_toks)
    r.close()


def test_24L_pp1024_two_blocks_bit_identical_and_match_oracle(dev):
    """A full 1024-token pass: two row blocks of 512 (64 x 256 GEMM tiles, grids of more than one
    wave of workgroups), bit-identical to one block and equal to the live oracle over the whole
    vocabulary."""
    cfg = W.HYBRID_24L
    weights = W.make_weights(cfg, seed=0)
    prompt = W.make_prompt(cfg, 1024, seed=1)
    outs = run_pair(cfg, weights, dev, [prompt], steps=1)
    rl = OracleModel(cfg, weights, C2).prefill(prompt)
    close(outs[0][1], rl, "pp1024 prefill logits")
    assert outs[0][0] == argmax_lowest(rl)
