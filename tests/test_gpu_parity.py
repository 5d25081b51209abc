"""GPU parity of the persistent HIP forward pass against the CPU oracle, through the C ABI.

Bar (for every compared position): greedy token ids equal to the oracle's, and
logits within max |error| 3e-2 and relative L2 error 1e-2.  Verify forwards
must reproduce sequential decode steps bit for bit (speculative decoding is
exact: the greedy output is the main model's greedy choice -- page
"업데이트: 단일 RTX 3090에서 Qwen 3.8 27B를 140 tok/s로 구동", accuracy section).
The tiny model is compared against the oracle run in the test; the 24-layer
workloads against stored oracle outputs (tests/golden/make_golden.py).
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
    """Drives one loaded model through the C ABI and returns host copies."""

    def __init__(self, cfg, weights, dev):
        import hybrid_deltanet_attention_persistent_amd as pkg
        self.cfg, self.dev = cfg, dev
        self.m = pkg.Model(cfg, weights, device=str(dev))
        self.tok = torch.zeros(W.HYBRID_24L.max_verify, dtype=torch.int32, device=dev)
        self.lg = torch.zeros((W.HYBRID_24L.max_verify, cfg.vocab), dtype=torch.float32, device=dev)
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
    return W.make_weights(W.TINY, seed=0)


def test_tiny_generate_matches_oracle(dev, tiny):
    cfg = W.TINY
    prompt = W.make_prompt(cfg, 16, seed=1)
    ref_toks, ref_logits = OracleModel(cfg, tiny, C2).generate(prompt, 16)
    r = Runner(cfg, tiny, dev)
    # greedy decode chained on the device: each step reads the previous step's argmax buffer
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros((17, cfg.vocab), dtype=torch.float32, device=dev)
    r.m.prefill(i32(prompt, dev), nxt, logits[0])
    outs = [nxt]
    for i in range(16):
        o = torch.zeros(1, dtype=torch.int32, device=dev)
        r.m.decode_step(outs[-1], o, logits[i + 1])
        outs.append(o)
    assert r.m.sync() == 32
    toks = [int(o.item()) for o in outs]
    assert toks == list(ref_toks)
    for i in range(17):
        close(logits[i].cpu().numpy(), ref_logits[i], f"position {i}")
    r.close()


def test_tiny_teacher_forced_random_tokens(dev, tiny):
    cfg = W.TINY
    prompt = W.make_prompt(cfg, 5, seed=21)
    feed = W.make_prompt(cfg, 40, seed=22)
    ref = OracleModel(cfg, tiny, C2)
    r = Runner(cfg, tiny, dev)
    g, lg = r.prefill(prompt)
    rl = ref.prefill(prompt)
    close(lg, rl, "prefill")
    assert g == argmax_lowest(rl)
    for i, t in enumerate(feed):          # runs to position 45, past a conv ring wrap and many key blocks
        g, lg = r.decode(int(t))
        rl = ref.decode(int(t))
        close(lg, rl, f"step {i}")
        assert g == argmax_lowest(rl), f"step {i}"
    r.close()


def test_tiny_weights_from_device_memory(dev, tiny):
    """mk_tensor.on_device = 1: weights handed over as GPU tensors load to the same model, bit for bit."""
    cfg = W.TINY
    prompt = W.make_prompt(cfg, 16, seed=1)
    dw = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).to(dev) for k, v in tiny.items()}
    outs = []
    for weights in (tiny, dw):
        r = Runner(cfg, weights, dev)
        g, lg = r.prefill(prompt)
        g2, lg2 = r.decode(g)
        outs.append((g, lg, g2, lg2))
        r.close()
    a, b = outs
    assert a[0] == b[0] and a[2] == b[2]
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[3].view(np.uint32), b[3].view(np.uint32))


def test_tiny_nonunit_gains(dev):
    cfg = W.TINY
    w = W.make_weights(cfg, seed=3, gain_std=0.1)
    prompt = W.make_prompt(cfg, 9, seed=4)
    ref_toks, ref_logits = OracleModel(cfg, w, C2).generate(prompt, 6)
    r = Runner(cfg, w, dev)
    g, lg = r.prefill(prompt)
    toks, lgs = [g], [lg]
    for _ in range(6):
        g, lg = r.decode(toks[-1])
        toks.append(g)
        lgs.append(lg)
    assert toks == list(ref_toks)
    for i in range(7):
        close(lgs[i], ref_logits[i], f"position {i}")
    r.close()


def test_tiny_single_token_prefill_and_full_context(dev, tiny):
    cfg = W.TINY
    ref = OracleModel(cfg, tiny, C2)
    r = Runner(cfg, tiny, dev)
    g, lg = r.prefill([7])
    rl = ref.prefill([7])
    close(lg, rl, "1-token prefill")
    assert g == argmax_lowest(rl)
    prompt = W.make_prompt(cfg, 59, seed=5)
    g, lg = r.prefill(prompt)                 # a second prefill appends at position 1
    rl = ref.prefill(prompt)
    close(lg, rl, "appended prefill")
    gr = argmax_lowest(rl)
    assert g == gr
    for i in range(4):                        # positions 60..63: the context is then full
        g, lg = r.decode(gr)                  # teacher-forced with the oracle's tokens
        rl = ref.decode(gr)
        close(lg, rl, f"step {i}")
        gr = argmax_lowest(rl)
        assert g == gr
    assert r.m.sync() == cfg.max_ctx
    r.close()


def test_tiny_context_limit_and_bad_token(dev, tiny):
    cfg = W.TINY
    import hybrid_deltanet_attention_persistent_amd as pkg
    r = Runner(cfg, tiny, dev)
    prompt = W.make_prompt(cfg, 60, seed=6)
    g, _ = r.prefill(prompt)
    for _ in range(4):
        g, _ = r.decode(g)
    assert r.m.sync() == cfg.max_ctx
    with pytest.raises(pkg.MkError) as e:
        r.decode(g)
    assert e.value.status == pkg.lib.MK_ECTX
    r.m.reset()
    assert r.m.sync() == 0
    with pytest.raises(pkg.MkError) as e:        # token id checked on the device, reported at sync
        r.m.decode_step(i32([cfg.vocab + 5], dev), r.tok[:1], None)
        r.m.sync()
    assert e.value.status == pkg.lib.MK_ETOKEN
    r.m.reset()
    assert r.m.sync() == 0
    r.close()


def test_tiny_rejects_empty_and_oversized_calls(dev, tiny):
    """Zero tokens, or a decode/verify wider than max_verify, is MK_EINVAL before anything is
    enqueued: the position stays where it was and the model keeps working."""
    cfg = W.TINY
    import hybrid_deltanet_attention_persistent_amd as pkg
    r = Runner(cfg, tiny, dev)
    buf = i32(list(range(cfg.max_verify + 1)), dev)
    out = torch.zeros(cfg.max_verify + 1, dtype=torch.int32, device=dev)
    for n in (0, cfg.max_verify + 1):
        with pytest.raises(pkg.MkError) as e:
            r.m.decode_step(buf, out, None, None, n_tokens=n)
        assert e.value.status == pkg.lib.MK_EINVAL
    with pytest.raises(pkg.MkError) as e:
        r.m.prefill(buf[:0], out[:1])
    assert e.value.status == pkg.lib.MK_EINVAL
    assert r.m.sync() == 0
    prompt = W.make_prompt(cfg, 4, seed=3)
    g, lg = r.prefill(prompt)
    ref = OracleModel(cfg, tiny, C2)
    close(lg, ref.prefill(prompt), "prefill after rejected calls")
    assert r.m.sync() == 4
    r.close()


def test_tiny_reset_reproduces_bits(dev, tiny):
    cfg = W.TINY
    prompt = W.make_prompt(cfg, 16, seed=1)
    r = Runner(cfg, tiny, dev)
    runs = []
    for _ in range(2):
        g, lg = r.prefill(prompt)
        out = [lg]
        for _ in range(5):
            g, lg = r.decode(g)
            out.append(lg)
        runs.append(np.stack(out))
        r.m.reset()
    assert np.array_equal(runs[0].view(np.uint32), runs[1].view(np.uint32))
    r.close()


@pytest.mark.parametrize("width,n_good", [(2, 1), (3, 0), (3, 2), (4, 1), (4, 3)])
def test_tiny_verify_narrower_than_five(dev, tiny, width, n_good):
    """A verify forward of 2..4 tokens: per-position argmax and logits bit-identical to sequential
    decode steps, n_accepted = 1 + the drafts that match, position advanced by n_accepted."""
    cfg = W.TINY
    prompt = W.make_prompt(cfg, 13, seed=12)
    seq = Runner(cfg, tiny, dev)
    g0, _ = seq.prefill(prompt)
    ref = OracleModel(cfg, tiny, C2)
    ref.prefill(prompt)
    drafts, t = [], g0
    for _ in range(width - 1):
        t = argmax_lowest(ref.decode(t))
        drafts.append(t)
    if n_good < width - 1:
        drafts[n_good] = (drafts[n_good] + 1) % cfg.vocab
    toks = [g0] + drafts
    s = [seq.decode(x) for x in toks]
    ver = Runner(cfg, tiny, dev)
    ver.prefill(prompt)
    vg, n_acc, vl = ver.verify(toks)
    assert vg == [x[0] for x in s]
    assert np.array_equal(vl.view(np.uint32), np.stack([x[1] for x in s]).view(np.uint32))
    assert n_acc == n_good + 1
    assert ver.m.sync() == len(prompt) + n_acc
    seq.close()
    ver.close()


@pytest.mark.parametrize("n_good", [0, 1, 2, 3, 4])
def test_tiny_verify_is_bit_identical_to_sequential_decode(dev, tiny, n_good):
    cfg = W.TINY
    prompt = W.make_prompt(cfg, 11, seed=8)
    seq = Runner(cfg, tiny, dev)
    g0, _ = seq.prefill(prompt)
    # drafts: the greedy continuation, corrupted at position n_good (none if n_good == 4)
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
    seq_g, seq_l = [], []
    for t in toks:
        g, lg = seq.decode(t)
        seq_g.append(g)
        seq_l.append(lg)
    ver = Runner(cfg, tiny, dev)
    ver.prefill(prompt)
    vg, n_acc, vl = ver.verify(toks)
    assert vg == seq_g
    assert np.array_equal(vl.view(np.uint32), np.stack(seq_l).view(np.uint32))
    assert n_acc == n_good + 1
    assert ver.m.sync() == len(prompt) + n_acc
    # the state is exactly "after the accepted tokens": continue both and compare bits
    seq2 = Runner(cfg, tiny, dev)
    seq2.prefill(prompt)
    for t in toks[:n_acc]:
        seq2.decode(t)
    nxt = vg[n_acc - 1]
    a = ver.decode(nxt)
    b = seq2.decode(nxt)
    assert a[0] == b[0] and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    # and a second verify right after (pending updates replayed, then new ones recorded)
    toks2 = [a[0]] + W.make_drafts(cfg, 1, 5, seed=9)[0].tolist()
    v2 = ver.verify(toks2)
    s2 = [seq2.decode(t) for t in toks2]
    assert v2[0] == [s[0] for s in s2]
    assert np.array_equal(v2[2].view(np.uint32), np.stack([s[1] for s in s2]).view(np.uint32))
    for x in (seq, ver, seq2):
        x.close()


def test_tiny_prefill_after_partial_verify(dev, tiny):
    """A prefill right after a verify applies the verify's pending delta-rule updates first
    (the state must be "after the accepted tokens"), then continues from there."""
    cfg = W.TINY
    prompt = W.make_prompt(cfg, 13, seed=31)
    ref = OracleModel(cfg, tiny, C2)
    r = Runner(cfg, tiny, dev)
    g, _ = r.prefill(prompt)
    t = argmax_lowest(ref.prefill(prompt))
    assert g == t
    # drafts: two correct greedy tokens, then a wrong one -> 3 accepted, 2 pending updates
    probe = OracleModel(cfg, tiny, C2)
    probe.prefill(prompt)
    d1 = argmax_lowest(probe.decode(t))
    d2 = argmax_lowest(probe.decode(d1))
    toks = [t, d1, d2, (d2 + 7) % cfg.vocab, 11]
    vg, n_acc, vl = r.verify(toks)
    rg, rn, rl = ref.verify(toks)
    assert n_acc == rn == 3 and vg == rg
    for i in range(5):
        close(vl[i], rl[i], f"verify column {i}")
    more = W.make_prompt(cfg, 21, seed=32)
    g, lg = r.prefill(more)
    rl = ref.prefill(more)
    close(lg, rl, "prefill after verify")
    gr = argmax_lowest(rl)
    assert g == gr
    for i in range(3):
        g, lg = r.decode(gr)
        rl = ref.decode(gr)
        close(lg, rl, f"decode {i}")
        gr = argmax_lowest(rl)
        assert g == gr
    r.close()


@pytest.mark.parametrize("lens", [[63], [64], [65, 1], [129, 70]])
def test_tiny_prefill_ragged_chunks(dev, tiny, lens):
    """Prompt lengths around the 64-token delta-rule chunk, in one or two calls."""
    cfg = dataclasses_replace(W.TINY, max_ctx=256)
    ref = OracleModel(cfg, tiny, C2)
    r = Runner(cfg, tiny, dev)
    for j, n in enumerate(lens):
        prompt = W.make_prompt(cfg, n, seed=40 + j)
        g, lg = r.prefill(prompt)
        rl = ref.prefill(prompt)
        close(lg, rl, f"prefill {j} ({n} tokens)")
        assert g == argmax_lowest(rl)
    g, lg = r.decode(g)
    rl = ref.decode(argmax_lowest(rl))
    close(lg, rl, "decode after prefill")
    r.close()


def dataclasses_replace(cfg, **kw):
    import dataclasses
    return dataclasses.replace(cfg, **kw)


def test_tiny_prompt_spanning_two_passes(dev, tiny):
    """1100 prompt tokens: two prefill passes (1024 + 76) in one call, then a second call whose
    start is not chunk aligned, then decode."""
    cfg = dataclasses_replace(W.TINY, max_ctx=1536)
    ref = OracleModel(cfg, tiny, C2)
    r = Runner(cfg, tiny, dev)
    prompt = W.make_prompt(cfg, 1100, seed=51)
    g, lg = r.prefill(prompt)
    rl = ref.prefill(prompt)
    close(lg, rl, "1100-token prefill")
    assert g == argmax_lowest(rl)
    more = W.make_prompt(cfg, 300, seed=52)
    g, lg = r.prefill(more)
    rl = ref.prefill(more)
    close(lg, rl, "300-token prefill at position 1100")
    gr = argmax_lowest(rl)
    assert g == gr
    for i in range(3):
        g, lg = r.decode(gr)
        rl = ref.decode(gr)
        close(lg, rl, f"decode {i}")
        gr = argmax_lowest(rl)
        assert g == gr
    assert r.m.sync() == 1403
    r.close()


# ---------------------------------------------------------------------------------- 24-layer model
def golden(name):
    path = os.path.join(GOLDEN, name + ".npz")
    if not os.path.exists(path):
        pytest.skip(f"stored oracle outputs {name}.npz not generated")
    return dict(np.load(path, allow_pickle=False))


@pytest.fixture(scope="module")
def big_weights():
    return W.make_weights(W.HYBRID_24L, seed=0)


def check_golden_logits(lg, gd, i):
    close(lg[gd["sample_ids"]], gd["sample_logits"][i], f"position {i} (sampled ids)")
    close(lg[gd["top_ids"][i]], gd["top_vals"][i], f"position {i} (oracle top-8)")


def test_24L_pp520_tg128(dev, big_weights):
    gd = golden("24L-pp520-tg128")
    cfg = W.HYBRID_24L
    r = Runner(cfg, big_weights, dev)
    prompt = W.make_prompt(cfg, 520, seed=1)
    assert np.array_equal(prompt, gd["prompt"])
    n = len(gd["tokens"])
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros((n, cfg.vocab), dtype=torch.float32, device=dev)
    r.m.prefill(i32(prompt, dev), nxt, logits[0])
    outs = [nxt]
    for i in range(n - 1):                   # device-chained greedy decode, no host round trip
        o = torch.zeros(1, dtype=torch.int32, device=dev)
        r.m.decode_step(outs[-1], o, logits[i + 1])
        outs.append(o)
    assert r.m.sync() == 520 + n - 1
    toks = np.array([int(o.item()) for o in outs])
    lg = logits.cpu().numpy()
    mism = np.nonzero(toks != gd["tokens"])[0]
    if len(mism):
        i = int(mism[0])
        pytest.fail(f"greedy token mismatch at position {i}: gpu {toks[i]} oracle {gd['tokens'][i]}, "
                    f"oracle top-2 margin {gd['margin'][i]:.3e}")
    for i in range(n):
        check_golden_logits(lg[i], gd, i)
    r.close()


def test_24L_verify5(dev, big_weights):
    gd = golden("24L-pp520-verify5")
    cfg = W.HYBRID_24L
    r = Runner(cfg, big_weights, dev)
    prompt = W.make_prompt(cfg, 520, seed=1)
    g0, _ = r.prefill(prompt)
    assert g0 == gd["committed"][0]
    committed = [g0]
    for f in range(len(gd["fwd_tokens"])):
        toks = gd["fwd_tokens"][f].tolist()
        assert toks[0] == committed[-1]
        greedy, n_acc, lg = r.verify(toks)
        assert greedy == gd["fwd_greedy"][f].tolist(), f"forward {f}"
        assert n_acc == gd["fwd_nacc"][f], f"forward {f}"
        for j in range(len(toks)):
            close(lg[j][gd["sample_ids"]], gd["fwd_sample_logits"][f][j], f"forward {f} position {j}")
        committed += greedy[:n_acc]
    assert np.array_equal(np.array(committed), gd["committed"])
    r.close()


@pytest.mark.parametrize("plen", [1, 67, 130])
def test_24L_ragged_prompt_matches_live_oracle(dev, big_weights, plen):
    """The hidden-1024 kernels against the live oracle at prompt lengths off the 64-token chunk
    grid (one token, one chunk + 3, two chunks + 2), then three chained greedy steps."""
    cfg = W.HYBRID_24L
    prompt = W.make_prompt(cfg, plen, seed=41)
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
    assert r.m.sync() == plen + 3
    assert [int(o.item()) for o in outs] == list(ref_toks)
    for i in range(4):
        close(logits[i].cpu().numpy(), ref_logits[i], f"prompt {plen}, position {i}")
    r.close()


def test_24L_appended_prompt_matches_live_oracle(dev, big_weights):
    """A second prompt appended at an unaligned position (after a prompt and two decode steps):
    the prefill picks up the conv history, the delta-rule state and the KV cache where decode left
    them, on the hidden-1024 kernels."""
    cfg = W.HYBRID_24L
    p1, p2 = W.make_prompt(cfg, 67, seed=43), W.make_prompt(cfg, 45, seed=44)
    ref = OracleModel(cfg, big_weights, C2)
    r = Runner(cfg, big_weights, dev)
    checks = [(r.prefill(p1), ref.prefill(p1))]
    t = checks[-1][0][0]
    for _ in range(2):
        checks.append((r.decode(t), ref.decode(t)))
        t = checks[-1][0][0]
    checks.append((r.prefill(p2), ref.prefill(p2)))
    t = checks[-1][0][0]
    for _ in range(2):
        checks.append((r.decode(t), ref.decode(t)))
        t = checks[-1][0][0]
    for i, ((g, lg), rl) in enumerate(checks):
        assert g == argmax_lowest(rl), f"call {i}"
        close(lg, rl, f"call {i}")
    assert r.m.sync() == 67 + 2 + 45 + 2
    r.close()


def test_24L_verify_bit_identical_to_decode(dev, big_weights):
    cfg = W.HYBRID_24L
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
        b.m.reset()                           # bring b to the accepted prefix
        b.prefill(prompt)
        for x in consumed:
            b.decode(x)
        t = vg[n_acc - 1]
    assert a.m.sync() == b.m.sync() == len(prompt) + len(consumed)
    a.close()
    b.close()


def test_24L_long_context(dev, big_weights):
    gd = golden("24L-pp8192-tg128")
    cfg = W.HYBRID_24L
    r = Runner(cfg, big_weights, dev)
    prompt = W.make_prompt(cfg, 8192, seed=1)
    assert np.array_equal(prompt, gd["prompt"])
    n = len(gd["tokens"])
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
        check_golden_logits(lg[i], gd, i)
    r.close()


def test_24L_pp520_full_vocab_live_oracle(dev, big_weights):
    """The headline workload's prompt (520 seeded tokens) and two chained greedy steps on the
    hidden-1024 kernels, every one of the 151,936 logits against the live oracle."""
    cfg = W.HYBRID_24L
    prompt = W.make_prompt(cfg, 520, seed=1)
    ref_toks, ref_logits = OracleModel(cfg, big_weights, C2).generate(prompt, 2)
    r = Runner(cfg, big_weights, dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros((3, cfg.vocab), dtype=torch.float32, device=dev)
    r.m.prefill(i32(prompt, dev), nxt, logits[0])
    outs = [nxt]
    for i in range(2):
        o = torch.zeros(1, dtype=torch.int32, device=dev)
        r.m.decode_step(outs[-1], o, logits[i + 1])
        outs.append(o)
    assert r.m.sync() == 522
    assert [int(o.item()) for o in outs] == list(ref_toks)
    lg = logits.cpu().numpy()
    for i in range(3):
        close(lg[i], ref_logits[i], f"position {i} (all {cfg.vocab} logits)")
    r.close()


class SeqReplay:
    """Sequential single-token decode from the prompt over a given token history: the reference a
    verify forward must reproduce bit for bit."""

    def __init__(self, cfg, weights, dev, prompt):
        self.r = Runner(cfg, weights, dev)
        self.prompt = prompt

    def run(self, history, toks):
        """Reset, prefill the prompt, decode `history` (the committed tokens), then decode `toks`
        one at a time; returns [(greedy, logits)] for `toks`."""
        self.r.m.reset()
        self.r.prefill(self.prompt)
        for x in history:
            self.r.decode(x)
        return [self.r.decode(x) for x in toks]

    def close(self):
        self.r.close()


@pytest.mark.parametrize("n_acc1", [1, 2, 3, 4, 5])
def test_24L_planted_draft_verify(dev, big_weights, n_acc1):
    """Verify forwards on the hidden-1024 kernels with drafts planted from the oracle's greedy
    continuation, corrupted at one position, so that every n_accepted in 1..5 occurs: the first
    forward accepts n_acc1 tokens, the second (which first replays the n_acc1 pending delta-rule
    updates) accepts 6 - n_acc1 (5 when n_acc1 is 1).  Per position, argmax and logits must equal
    sequential decode steps bit for bit, and the oracle within the parity bar; after the second
    forward a decode step continues from exactly the accepted prefix."""
    cfg = W.HYBRID_24L
    prompt = W.make_prompt(cfg, 70, seed=31)
    ref = OracleModel(cfg, big_weights, C2)
    g_ref, _ = ref.generate(prompt, 11)            # g0 .. g11, the oracle's greedy continuation
    g_ref = [int(t) for t in g_ref]
    ver = Runner(cfg, big_weights, dev)
    seq = SeqReplay(cfg, big_weights, dev, prompt)
    g0, _ = ver.prefill(prompt)
    assert g0 == g_ref[0]
    ref = OracleModel(cfg, big_weights, C2)
    ref.prefill(prompt)
    committed = []                                   # tokens consumed after the prompt
    for f, want in enumerate([n_acc1, 6 - n_acc1 if n_acc1 > 1 else 5]):
        base = len(committed)
        toks = g_ref[base:base + 5]                  # [last accepted, 4 greedy drafts]
        if want < 5:                                 # corrupt draft `want` -> n_accepted == want
            toks[want] = (toks[want] + 1 + f) % cfg.vocab
        vg, n_acc, vl = ver.verify(toks)
        s = seq.run(committed, toks)
        assert vg == [x[0] for x in s], f"forward {f}"
        assert np.array_equal(vl.view(np.uint32), np.stack([x[1] for x in s]).view(np.uint32)), f"forward {f}"
        rg, rn, rl = ref.verify(toks)
        assert n_acc == rn == want, f"forward {f}: n_accepted {n_acc}, oracle {rn}, planted {want}"
        assert vg[:n_acc] == rg[:n_acc]
        for j in range(5):
            close(vl[j], rl[j], f"forward {f} position {j}")
        committed += toks[:n_acc]
        assert vg[n_acc - 1] == g_ref[len(committed)]
    assert ver.m.sync() == len(prompt) + len(committed)
    nxt = g_ref[len(committed)]
    a = ver.decode(nxt)
    b = seq.run(committed, [nxt])[0]
    assert a[0] == b[0] and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    rl = ref.decode(nxt)
    close(a[1], rl, "decode after the rollback")
    assert a[0] == argmax_lowest(rl)
    ver.close()
    seq.close()
