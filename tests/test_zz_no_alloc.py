"""mk_decode_step_static -- the decode/verify entry point that allocates nothing and takes no
workspace: its exchange slots live in a static device array -- against mk_decode_step, through
the C ABI.  The two run the same kernels with the same arithmetic, so argmax, logits and
n_accepted must agree bit for bit, on consecutive calls (the static array keeps the previous
call's slots; tags keep them apart) and with a narrower second call."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    import hybrid_deltanet_attention_persistent_amd as pkg
    pkg.load_library()
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def i32(x, dev):
    return torch.tensor(np.asarray(x, dtype=np.int32).reshape(-1), dtype=torch.int32, device=dev)


def step(lib, model, static, toks, dev, vocab):
    n = len(toks)
    am = torch.zeros(n, dtype=torch.int32, device=dev)
    lg = torch.zeros((n, vocab), dtype=torch.float32, device=dev)
    na = torch.zeros(1, dtype=torch.int32, device=dev)
    f = lib.mk_decode_step_static if static else lib.mk_decode_step
    f(model.handle, i32(toks, dev), n, am, lg, na if n > 1 else None)
    pos = model.sync()
    return am.cpu().numpy(), lg.cpu().numpy(), int(na.item()) if n > 1 else 1, pos


def bits_equal(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


def test_static_decode_matches_arena_decode_24L(dev):
    import hybrid_deltanet_attention_persistent_amd as pkg
    lib = pkg.lib
    cfg = W.HYBRID_24L
    w = W.make_weights(cfg, seed=0)
    a = pkg.Model(cfg, w, device=str(dev))
    b = pkg.Model(cfg, w, device=str(dev))
    del w
    prompt = i32(W.make_prompt(cfg, 40, seed=61), dev)
    ga = torch.zeros(1, dtype=torch.int32, device=dev)
    gb = torch.zeros(1, dtype=torch.int32, device=dev)
    a.prefill(prompt, ga)
    b.prefill(prompt, gb)
    assert a.sync() == b.sync() == 40
    t = int(ga.item())
    assert t == int(gb.item())
    for i in range(2):                            # two calls in a row on the static slots
        ra = step(lib, a, False, [t], dev, cfg.vocab)
        rb = step(lib, b, True, [t], dev, cfg.vocab)
        assert ra[0].tolist() == rb[0].tolist(), f"call {i}"
        assert bits_equal(ra[1], rb[1]), f"call {i}"
        assert ra[3] == rb[3] == 41 + i
        t = int(ra[0][0])
    # a verify forward of this model needs 5 x 14.2 MiB of slots: rejected before anything is
    # enqueued, the position stays where it was
    with pytest.raises(lib.MkError) as e:
        lib.mk_decode_step_static(b.handle, i32([t, 1, 2, 3, 4], dev), 5,
                                  torch.zeros(5, dtype=torch.int32, device=dev))
    assert e.value.status == lib.MK_EINVAL
    assert b.sync() == 42
    rb = step(lib, b, True, [t], dev, cfg.vocab)
    ra = step(lib, a, False, [t], dev, cfg.vocab)
    assert ra[0].tolist() == rb[0].tolist() and bits_equal(ra[1], rb[1])
    a.close()
    b.close()


def test_static_verify_matches_arena_verify_tiny(dev):
    """Tiny model: a 5-token verify, then a narrower 3-token one, then a decode step, on the static
    slots and on the arena's."""
    import hybrid_deltanet_attention_persistent_amd as pkg
    lib = pkg.lib
    cfg = W.TINY
    w = W.make_weights(cfg, seed=0)
    a = pkg.Model(cfg, w, device=str(dev))
    b = pkg.Model(cfg, w, device=str(dev))
    prompt = i32(W.make_prompt(cfg, 9, seed=62), dev)
    g = torch.zeros(1, dtype=torch.int32, device=dev)
    a.prefill(prompt, g)
    b.prefill(prompt, g)
    t = int(g.item())
    drafts = W.make_drafts(cfg, 2, 5, seed=63)
    pos = 9
    for width, d in ((5, drafts[0]), (3, drafts[1])):
        toks = [t] + d[:width - 1].tolist()
        ra = step(lib, a, False, toks, dev, cfg.vocab)
        rb = step(lib, b, True, toks, dev, cfg.vocab)
        assert ra[0].tolist() == rb[0].tolist(), f"width {width}"
        assert bits_equal(ra[1], rb[1]), f"width {width}"
        assert ra[2] == rb[2]
        pos += ra[2]
        assert ra[3] == rb[3] == pos
        t = int(ra[0][ra[2] - 1])
    ra = step(lib, a, False, [t], dev, cfg.vocab)
    rb = step(lib, b, True, [t], dev, cfg.vocab)
    assert ra[0].tolist() == rb[0].tolist() and bits_equal(ra[1], rb[1])
    a.close()
    b.close()
