"""Host logic of the weight-free lookup draft (mk_lookup_draft in include/mk.h), through the C ABI,
no GPU: hand-worked cases and a brute-force restatement of the rule on random short histories.

The rule ("lookup-augmented draft", RTX 3090 tag page; drafts checked by verify with greedy
output unchanged, speed section of the page "업데이트: 단일 RTX 3090에서 Qwen 3.8 27B를 140 tok/s로
구동"): the longest suffix of the history, of length ngram_max down to ngram_min, that occurs
earlier; at its most recent earlier occurrence, the tokens that followed it, at most max_draft.
"""
import numpy as np
import pytest

import hybrid_deltanet_attention_persistent_amd as pkg


@pytest.fixture(scope="module")
def lib():
    return pkg.load_library()


def brute(h, gmin, gmax, max_draft):
    n = len(h)
    for g in range(min(gmax, n - 1), gmin - 1, -1):
        starts = [i for i in range(0, n - g) if list(h[i:i + g]) == list(h[n - g:])]
        if starts:
            i = max(starts)
            return list(h[i + g:i + g + max_draft])
    return []


@pytest.mark.parametrize("h, gmin, gmax, k, want", [
    ([1, 2, 3, 4, 1, 2], 1, 3, 4, [3, 4, 1, 2]),        # suffix [1 2] seen at 0
    ([1, 2, 3, 4, 1, 2], 1, 3, 2, [3, 4]),              # capped at max_draft
    ([5, 6, 7], 1, 3, 4, []),                           # nothing recurs
    ([1, 2, 3, 1, 2, 3, 1, 2], 1, 3, 4, [3, 1, 2]),     # suffix [3 1 2]: most recent earlier start 2, history ends
    ([9, 1, 7, 2, 1, 7, 3, 1, 7], 2, 2, 4, [3, 1, 7]),  # [1 7] last seen at 4 (not at 1)
    ([4, 8, 1, 9, 8, 1], 1, 3, 3, [9, 8, 1]),           # longest suffix [8 1] (not [1]) decides
    ([4, 8, 1, 9, 2, 1], 2, 3, 3, []),                  # [2 1] never seen before; g = 1 not allowed
    ([4, 8, 1, 9, 2, 1], 1, 3, 3, [9, 2, 1]),           # g = 1: [1] last seen at 2
    ([3, 3, 3, 3], 1, 3, 4, [3]),                       # overlapping occurrence, one token follows it
    ([7], 1, 3, 4, []),
    ([], 1, 3, 4, []),
])
def test_hand_cases(lib, h, gmin, gmax, k, want):
    assert pkg.mk_lookup_draft(h, gmin, gmax, k) == want
    assert brute(h, gmin, gmax, k) == want


def test_matches_brute_force_on_random_histories(lib):
    rng = np.random.default_rng(7)
    for trial in range(400):
        n = int(rng.integers(0, 40))
        h = rng.integers(0, int(rng.integers(2, 6)), size=n).tolist()
        gmin = int(rng.integers(1, 3))
        gmax = gmin + int(rng.integers(0, 3))
        k = int(rng.integers(0, 5))
        assert pkg.mk_lookup_draft(h, gmin, gmax, k) == brute(h, gmin, gmax, k), (h, gmin, gmax, k)


@pytest.mark.parametrize("gmin, gmax, k", [(0, 3, 4), (3, 2, 4), (1, 3, -1)])
def test_bad_arguments_rejected(lib, gmin, gmax, k):
    with pytest.raises(pkg.MkError) as e:
        pkg.mk_lookup_draft([1, 2, 1, 2], gmin, gmax, k)
    assert e.value.status == pkg.lib.MK_EINVAL
