"""Pins of the oracle's token-drop scoring/selection, greedy argmax and prefix
acceptance: invariants, brute force and library routines."""
import itertools
import os.path
import numpy as np
import pytest
import torch

from oracle import drop as D, accept as AC, logits as LG, attention as A


def test_scores_sum_to_number_of_probes_and_match_torch_softmax():
    rng = np.random.default_rng(0)
    K = rng.standard_normal((500, 32))
    P = rng.standard_normal((9, 32))
    s = D.scores(K, P, 32 ** -0.5)
    assert np.isclose(s.sum(), 9.0, atol=1e-10)
    ref = torch.softmax(torch.from_numpy(P @ K.T * 32 ** -0.5), dim=-1).sum(0).numpy()
    assert np.max(np.abs(s - ref)) < 1e-13


def test_equal_keys_keep_lowest_indices():
    K = np.ones((40, 8))
    P = np.random.default_rng(1).standard_normal((4, 8))
    s = D.scores(K, P, 1.0)
    assert np.allclose(s, 4 / 40)
    assert list(D.select(s, 10)) == list(range(10))


def test_heavy_hitter_is_kept():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((64, 16))
    P = rng.standard_normal((8, 16)) + 3.0
    K[45] = 4.0
    s = D.scores(K, P, 0.25)
    assert 45 in D.select(s, 4)


@pytest.mark.parametrize("seed", range(5))
def test_select_matches_brute_force_ranking(seed):
    rng = np.random.default_rng(seed)
    N = 60
    s = rng.integers(0, 7, size=N).astype(np.float32)   # many ties
    keep = D.n_keep(N, 0.25)
    brute = sorted(range(N), key=lambda n: (-float(s[n]), n))[:keep]
    got = D.select(s, keep)
    assert list(got) == sorted(brute)
    kept = set(got.tolist())
    dropped = [n for n in range(N) if n not in kept]
    assert min(s[list(kept)]) >= max(s[dropped])


def test_n_keep():
    assert D.n_keep(131072, 0.25) == 32768
    assert D.n_keep(10, 0.25) == 3
    assert D.n_keep(8, 1.0) == 8


def test_keep_all_gather_is_dense_bitwise():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((2, 64, 16)).astype(np.float32)
    V = rng.standard_normal((2, 64, 16)).astype(np.float32)
    q = rng.standard_normal((4, 16)).astype(np.float32)
    idx = [D.select(D.scores(K[h], q[:2], 0.25), 64) for h in range(2)]
    Kg = np.stack([D.gather(K[h], idx[h]) for h in range(2)])
    Vg = np.stack([D.gather(V[h], idx[h]) for h in range(2)])
    assert np.array_equal(Kg, K) and np.array_equal(Vg, V)
    o1, l1 = A.decode(q, Kg, Vg, 0.25)
    o2, l2 = A.decode(q, K, V, 0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_argmax_ties_go_to_lowest_index():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [0.0, -1.0, 0.5, 0.5]])
    assert list(LG.argmax_lowest(x)) == [1, 0, 2]
    rng = np.random.default_rng(4)
    y = rng.integers(0, 5, size=(50, 30)).astype(np.float64)
    assert np.array_equal(LG.argmax_lowest(y), np.argmax(y, axis=-1))


def test_tokens_from_outputs_uses_head_mean():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((2, 4, 3, 8))
    W = rng.standard_normal((20, 8))
    t = LG.tokens_from_outputs(o, W)
    for b in range(2):
        for i in range(3):
            u = sum(o[b, h, i] for h in range(4)) / 4
            assert t[b, i] == int(np.argmax(W @ u))


def test_accept_brute_force_all_short_strings():
    for k in range(1, 6):
        for dr in itertools.product(range(3), repeat=k):
            for tg in itertools.product(range(3), repeat=k):
                a, n, c = AC.accept_row(list(dr), list(tg))
                pre = os.path.commonprefix([list(dr), list(tg)])
                assert a == len(pre)
                expect = list(pre) + ([tg[a]] if a < k else [])
                assert c == expect and n == len(expect)
                # committed tokens always equal the target's greedy tokens
                assert c == list(tg[: n])


def test_accept_batched_layout():
    d = np.array([[1, 2, 3, 4], [1, 2, 3, 4], [9, 2, 3, 4]])
    t = np.array([[1, 2, 3, 4], [1, 2, 0, 4], [1, 2, 3, 4]])
    a, n, c = AC.accept(d, t)
    assert list(a) == [4, 2, 0] and list(n) == [4, 3, 1]
    assert c.tolist() == [[1, 2, 3, 4], [1, 2, 0, -1], [1, -1, -1, -1]]
    assert [AC.cache_advance(x, 4) for x in a] == [4, 3, 1]
