"""Pins of the oracle decoder and its draft-and-verify round: torch's rms_norm and
silu, rotary invariants and a hand-computed rotation, causal consistency of cached
forward passes, and the pages' invariant that draft-and-verify output equals greedy
full-KV decoding for any drafter."""
import numpy as np
import pytest
import torch

from oracle import model as M


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 48))
    w = rng.standard_normal(48)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(w), eps=1e-5).numpy()
    assert np.max(np.abs(M.rmsnorm(x, w) - ref)) < 1e-12


def test_silu_matches_torch():
    x = np.linspace(-20, 20, 401)
    assert np.max(np.abs(M.silu(x) - torch.nn.functional.silu(torch.from_numpy(x)).numpy())) < 1e-12


def test_rope_hand_rotation_and_invariants():
    # hd = 2: the single pair rotates by pos * theta^0 = pos radians
    x = np.array([[[1.0, 0.0]]])
    y = M.rope(x, np.array([1.0]), theta=10000.0)
    assert np.allclose(y[0, 0], [np.cos(1.0), np.sin(1.0)], atol=1e-15)
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 3, 16))
    k = rng.standard_normal((5, 3, 16))
    assert np.allclose(M.rope(q, np.zeros(5)), q)                                 # position 0: identity
    qr = M.rope(q, np.arange(5) + 3)
    assert np.allclose(np.linalg.norm(qr, axis=-1), np.linalg.norm(q, axis=-1))  # rotation keeps norms
    # scores depend on the position difference only
    p1, p2, s = np.array([7.0] * 5), np.array([2.0] * 5), 11.0
    d1 = np.sum(M.rope(q, p1) * M.rope(k, p2), axis=-1)
    d2 = np.sum(M.rope(q, p1 + s) * M.rope(k, p2 + s), axis=-1)
    assert np.allclose(d1, d2, atol=1e-12)
    # the pair (j, j + hd/2) of frequency index j turns by pos * theta^(-2j/hd)
    x = np.zeros((1, 1, 8))
    x[0, 0, 1] = 1.0
    y = M.rope(x, np.array([3.0]), theta=100.0)
    ang = 3.0 * 100.0 ** (-2.0 / 8)
    assert np.allclose([y[0, 0, 1], y[0, 0, 5]], [np.cos(ang), np.sin(ang)], atol=1e-15)


CFG = M.Config(layers=2, d_model=64, Hq=4, Hkv=2, hd=16, ffn=96, vocab=50)


def _dec(seed=0, std=0.3):
    return M.Decoder(CFG, M.random_weights(CFG, np.random.default_rng(seed), std=std))


def test_cached_forward_is_causally_consistent():
    """Processing tokens one at a time with a growing cache gives the same logits as
    processing them together."""
    dec = _dec(1)
    rng = np.random.default_rng(2)
    toks = list(rng.integers(0, CFG.vocab, size=12))
    empty = [(np.zeros((CFG.Hkv, 0, CFG.hd)), np.zeros((CFG.Hkv, 0, CFG.hd))) for _ in range(CFG.layers)]
    lg_all, _ = dec.forward_full(toks, 0, empty)
    kv = empty
    for i, t in enumerate(toks):
        lg, new = dec.forward_full([t], i, kv)
        kv = [(np.concatenate([K, nk], 1), np.concatenate([V, nv], 1)) for (K, V), (nk, nv) in zip(kv, new)]
        assert np.allclose(lg[0], lg_all[i], atol=1e-11)


def test_draft_on_uncompressed_cache_equals_full_forward():
    """With 16-bit float32-scale quantization of nothing (all rows in the tail) the
    draft forward is the full forward."""
    dec = _dec(3)
    rng = np.random.default_rng(4)
    prompt = list(rng.integers(0, CFG.vocab, size=9))
    kv, tok = M.prefill(dec, prompt)
    ccache = [(np.zeros((CFG.Hkv, 0, CFG.hd)), np.zeros((CFG.Hkv, 0, CFG.hd)), K.copy(), V.copy()) for K, V in kv]
    lg_d = dec.forward_draft(tok, len(prompt), ccache)
    lg_f, _ = dec.forward_full([tok], len(prompt), kv)
    assert np.allclose(lg_d, lg_f[0], atol=1e-11)


@pytest.mark.parametrize("drafter", ["compressed", "adversarial", "perfect"])
@pytest.mark.parametrize("seed", [0, 1])
def test_vericache_output_equals_greedy(drafter, seed):
    dec = _dec(10 + seed)
    rng = np.random.default_rng(20 + seed)
    prompt = list(rng.integers(0, CFG.vocab, size=37))
    T, k = 40, 6
    ref = M.greedy(dec, prompt, T)
    st = M.RoundStats()
    got = M.vericache(dec, prompt, T, k, bits=(2, 2), group=8, drafter=drafter, rng=rng, stats=st)
    assert got == ref
    if drafter == "perfect":
        assert all(a == k for a in st.accept_lens)
    if drafter == "adversarial":
        assert st.rounds >= (T - 1) // 2   # random drafts are almost never accepted


def test_compressed_drafts_are_not_all_exact():
    """The 2-bit compressed drafter does diverge sometimes (so the verification
    actually corrects it) while still producing the greedy output."""
    dec = _dec(30)
    rng = np.random.default_rng(31)
    prompt = list(rng.integers(0, CFG.vocab, size=40))
    st = M.RoundStats()
    got = M.vericache(dec, prompt, 60, 8, bits=(2, 2), group=8, drafter="compressed", stats=st)
    assert got == M.greedy(dec, prompt, 60)
    assert min(st.accept_lens) < 8
