"""GPU parity: head mean, greedy logits argmax (agreement on every non-tied row,
lowest index on exact ties) and prefix acceptance (bit exact), through the C ABI."""
import numpy as np
import pytest
import torch

import lossy_kv_draft_amd as L
from workloads import configs as C, gen as G
from oracle import logits as OL, accept as OC
from gpu_util import T, np32, say

pytestmark = pytest.mark.gpu


def test_head_mean_matches_oracle():
    w = C.small(C.LLAMA8B)
    o = G.normal(w, (1,), (w.B, w.Hq, w.k, w.d), dtype="bf16")
    u = torch.empty(w.B * w.k, w.d, device="cuda")
    L.vc_head_mean(T(o, torch.bfloat16), u)
    o3 = o[:, :, 0]
    u3 = torch.empty(w.B, w.d, device="cuda")
    L.vc_head_mean(T(o3, torch.bfloat16), u3)
    torch.cuda.synchronize()
    ref = OL.head_mean(np.moveaxis(o, 2, 1)).reshape(w.B * w.k, w.d)
    assert np.abs(np32(u) - ref).max() < 1e-5
    assert np.abs(np32(u3) - OL.head_mean(o3)).max() < 1e-5


def _tie_eps(u, W):
    """Bound on |GPU logit - exact logit| per row: u is split into two bf16 parts
    (relative error <= 2^-16 per element) and accumulated in float32 (<= K 2^-24
    of sum |u||W|), doubled for the two logits compared."""
    K = u.shape[1]
    mag = np.abs(u) @ np.abs(W.astype(np.float64)).T
    return 2 * (2.0 ** -15 + K * 2.0 ** -23) * mag.max(axis=1)


@pytest.mark.parametrize("case", ["f32_64x1000", "bf16_128x151936", "bf16_64x5000", "bf16u_128x3001"])
def test_logits_argmax_agrees_on_untied_rows(case):
    u_dt = torch.float32
    if case == "f32_64x1000":
        w, R, Wd = C.TINY, 40, "f32"
        W = G.projection(w)
    elif case == "bf16_128x151936":
        w, R, Wd = C.QWEN30B, 640, "bf16"
        W = G.projection(w)
    elif case == "bf16_64x5000":
        w, R, Wd = C.TINY, 100, "bf16"
        W = G.normal(w, (3,), (5000, 64), dtype="bf16")
    else:  # bf16 u (one product per step), ragged row and vocabulary counts
        w, R, Wd = C.TINY, 37, "bf16"
        W = G.normal(w, (6,), (3001, 128), dtype="bf16")
        u_dt = torch.bfloat16
    say(f"[argmax] {case}")
    u = G.normal(w, (2, len(case), R), (R, W.shape[1]), std=0.05, dtype="bf16" if u_dt == torch.bfloat16 else "f32")
    tok = torch.empty(R, dtype=torch.int32, device="cuda")
    L.vc_logits_argmax(T(u, u_dt), T(W, torch.float32 if Wd == "f32" else torch.bfloat16), tok)
    torch.cuda.synchronize()
    got = tok.cpu().numpy()
    lg = OL.logits(u, W)
    ref = OL.argmax_lowest(lg)
    eps = _tie_eps(u, W)
    gap = lg[np.arange(R), ref] - lg[np.arange(R), got]
    assert np.all(gap >= 0)
    untied = ~(gap <= eps)
    assert np.array_equal(got[untied], ref[untied]) if untied.any() else True
    assert (got == ref).mean() > 0.95


def test_logits_argmax_exact_ties_take_lowest_index():
    w = C.TINY
    W = G.normal(w, (4,), (3000, 128), dtype="bf16")
    u = G.normal(w, (5,), (20, 128))
    best = OL.argmax_lowest(OL.logits(u, W))
    # duplicate each row's winner at a higher and a lower index: the lower copy must win
    for r, j in enumerate(best[:5]):
        W[2990 - r] = W[j]
        W[r] = W[j]
    tok = torch.empty(20, dtype=torch.int32, device="cuda")
    L.vc_logits_argmax(T(u), T(W, torch.bfloat16), tok)
    torch.cuda.synchronize()
    got = tok.cpu().numpy()
    ref = OL.argmax_lowest(OL.logits(u, W))
    for r in range(5):
        assert got[r] == min(np.flatnonzero(np.all(W == W[ref[r]], axis=1)))


@pytest.mark.parametrize("k", [1, 5, 32, 40, 64])
def test_accept_bit_exact(k):
    w = C.small(C.QWEN30B, B=16)
    rng = np.random.default_rng(k)
    tgt = rng.integers(0, 50, size=(16, k)).astype(np.int32)
    dr = tgt.copy()
    for b in range(16):
        cut = int(rng.integers(0, k + 1))      # planted first mismatch (k = none)
        if cut < k:
            dr[b, cut] = (tgt[b, cut] + 1 + int(rng.integers(49))) % 50
            dr[b, cut + 1:] = rng.integers(0, 50, size=k - cut - 1)
    a = torch.empty(16, dtype=torch.int32, device="cuda")
    n = torch.empty_like(a)
    c = torch.empty(16, k, dtype=torch.int32, device="cuda")
    L.vc_accept(T(dr, torch.int32), T(tgt, torch.int32), a, n, c)
    torch.cuda.synchronize()
    ra, rn, rc = OC.accept(dr, tgt)
    assert np.array_equal(a.cpu().numpy(), ra)
    assert np.array_equal(n.cpu().numpy(), rn)
    assert np.array_equal(c.cpu().numpy(), rc)
