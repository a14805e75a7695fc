"""GPU parity: full-KV verify attention against the oracle, batch invariance (row i
of a k-row window equals the 1-row call at context L + i, bit for bit), ragged
context lengths and determinism, through the C ABI."""
import numpy as np
import pytest
import torch

import lossy_kv_draft_amd as L
from workloads import configs as C, gen as G
from oracle import attention as OA
from gpu_util import assert_close, T, np32, tdtype, inputs, TOL, LSE_TOL, say

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_fp32": C.TINY,
    "llama8b": C.small(C.LLAMA8B, N=3000),                 # H=4, k=32: M=128
    "drop_k40": C.small(C.DROP, N=2500, Hkv=1, Hq=4),      # H=4, k=40: M=160 (one 8-wave block)
    "qwen30b_k40": C.small(C.QWEN30B, N=1100, Hkv=1, Hq=8),  # H=8, k=40: M=320 (one mixed 8-wave block)
    "qwen30b_k33": C.small(C.QWEN30B, N=1100, Hkv=1, Hq=8, k=33),  # M=264: mixed block, padding rows, one idle wave
    "qwen30b_k64": C.small(C.QWEN30B, N=900, Hkv=1, Hq=8, k=64),   # M=512: four 128-row 4-wave blocks
    "d64_k7": C.small(C.LLAMA8B, N=700, d=64, k=7),
}


def _cache(K, V, Kw, Vw, dt, extra=0):
    kc = np.concatenate([K, Kw, np.zeros(K.shape[:2] + (extra, K.shape[3]), np.float32)], 2)
    vc = np.concatenate([V, Vw, np.zeros(V.shape[:2] + (extra, V.shape[3]), np.float32)], 2)
    return T(kc, dt), T(vc, dt)


def _run(w, q, kc, vc, ctx, split=0, ctx_lens=None):
    dt = q.dtype
    B, Hq, k, d = q.shape
    out = torch.empty(B, Hq, k, d, device="cuda", dtype=dt)
    lse = torch.empty(B, Hq, k, device="cuda")
    L.vc_verify_attn_full(q, kc, vc, ctx, out, lse=lse, split_tokens=split, ctx_lens=ctx_lens)
    return out, lse


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("split", [0, 512])
def test_verify_matches_oracle(name, split):
    w = SMALL[name]
    say(f"[verify] {name} split={split}")
    K, V, Q, Kw, Vw = inputs(w)
    dt = tdtype(w.dtype)
    kc, vc = _cache(K, V, Kw, Vw, dt, extra=3)
    out, lse = _run(w, T(Q, dt), kc, vc, w.N, split)
    torch.cuda.synchronize()
    for b in range(w.B):
        o, l = OA.verify_masked(Q[b], K[b], V[b], Kw[b], Vw[b], w.d ** -0.5)
        assert_close(np32(out[b]), o, w.dtype, f"b={b}")
        assert np.abs(np32(lse[b]) - l).max() <= LSE_TOL[w.dtype]


@pytest.mark.parametrize("name", ["tiny_fp32", "llama8b", "drop_k40", "qwen30b_k40", "qwen30b_k33", "qwen30b_k64", "d64_k7"])
def test_verify_batch_invariance(name):
    """Row i of the k-row window == the 1-row call with context L + i (same split
    size), bit for bit; this is what makes verified output identical to greedy
    decoding done with the same kernel."""
    w = SMALL[name]
    K, V, Q, Kw, Vw = inputs(w)
    dt = tdtype(w.dtype)
    kc, vc = _cache(K, V, Kw, Vw, dt)
    split = L.vc_verify_split_tokens(w.B, w.Hkv, kc.shape[2])
    q = T(Q, dt)
    out, lse = _run(w, q, kc, vc, w.N, split)
    for i in [0, 1, w.k // 2, w.k - 1]:
        o1, l1 = _run(w, q[:, :, i:i + 1].contiguous(), kc, vc, w.N + i, split)
        torch.cuda.synchronize()
        assert torch.equal(o1[:, :, 0], out[:, :, i]), f"row {i} differs"
        assert torch.equal(l1[:, :, 0], lse[:, :, i])


@pytest.mark.parametrize("base", ["llama8b", "drop_k40"])
@pytest.mark.parametrize("split", [0, 256])
def test_verify_ragged_context_lengths(base, split):
    """Per-sequence context lengths (one of them empty), with 128 rows per kv-head
    (4-wave blocks) and 160 (one 8-wave block); the default split and 256-row splits
    (6 of them: the merge's one-round path, with the splits past a short sequence's end
    empty)."""
    w = C.small(C.LLAMA8B if base == "llama8b" else C.DROP, B=3, N=1500, **({} if base == "llama8b" else {"Hkv": 1, "Hq": 4}))
    say(f"[verify ragged] {base} split={split}")
    K, V, Q, Kw, Vw = inputs(w)
    lens = [1500, 700, 0]
    cap = 1500 + w.k
    kc = np.zeros((w.B, w.Hkv, cap, w.d), np.float32)
    vc = np.zeros_like(kc)
    for b, Lb in enumerate(lens):
        kc[b, :, :Lb], vc[b, :, :Lb] = K[b, :, :Lb], V[b, :, :Lb]
        kc[b, :, Lb:Lb + w.k], vc[b, :, Lb:Lb + w.k] = Kw[b], Vw[b]
    out, lse = _run(w, T(Q, torch.bfloat16), T(kc, torch.bfloat16), T(vc, torch.bfloat16), 1500, split,
                    ctx_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for b, Lb in enumerate(lens):
        o, l = OA.verify_masked(Q[b], K[b, :, :Lb], V[b, :, :Lb], Kw[b], Vw[b], w.d ** -0.5)
        assert_close(np32(out[b]), o, 'bf16')
        assert np.abs(np32(lse[b]) - l).max() <= LSE_TOL["bf16"]


def test_verify_ctx_lens_above_ctx_len_are_clamped():
    """ctx_len is the call's longest context (it sizes the splits and the workspace);
    an entry of ctx_lens above it reads as ctx_len: the output equals the call with
    that entry lowered to ctx_len, bit for bit, and the oracle at that length."""
    w = C.small(C.LLAMA8B, B=2, N=1500)
    K, V, Q, Kw, Vw = inputs(w)
    Lc = 1000
    rows = w.N + w.k + 600
    rng = np.random.default_rng(11)
    kc = rng.standard_normal((w.B, w.Hkv, rows, w.d)).astype(np.float32)   # rows past the window: noise
    vc = rng.standard_normal((w.B, w.Hkv, rows, w.d)).astype(np.float32)
    kc[:, :, :Lc], vc[:, :, :Lc] = K[:, :, :Lc], V[:, :, :Lc]
    kc[:, :, Lc:Lc + w.k], vc[:, :, Lc:Lc + w.k] = Kw, Vw
    kc, vc = G.to_storage(kc, "bf16"), G.to_storage(vc, "bf16")
    q = T(Q, torch.bfloat16)
    kd, vd = T(kc, torch.bfloat16), T(vc, torch.bfloat16)
    lens = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")
    a, la = _run(w, q, kd, vd, Lc, ctx_lens=lens([Lc + 700, Lc]))
    b, lb = _run(w, q, kd, vd, Lc, ctx_lens=lens([Lc, Lc]))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    for bb in range(w.B):
        o, l = OA.verify_masked(Q[bb], kc[bb, :, :Lc], vc[bb, :, :Lc], kc[bb, :, Lc:Lc + w.k], vc[bb, :, Lc:Lc + w.k],
                                w.d ** -0.5)
        assert_close(np32(a[bb]), o, 'bf16')
        assert np.abs(np32(la[bb]) - l).max() <= LSE_TOL["bf16"]


def test_verify_deterministic():
    w = SMALL["llama8b"]
    K, V, Q, Kw, Vw = inputs(w)
    kc, vc = _cache(K, V, Kw, Vw, torch.bfloat16)
    q = T(Q, torch.bfloat16)
    a, _ = _run(w, q, kc, vc, w.N)
    b, _ = _run(w, q, kc, vc, w.N)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["llama8b", "drop", "qwen30b"])
def test_full_size_verify_sampled_rows(name):
    """The benchmark's verify shapes at full size, in the launch configuration it
    times (Llama-3-8B-shaped 32k, k 32: 128 rows per kv-head; token-dropping 131k,
    k 40: 160 rows, one 8-wave block; Qwen-shaped 64k, k 40: 320 rows, one mixed
    8-wave block of 3- and 2-tile waves); sampled rows against the oracle."""
    w = {"llama8b": C.LLAMA8B, "drop": C.DROP, "qwen30b": C.QWEN30B}[name]
    dt = torch.bfloat16
    rows = w.N + w.k
    kc = torch.empty(w.B, w.Hkv, rows, w.d, dtype=dt, device="cuda")
    vc = torch.empty_like(kc)
    say(f"[full verify] {name}: generating inputs")
    for b in range(w.B):
        for h in range(w.Hkv):
            kc[b, h, :w.N] = T(G.kv_slice(w, "k", b, h), dt)
            vc[b, h, :w.N] = T(G.kv_slice(w, "v", b, h), dt)
            kc[b, h, w.N:] = T(G.window_kv(w, "k", b, h), dt)
            vc[b, h, w.N:] = T(G.window_kv(w, "v", b, h), dt)
    Q = G.full_window_q(w)
    out, _ = _run(w, T(Q, dt), kc, vc, w.N)
    torch.cuda.synchronize()
    del kc, vc
    rng = np.random.default_rng(3)
    grp = w.Hq // w.Hkv
    for _ in range(4):
        b, hq, i = int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.k))
        h = hq // grp
        say(f"[full verify] {name} b={b} hq={hq} row={i}")
        K, V = G.kv_slice(w, "k", b, h), G.kv_slice(w, "v", b, h)
        Kw, Vw = G.window_kv(w, "k", b, h), G.window_kv(w, "v", b, h)
        o, _ = OA.decode(Q[b, hq:hq + 1, i], K[None], V[None], w.d ** -0.5, Kw[None, :i + 1], Vw[None, :i + 1])
        assert_close(np32(out[b, hq, i]), o[0], 'bf16')
