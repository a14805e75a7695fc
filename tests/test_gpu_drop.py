"""GPU parity: token-drop scoring (tolerance), top-k selection (bit exact on the
same float32 scores; on GPU-computed scores exact outside the near-threshold band),
row gather (bit exact) and decode over the kept rows, through the C ABI."""
import numpy as np
import pytest
import torch

import lossy_kv_draft_amd as L
from workloads import configs as C, gen as G
from oracle import drop as OD, attention as OA
from gpu_util import LSE_TOL, assert_close, T, np32, say, TOL

pytestmark = pytest.mark.gpu

SMALL = C.small(C.DROP, N=5000)   # 3 scoring chunks, ragged last chunk


def _scores_oracle(w, K, P):
    return np.stack([np.stack([OD.scores(K[b, h], P[h], w.d ** -0.5) for h in range(w.Hkv)]) for b in range(w.B)])


def test_drop_scores_match_oracle():
    w = SMALL
    K = G.full_kv(w, "k")
    P = G.full_probes(w)
    sc = torch.empty(w.B, w.Hkv, w.N, device="cuda")
    L.vc_drop_scores(T(K, torch.bfloat16), T(P, torch.bfloat16), sc)
    torch.cuda.synchronize()
    ref = _scores_oracle(w, K, P)
    got = np32(sc)
    assert np.abs(got - ref).max() <= 1e-5 * ref.max() + 1e-9
    assert np.allclose(got.sum(axis=-1), w.n_probes, rtol=1e-4)


# single-slice and multi-slice (8192 scores per selecting workgroup; 25093 ends in a
# ragged slice) sizes; step 0.5 leaves a handful of distinct scores, so the threshold's
# equal scores span several slices and are cut part-way through one
@pytest.mark.parametrize("N,keep,step", [(5000, 1250, 8), (4096, 1024, 8), (777, 1, 8), (777, 777, 8),
                                         (300, 299, 8), (25093, 6274, 8), (25093, 1, 8), (25093, 25093, 8),
                                         (25093, 25092, 8), (16384, 4096, 8), (25093, 9001, 0.5)])
def test_drop_select_bit_exact_on_same_scores(N, keep, step):
    """The oracle's scores, rounded to float32 and coarsened to force many exact ties,
    are the input of both selections."""
    w = SMALL.with_(N=N)
    rng = np.random.default_rng(N + keep)
    s = rng.gamma(2.0, 1.0, size=(w.B, w.Hkv, N)).astype(np.float32)
    s = np.round(s * step) / step               # many ties
    s = s.astype(np.float32)
    kept = torch.empty(w.B, w.Hkv, keep, dtype=torch.int32, device="cuda")
    L.vc_drop_select(T(s), keep, kept)
    torch.cuda.synchronize()
    got = kept.cpu().numpy()
    for b in range(w.B):
        for h in range(w.Hkv):
            assert np.array_equal(got[b, h], OD.select(s[b, h], keep)), (b, h)


@pytest.mark.parametrize("keep", [1, 700, 1999])
def test_drop_select_mixed_sign_zeros_and_nan(keep):
    """Scores of either sign with many ties, -0.0 next to +0.0 (equal scores), -inf and
    NaNs (ranked below every other score): the kept set equals the oracle's."""
    w = SMALL.with_(N=2000)
    rng = np.random.default_rng(keep)
    s = (np.round(rng.standard_normal((w.B, w.Hkv, w.N)) * 4) / 4).astype(np.float32)
    s[..., 10], s[..., 11], s[..., 12], s[..., 13] = -0.0, 0.0, np.nan, -np.inf
    s[..., 14] = np.float32(-np.nan)
    s[..., 1500:1520] = 0.0
    s[..., 1520:1540] = -0.0
    kept = torch.empty(w.B, w.Hkv, keep, dtype=torch.int32, device="cuda")
    L.vc_drop_select(T(s), keep, kept)
    torch.cuda.synchronize()
    got = kept.cpu().numpy()
    for b in range(w.B):
        for h in range(w.Hkv):
            assert np.array_equal(got[b, h], OD.select(s[b, h], keep)), (b, h)


@pytest.mark.parametrize("d", [128, 48])  # rows of 16 (a power of two) and of 6 16-byte pieces
def test_gather_rows_bit_exact(d):
    w = SMALL
    K = G.full_kv(w, "k")[..., :d]
    idx = np.sort(np.random.default_rng(1).choice(w.N, size=(w.B, w.Hkv, 100), replace=True), axis=-1)
    dst = torch.zeros(w.B, w.Hkv, 128, d, dtype=torch.bfloat16, device="cuda")
    L.vc_gather_rows(T(K, torch.bfloat16), T(idx, torch.int32), 100, dst)
    torch.cuda.synchronize()
    got = np32(dst)
    for b in range(w.B):
        for h in range(w.Hkv):
            assert np.array_equal(got[b, h, :100], OD.gather(K[b, h], idx[b, h]))
            assert np.all(got[b, h, 100:] == 0)


def test_compress_drop_end_to_end_and_decode():
    w = SMALL
    say(f"[drop] B{w.B} Hkv{w.Hkv} N{w.N} keep {w.keep_ratio}")
    K, V = G.full_kv(w, "k"), G.full_kv(w, "v")
    P = G.full_probes(w)
    keep = OD.n_keep(w.N, w.keep_ratio)
    assert L.vc_drop_keep_count(w.keep_ratio, w.N) == keep
    ckv = L.Ckv("drop", w.B, w.Hkv, w.d, keep, keep_ratio=w.keep_ratio, kv_dtype="bf16")
    Kd, Vd = T(K, torch.bfloat16), T(V, torch.bfloat16)
    L.vc_compress(ckv, Kd, Vd, probes=T(P, torch.bfloat16))
    ckv.n_main = keep
    torch.cuda.synchronize()
    ref_scores = _scores_oracle(w, K, P)
    idx = ckv.kept_idx.cpu().numpy()
    kk, vk = np32(ckv.k_kept), np32(ckv.v_kept)
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = OD.select(ref_scores[b, h], keep)
            s = ref_scores[b, h]
            thr = np.sort(s)[::-1][keep - 1]
            band = np.abs(s - thr) <= 1e-6 * s.max()
            # outside the near-threshold band both selections agree exactly
            g, r = np.zeros(w.N, bool), np.zeros(w.N, bool)
            g[idx[b, h]] = True
            r[ref] = True
            assert np.array_equal(g[~band], r[~band])
            assert np.all(np.diff(idx[b, h]) > 0) and g.sum() == keep
            assert np.array_equal(kk[b, h], K[b, h, idx[b, h]]) and np.array_equal(vk[b, h], V[b, h, idx[b, h]])
    # decode over the kept rows
    Q = G.full_window_q(w)[:, :, 0]
    out = torch.empty(w.B, w.Hq, w.d, device="cuda", dtype=torch.bfloat16)
    L.vc_decode_attn_compressed(ckv, T(Q, torch.bfloat16), out)
    torch.cuda.synchronize()
    for b in range(w.B):
        o, _ = OA.decode(Q[b], kk[b], vk[b], w.d ** -0.5)
        assert_close(np32(out[b]), o, 'bf16')


@pytest.mark.parametrize("tail", [1, 64, 97])
def test_kept_row_decode_with_tails(tail):
    """Decode over kept rows plus a full-precision tail (merged by the decode's merge
    kernel in chunks of 64 rows) against the oracle over the kept rows and the tail."""
    w = SMALL.with_(k=max(tail, 1))
    K, V = G.full_kv(w, "k"), G.full_kv(w, "v")
    P = G.full_probes(w)
    keep = OD.n_keep(w.N, w.keep_ratio)
    ckv = L.Ckv("drop", w.B, w.Hkv, w.d, keep, keep_ratio=w.keep_ratio, kv_dtype="bf16", tail_cap=tail)
    L.vc_compress(ckv, T(K, torch.bfloat16), T(V, torch.bfloat16), probes=T(P, torch.bfloat16))
    ckv.n_main = keep
    Kw, Vw = G.full_window_kv(w, "k"), G.full_window_kv(w, "v")
    Kw, Vw = np32(T(Kw, torch.bfloat16)), np32(T(Vw, torch.bfloat16))  # the bf16 values the kernel reads
    ckv.tail_len = tail
    ckv.tail_k[:] = T(Kw[:, :, :tail], torch.bfloat16)
    ckv.tail_v[:] = T(Vw[:, :, :tail], torch.bfloat16)
    say(f"[drop decode tail] tail={tail}")
    Q = G.full_window_q(w)[:, :, tail - 1]
    out = torch.empty(w.B, w.Hq, w.d, device="cuda", dtype=torch.bfloat16)
    L.vc_decode_attn_compressed(ckv, T(Q, torch.bfloat16), out)
    torch.cuda.synchronize()
    kk, vk = np32(ckv.k_kept), np32(ckv.v_kept)
    for b in range(w.B):
        o, _ = OA.decode(Q[b], kk[b], vk[b], w.d ** -0.5, Kw[b, :, :tail], Vw[b, :, :tail])
        assert_close(np32(out[b]), o, 'bf16', f"b={b}")


@pytest.mark.parametrize("case", ["f32_d128", "bf16_d64", "bf16_h32"])
def test_kept_row_decode_generic_kernel(case):
    """Decode over kept rows where the tile loop does not apply and the generic kernel
    runs: float32 caches, d = 64, or more than 16 q-heads per kv-head; with a 5-row
    tail, against the oracle over the kept rows and the tail."""
    base = SMALL.with_(N=2000, k=5)
    w = {"f32_d128": base, "bf16_d64": base.with_(d=64), "bf16_h32": base.with_(Hq=32, Hkv=1)}[case]
    kvdt = "f32" if case == "f32_d128" else "bf16"
    tdt = torch.float32 if kvdt == "f32" else torch.bfloat16
    tail = w.k
    say(f"[drop decode generic] {case}")
    K, V = G.full_kv(w, "k"), G.full_kv(w, "v")
    P = G.full_probes(w)
    keep = OD.n_keep(w.N, w.keep_ratio)
    ckv = L.Ckv("drop", w.B, w.Hkv, w.d, keep, keep_ratio=w.keep_ratio, kv_dtype=kvdt, tail_cap=tail)
    L.vc_compress(ckv, T(K, tdt), T(V, tdt), probes=T(P, torch.bfloat16))
    ckv.n_main = keep
    Kw, Vw = G.full_window_kv(w, "k"), G.full_window_kv(w, "v")
    Kw, Vw = np32(T(Kw, tdt)), np32(T(Vw, tdt))  # the stored values the kernel reads
    ckv.tail_len = tail
    ckv.tail_k[:] = T(Kw, tdt)
    ckv.tail_v[:] = T(Vw, tdt)
    Q = G.full_window_q(w)[:, :, tail - 1]
    out = torch.empty(w.B, w.Hq, w.d, device="cuda", dtype=tdt)
    L.vc_decode_attn_compressed(ckv, T(Q, tdt), out)
    torch.cuda.synchronize()
    kk, vk = np32(ckv.k_kept), np32(ckv.v_kept)
    for b in range(w.B):
        o, _ = OA.decode(Q[b], kk[b], vk[b], w.d ** -0.5, Kw[b], Vw[b])
        assert_close(np32(out[b]), o, kvdt, f"b={b}")


def test_kept_row_decode_ragged_lengths():
    """Per-sequence kept-row counts and tail lengths on the tile-loop decode: all kept
    rows, a prefix ending mid-tile, an empty sequence (zero output, log-sum-exp
    -inf) and one with no kept rows but a tail."""
    w = SMALL.with_(B=4, N=2000, k=5)
    K, V = G.full_kv(w, "k"), G.full_kv(w, "v")
    P = G.full_probes(w)
    keep = OD.n_keep(w.N, w.keep_ratio)
    ckv = L.Ckv("drop", w.B, w.Hkv, w.d, keep, keep_ratio=w.keep_ratio, kv_dtype="bf16", tail_cap=w.k)
    L.vc_compress(ckv, T(K, torch.bfloat16), T(V, torch.bfloat16), probes=T(P, torch.bfloat16))
    ckv.n_main = keep
    Kw, Vw = G.full_window_kv(w, "k"), G.full_window_kv(w, "v")
    Kw, Vw = np32(T(Kw, torch.bfloat16)), np32(T(Vw, torch.bfloat16))
    ckv.tail_len = w.k
    ckv.tail_k[:] = T(Kw, torch.bfloat16)
    ckv.tail_v[:] = T(Vw, torch.bfloat16)
    main = [keep, keep // 3 + 7, 0, 0]
    tl = [w.k, 2, 0, w.k]
    say(f"[drop decode ragged] main {main} tail {tl}")
    Q = G.full_window_q(w)[:, :, 0]
    out = torch.empty(w.B, w.Hq, w.d, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(w.B, w.Hq, device="cuda")
    L.vc_decode_attn_compressed(ckv, T(Q, torch.bfloat16), out, lse=lse,
                                main_lens=torch.tensor(main, dtype=torch.int32, device="cuda"),
                                tail_lens=torch.tensor(tl, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    kk, vk = np32(ckv.k_kept), np32(ckv.v_kept)
    for b in (0, 1, 3):
        o, l = OA.decode(Q[b], kk[b, :, :main[b]], vk[b, :, :main[b]], w.d ** -0.5, Kw[b, :, :tl[b]], Vw[b, :, :tl[b]])
        assert_close(np32(out[b]), o, 'bf16', f"b={b}")
        assert np.abs(np32(lse[b]) - l).max() <= LSE_TOL["bf16"]
    assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))


def test_keep_all_decode_equals_dense_decode():
    w = SMALL.with_(N=1000, keep_ratio=1.0)
    K, V = G.full_kv(w, "k"), G.full_kv(w, "v")
    P = G.full_probes(w)
    ckv = L.Ckv("drop", w.B, w.Hkv, w.d, w.N, keep_ratio=1.0, kv_dtype="bf16")
    L.vc_compress(ckv, T(K, torch.bfloat16), T(V, torch.bfloat16), probes=T(P, torch.bfloat16))
    ckv.n_main = w.N
    torch.cuda.synchronize()
    assert np.array_equal(ckv.kept_idx.cpu().numpy(), np.broadcast_to(np.arange(w.N), (w.B, w.Hkv, w.N)))
    assert torch.equal(ckv.k_kept, T(K, torch.bfloat16))


def test_full_size_kept_row_decode_sampled():
    """Decode over kept rows at the token-dropping workload's full size (B4, 32/8
    heads, 32768 kept rows of 131072, d 128) plus a ragged tail, in the launch
    configuration the benchmark times; sampled (sequence, q-head) outputs against
    the oracle.  The kept rows are seeded rows of the layer (the decode reads the
    gathered rows only; selection is checked on the reduced shapes above)."""
    w = C.DROP
    keep = L.vc_drop_keep_count(w.keep_ratio, w.N)
    tl = 17
    ckv = L.Ckv("drop", w.B, w.Hkv, w.d, keep, keep_ratio=w.keep_ratio, kv_dtype="bf16", tail_cap=w.k)
    say("[full drop decode] generating inputs")
    kept = {}
    for b in range(w.B):
        for h in range(w.Hkv):
            K, V = G.kv_slice(w, "k", b, h)[:keep], G.kv_slice(w, "v", b, h)[:keep]
            ckv.k_kept[b, h] = T(K, torch.bfloat16)
            ckv.v_kept[b, h] = T(V, torch.bfloat16)
            kept[b, h] = (np32(ckv.k_kept[b, h]), np32(ckv.v_kept[b, h]))
            ckv.tail_k[b, h] = T(G.window_kv(w, "k", b, h), torch.bfloat16)
            ckv.tail_v[b, h] = T(G.window_kv(w, "v", b, h), torch.bfloat16)
    ckv.n_main = keep
    ckv.tail_len = tl
    Q = G.full_window_q(w)[:, :, tl - 1]
    out = torch.empty(w.B, w.Hq, w.d, device="cuda", dtype=torch.bfloat16)
    L.vc_decode_attn_compressed(ckv, T(Q, torch.bfloat16), out)
    torch.cuda.synchronize()
    tk, tv = np32(ckv.tail_k), np32(ckv.tail_v)
    rng = np.random.default_rng(5)
    grp = w.Hq // w.Hkv
    for _ in range(4):
        b, hq = int(rng.integers(w.B)), int(rng.integers(w.Hq))
        h = hq // grp
        say(f"[full drop decode] b={b} hq={hq}")
        K, V = kept[b, h]
        o, _ = OA.decode(Q[b, hq:hq + 1], K[None], V[None], w.d ** -0.5, tk[b, h][None, :tl], tv[b, h][None, :tl])
        assert_close(np32(out[b, hq]), o[0], 'bf16')
