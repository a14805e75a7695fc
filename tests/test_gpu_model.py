"""GPU parity of the decoder-layer kernels (vc_model.h) against the oracle decoder's
functions, and of the end-to-end draft-and-verify round: its output must equal
greedy full-KV decoding with the same kernels, token for token ("VeriCache: Turning
Lossy KV Cache into Lossless LLM Inference", summary page, "Original abstract")."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, T, np32, storage_half_ulp, say
from workloads import configs as C, gen as G
from oracle import model as OM, quant as OQ
from oracle.logits import argmax_lowest

pytestmark = pytest.mark.gpu

L = pytest.importorskip("lossy_kv_draft_amd")
from lossy_kv_draft_amd import round as R  # noqa: E402

W = C.E2E


def bf16(x):
    return G.to_storage(np.asarray(x, np.float32), "bf16")


def rnd(key, shape, std=1.0):
    return G.normal(W, key, shape, std, "bf16")


# ---------------------------------------------------------------- single kernels

@pytest.mark.parametrize("M,N,K", [(1, 16, 32), (5, 40, 96), (37, 3072, 2048), (130, 72, 512)])
@pytest.mark.parametrize("out", ["f32", "bf16", "bf16+res"])
def test_gemm_matches_fp64(M, N, K, out):
    say(f"gemm M{M} N{N} K{K} {out}")
    a, w = rnd((1, M, K), (M, K)), rnd((2, N, K), (N, K), 0.05)
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    bound = 2.0 ** -22 * K * (np.abs(a).astype(np.float64) @ np.abs(w).astype(np.float64).T) + 1e-30
    A, Wt = T(a, torch.bfloat16), T(w, torch.bfloat16)
    if out == "f32":
        Cg = torch.empty(M, N, device=DEV)
        L.vc_gemm_bf16(A, Wt, Cg)
        err = np.abs(np32(Cg) - ref)
        assert (err <= bound).all(), f"max excess {(err - bound).max():.3g}"
        return
    res = None
    if out == "bf16+res":
        r = rnd((3, M, N), (M, N))
        ref = ref + r
        res = T(r, torch.bfloat16)
    Cg = torch.empty(M, N, device=DEV, dtype=torch.bfloat16)
    L.vc_gemm_bf16(A, Wt, Cg, R=res)
    err = np.abs(np32(Cg) - ref)
    tol = bound + storage_half_ulp(ref, "bf16") + 2.0 ** -24 * np.abs(ref)
    assert (err <= tol).all(), f"max excess {(err - tol).max():.3g}"


def test_gemm_in_place_residual():
    """x += h W^T with C and R the same buffer (the decoder's residual update)."""
    M, N, K = 9, 48, 64
    a, w, x = rnd((4, 0), (M, K)), rnd((4, 1), (N, K), 0.05), rnd((4, 2), (M, N))
    X = T(x, torch.bfloat16)
    L.vc_gemm_bf16(T(a, torch.bfloat16), T(w, torch.bfloat16), X, R=X)
    Y = torch.empty_like(X)
    L.vc_gemm_bf16(T(a, torch.bfloat16), T(w, torch.bfloat16), Y, R=T(x, torch.bfloat16))
    assert torch.equal(X, Y)


def test_gemm_rows_are_batch_invariant():
    """A row's result does not depend on how many rows are multiplied together --
    what makes the k-row verify pass equal to k one-row greedy steps."""
    N, K = 200, 1024
    a, w = rnd((5, 0), (130, K)), rnd((5, 1), (N, K), 0.05)
    A, Wt = T(a, torch.bfloat16), T(w, torch.bfloat16)
    full = torch.empty(130, N, device=DEV)
    L.vc_gemm_bf16(A, Wt, full)
    for m0, n in [(0, 1), (17, 1), (3, 4), (100, 30), (64, 66)]:
        part = torch.empty(n, N, device=DEV)
        L.vc_gemm_bf16(A[m0:m0 + n], Wt, part)
        assert torch.equal(part, full[m0:m0 + n]), (m0, n)


@pytest.mark.parametrize("M,d", [(1, 64), (7, 512), (33, 2048), (4, 4000)])
def test_rmsnorm_matches_oracle(M, d):
    x, w = rnd((6, M, d), (M, d), 3.0), bf16(1.0 + rnd((7, d), (d,), 0.1))
    ref = OM.rmsnorm(x, w)
    y = torch.empty(M, d, device=DEV, dtype=torch.bfloat16)
    L.vc_rmsnorm(T(x, torch.bfloat16), T(w, torch.bfloat16), y)
    err = np.abs(np32(y) - ref)
    tol = storage_half_ulp(ref, "bf16") + 1e-5 * np.abs(ref) + 1e-6
    assert (err <= tol).all(), f"max excess {(err - tol).max():.3g}"


@pytest.mark.parametrize("B,k,Hq,Hkv,hd,pos_max", [(1, 1, 4, 2, 128, 10), (3, 5, 16, 4, 128, 20000),
                                                   (2, 8, 6, 2, 64, 3000)])
def test_rope_qkv_matches_oracle(B, k, Hq, Hkv, hd, pos_max):
    say(f"rope B{B} k{k} Hq{Hq} Hkv{Hkv} hd{hd}")
    width = (Hq + 2 * Hkv) * hd
    qkv = rnd((8, B, k), (B * k, width))
    pos = G.uniform_ints(W, (8, B, k), (B * k,), 0, pos_max)
    rows = k + 12
    row0 = G.uniform_ints(W, (9, B, k), (B,), 0, rows - k + 1)
    q = torch.empty(B, Hq, k, hd, device=DEV, dtype=torch.bfloat16)
    kd = torch.zeros(B, Hkv, rows, hd, device=DEV, dtype=torch.bfloat16)
    vd = torch.zeros_like(kd)
    L.vc_rope_qkv(T(qkv, torch.bfloat16), B, k, Hq, Hkv, hd, T(pos, torch.int32), q, kd, vd, T(row0, torch.int32))
    x = qkv.reshape(B * k, Hq + 2 * Hkv, hd)
    rq = OM.rope(x[:, :Hq], pos)
    rk = OM.rope(x[:, Hq:Hq + Hkv], pos)
    # float32 angle: |error| <= pos * 2^-22 radians (product and exp2 rounding), times |pair|
    pair = np.sqrt(np.concatenate([x[..., : hd // 2] ** 2 + x[..., hd // 2:] ** 2] * 2, -1))
    ang_tol = (pos[:, None, None] + 1) * 2.0 ** -21 * pair
    gq = np32(q).transpose(0, 2, 1, 3).reshape(B * k, Hq, hd)
    tq = storage_half_ulp(rq, "bf16") + ang_tol[:, :Hq] + 1e-6
    assert (np.abs(gq - rq) <= tq).all()
    gk, gv = np32(kd), np32(vd)
    want_k = np.zeros_like(gk)
    want_v = np.zeros_like(gv)
    for b in range(B):
        for i in range(k):
            r = b * k + i
            want_k[b, :, row0[b] + i] = rk[r]
            want_v[b, :, row0[b] + i] = x[r, Hq + Hkv:]
    tk = storage_half_ulp(want_k, "bf16") + 1e-6
    for b in range(B):
        for i in range(k):
            tk[b, :, row0[b] + i] += ang_tol[b * k + i, Hq:Hq + Hkv]
    assert (np.abs(gk - want_k) <= tk).all()
    assert np.array_equal(gv, want_v)       # values are copied, untouched rows stay zero


def test_swiglu_matches_oracle():
    M, F = 5, 1000
    gu = rnd((10,), (M, 2 * F), 4.0)
    ref = OM.silu(gu[:, :F]) * gu[:, F:]
    out = torch.empty(M, F, device=DEV, dtype=torch.bfloat16)
    L.vc_swiglu(T(gu, torch.bfloat16), out)
    err = np.abs(np32(out) - ref)
    tol = storage_half_ulp(ref, "bf16") + 1e-5 * np.abs(ref) + 1e-6
    assert (err <= tol).all()


def test_embed_heads_to_rows_and_argmax_rows_exact():
    V, d = 50, 64
    E = rnd((11,), (V, d))
    toks = np.array([3, 0, 49, 7, 7, -1, 50], np.int64)
    x = torch.empty(len(toks), d, device=DEV, dtype=torch.bfloat16)
    L.vc_embed(T(E, torch.bfloat16), T(toks, torch.int32), x)
    want = np.where(((toks >= 0) & (toks < V))[:, None], E[np.clip(toks, 0, V - 1)], 0.0)
    assert np.array_equal(np32(x), want)
    o = rnd((12,), (2, 3, 4, 16))
    rows = torch.empty(8, 48, device=DEV, dtype=torch.bfloat16)
    L.vc_heads_to_rows(T(o, torch.bfloat16), rows)
    assert np.array_equal(np32(rows), o.transpose(0, 2, 1, 3).reshape(8, 48))
    lg = G.normal(W, (13,), (6, 1000), 1.0, "f32")
    lg[1, [5, 900]] = 50.0                                   # tie: lowest index wins
    lg[2, :] = 0.0
    lg[3, 999] = 1e9
    lg[4, [0, 1, 2]] = -1e9
    tk = torch.empty(6, dtype=torch.int32, device=DEV)
    L.vc_argmax_rows(T(lg), tk)
    assert list(tk.cpu().numpy()) == [argmax_lowest(r) for r in lg]


@pytest.mark.parametrize("V", [32000, 40000, 32003])
def test_argmax_rows_large_and_ragged(V):
    """Vocabularies past one sweep of the workgroup (40000 > 8 x 1024 x 4) and a row
    length that is not a multiple of 4 (the scalar path); planted ties far apart."""
    lg = G.normal(W, (15, V), (5, V), 1.0, "f32")
    lg[0, [7, V - 2]] = 40.0
    lg[1, [V - 1]] = 40.0
    lg[2, [4096, 4097, 30000]] = 40.0
    tk = torch.empty(5, dtype=torch.int32, device=DEV)
    L.vc_argmax_rows(T(lg), tk)
    assert list(tk.cpu().numpy()) == [argmax_lowest(r) for r in lg]


def test_copy_kv_rows_exact():
    B, Hkv, d, sr, dr = 3, 2, 128, 40, 20
    sk, sv = rnd((14, 0), (B, Hkv, sr, d)), rnd((14, 1), (B, Hkv, sr, d))
    s0, d0, cnt = np.array([0, 30, 5]), np.array([2, 10, 19]), np.array([4, 0, 1])
    dk = torch.zeros(B, Hkv, dr, d, device=DEV, dtype=torch.bfloat16)
    dv = torch.zeros_like(dk)
    i32 = lambda a: T(a, torch.int32)
    L.vc_copy_kv_rows(T(sk, torch.bfloat16), T(sv, torch.bfloat16), i32(s0), dk, dv, i32(d0), i32(cnt), 4)
    wk, wv = np.zeros((B, Hkv, dr, d)), np.zeros((B, Hkv, dr, d))
    for b in range(B):
        wk[b, :, d0[b]:d0[b] + cnt[b]] = sk[b, :, s0[b]:s0[b] + cnt[b]]
        wv[b, :, d0[b]:d0[b] + cnt[b]] = sv[b, :, s0[b]:s0[b] + cnt[b]]
    assert np.array_equal(np32(dk), wk) and np.array_equal(np32(dv), wv)


# ---------------------------------------------------------------- end to end

def _shape(w):
    return R.ModelShape(layers=w.layers, d_model=w.d_model, Hq=w.Hq, Hkv=w.Hkv, hd=w.d, ffn=w.ffn, vocab=w.vocab)


def _setup(w, std, chunk=512):
    shape = _shape(w)
    seed = lambda key, shp, s: G.normal(w, key, shp, s, "f32")
    wcpu = R.random_weights(shape, seed, std=std, device="cpu")
    prompt = G.tokens(w, 0, shape=(w.B, w.N), high=w.vocab)
    dec = R.DecoderGPU(shape, R.weights_to(wcpu, DEV), max_rows=w.B * max(w.k, chunk))
    sess = R.Session(dec, prompt, w.k, w.gen_tokens, chunk=chunk, group=w.group, bits=(w.k_bits, w.v_bits))
    return shape, wcpu, prompt, dec, sess


SMALL = W.with_(B=3, Hq=4, Hkv=2, N=300, k=8, layers=2, d_model=512, ffn=1024, vocab=1000, gen_tokens=40)


def test_decoder_prefill_logits_match_oracle():
    """The composed decoder (all kernels chained, prompt through chunked verify
    attention) against the float64 oracle decoder on the same bf16 weights; bf16
    activations between the kernels bound the agreement (relative L2 norm)."""
    w = SMALL
    shape, wcpu, prompt, dec, sess = _setup(w, std=0.08, chunk=128)
    odec = _oracle_decoder(shape, wcpu)
    got = np32(sess.first_logits)
    first = sess.first.cpu().numpy()
    empty = [(np.zeros((shape.Hkv, 0, shape.hd)), np.zeros((shape.Hkv, 0, shape.hd))) for _ in range(shape.layers)]
    for b in range(w.B):
        lg, _ = odec.forward_full(list(prompt[b]), 0, empty)
        ref = lg[-1]
        rel = np.linalg.norm(got[b] - ref) / np.linalg.norm(ref)
        say(f"seq {b}: relative L2 error of the logits {rel:.3g}")
        assert rel < 0.03
        top2 = np.sort(ref)[-2:]
        if top2[1] - top2[0] > 0.1 * np.abs(ref).max():
            assert first[b] == argmax_lowest(ref)


def _oracle_decoder(shape, wcpu):
    f = lambda t: t.double().numpy()
    ow = OM.Weights(E=f(wcpu["E"]), wqkv=[f(x) for x in wcpu["wqkv"]], wo=[f(x) for x in wcpu["wo"]],
                    wgu=[f(x) for x in wcpu["wgu"]], wd=[f(x) for x in wcpu["wd"]], n1=[f(x) for x in wcpu["n1"]],
                    n2=[f(x) for x in wcpu["n2"]], nf=f(wcpu["nf"]), head=f(wcpu["head"]))
    return OM.Decoder(OM.Config(shape.layers, shape.d_model, shape.Hq, shape.Hkv, shape.hd, shape.ffn, shape.vocab),
                      ow)


def _small_model(std):
    w = SMALL
    shape = _shape(w)
    wcpu = R.random_weights(shape, lambda key, shp, s: G.normal(w, key, shp, s, "f32"), std=std, device="cpu")
    return w, shape, wcpu, _oracle_decoder(shape, wcpu)


def _rel(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("std", [0.02, 0.08])
def test_draft_forward_matches_oracle(std):
    """One draft step of the composed decoder (rotary at the next position, append to
    the tail, decode attention over 2-bit groups + tail, per-sequence lengths) against
    the oracle's draft forward on the same seeded caches."""
    w, shape, wcpu, odec = _small_model(std)
    B, Gs, hd, Hkv = 2, w.group, shape.hd, shape.Hkv
    m, t = [256, 192], [5, 17]
    cap, tcap = 256, 24
    kv = [[G.normal(w, (20, l, b, j), (Hkv, m[b] + t[b], hd), 1.0, "bf16") for j in range(2)]
          for l in range(shape.layers) for b in range(B)]
    kv = [kv[l * B:(l + 1) * B] for l in range(shape.layers)]
    tokens = np.array([17, 933])
    dec = R.DecoderGPU(shape, R.weights_to(wcpu, DEV), max_rows=8)
    ckvs = []
    for l in range(shape.layers):
        c = L.Ckv("quant", B, Hkv, hd, cap, k_bits=2, v_bits=2, group=Gs, param_dtype="bf16", kv_dtype="bf16",
                  tail_cap=tcap, device=DEV)
        src = [np.zeros((B, Hkv, cap, hd), np.float32) for _ in range(2)]
        for b in range(B):
            for j in range(2):
                src[j][b, :, : m[b]] = kv[l][b][j][:, : m[b]]
                getattr(c, "tail_k" if j == 0 else "tail_v")[b, :, : t[b]] = T(kv[l][b][j][:, m[b]:], torch.bfloat16)
        L.vc_compress(c, T(src[0], torch.bfloat16), T(src[1], torch.bfloat16), n_tokens=cap)
        c.n_main, c.tail_len = cap, tcap
        ckvs.append(c)
    i32 = lambda a: T(np.asarray(a), torch.int32)
    pos = i32([m[b] + t[b] for b in range(B)])
    ws = L.workspace(L.vc_decode_workspace_bytes(ckvs[0], shape.Hq), DEV)
    attend = R.attend_draft(dec, ckvs, B, pos, i32(t), i32(m), i32([x + 1 for x in t]), ws)
    got = np32(dec.forward(i32(tokens), B, 1, attend))
    for b in range(B):
        occ = []
        for l in range(shape.layers):
            K, V = kv[l][b]
            Kh, Vh = np.zeros((Hkv, m[b], hd)), np.zeros((Hkv, m[b], hd))
            for h in range(Hkv):
                for g0 in range(0, m[b], Gs):
                    cs = OQ.compress_slice(K[h, g0:g0 + Gs], V[h, g0:g0 + Gs], 2, 2, Gs, "bf16")
                    Kh[h, g0:g0 + Gs], Vh[h, g0:g0 + Gs] = OQ.dequantize_slice(cs, hd, 2, 2, Gs)
            occ.append((Kh, Vh, K[:, m[b]:].astype(np.float64), V[:, m[b]:].astype(np.float64)))
        ref = odec.forward_draft(int(tokens[b]), m[b] + t[b], occ)
        rel = _rel(got[b], ref)
        say(f"draft seq {b}: relative L2 error {rel:.3g}")
        assert rel < 0.03


@pytest.mark.parametrize("std", [0.02, 0.08])
def test_verify_forward_matches_oracle(std):
    """The k-row verify pass of the composed decoder (rotary at positions L_b + i,
    window keys/values written at rows L_b + i, causal attention over the full cache,
    per-sequence context lengths) against the oracle's full forward."""
    w, shape, wcpu, odec = _small_model(std)
    B, k, hd, Hkv = 2, 6, shape.hd, shape.Hkv
    Lb = [300, 131]
    rows = 320
    kv = [[G.normal(w, (21, l, b, j), (Hkv, Lb[b], hd), 1.0, "bf16") for j in range(2)]
          for l in range(shape.layers) for b in range(B)]
    kv = [kv[l * B:(l + 1) * B] for l in range(shape.layers)]
    toks = G.uniform_ints(w, (22,), (B, k), 0, shape.vocab)
    cache = R.FullCache(shape, B, rows, DEV)
    for l in range(shape.layers):
        for b in range(B):
            cache.k[l][b, :, : Lb[b]] = T(kv[l][b][0], torch.bfloat16)
            cache.v[l][b, :, : Lb[b]] = T(kv[l][b][1], torch.bfloat16)
    split = L.vc_verify_split_tokens(B, Hkv, rows)
    ws = L.workspace(L.vc_verify_workspace_bytes(B, shape.Hq, Hkv, hd, k, rows, split), DEV)
    dec = R.DecoderGPU(shape, R.weights_to(wcpu, DEV), max_rows=B * k)
    i32 = lambda a: T(np.asarray(a), torch.int32)
    vpos = i32((np.array(Lb)[:, None] + np.arange(k)[None, :]).reshape(-1))
    row0 = i32(Lb)
    attend = R.attend_full(dec, cache, B, k, vpos, row0, max(Lb), row0, split, ws)
    got = np32(dec.forward(i32(toks.reshape(-1)), B, k, attend)).reshape(B, k, -1)
    for b in range(B):
        okv = [(kv[l][b][0].astype(np.float64), kv[l][b][1].astype(np.float64)) for l in range(shape.layers)]
        ref, _ = odec.forward_full(list(toks[b]), Lb[b], okv)
        for i in range(k):
            rel = _rel(got[b, i], ref[i])
            assert rel < 0.03, (b, i, rel)
        say(f"verify seq {b}: max relative L2 error {max(_rel(got[b, i], ref[i]) for i in range(k)):.3g}")


@pytest.mark.parametrize("slots,graph", [(1, True), (2, False), (None, True)])
def test_round_output_equals_greedy_small(slots, graph):
    """slots: device layer slots of the staged full KV (1: a ring smaller than the
    model, 2: every layer staged during drafting, None: full KV resident); graph:
    draft loop captured as a HIP graph or launched step by step."""
    w = SMALL
    _, _, _, dec, sess = _setup(w, std=0.08, chunk=128)
    ref = R.Greedy(sess).run()
    assert np.array_equal(R.Greedy(sess, graph=False).run(), ref)
    staged = R.Greedy(sess, slots=1).run(12)
    assert np.array_equal(staged, ref[:, :12])
    loop = R.VeriCacheLoop(sess, slots=slots, graph=graph)
    got = loop.run()
    say(f"rounds {loop.rounds}, mean accept {np.mean(loop.accept_lens):.2f}")
    assert np.array_equal(got, ref)
    assert loop.rounds < w.gen_tokens          # drafts are accepted at least sometimes


def test_staggered_batches_equal_greedy():
    """Two batches decoded at once by Staggered (one host thread and compute stream
    each, full KV staged through one device slot each): each batch's output equals its
    own greedy output, and equals the same loop run alone."""
    w = SMALL
    shape = _shape(w)
    seed = lambda key, shp, s: G.normal(w, key, shp, s, "f32")
    weights = R.weights_to(R.random_weights(shape, seed, std=0.08, device="cpu"), DEV)
    sessions = []
    for i in range(2):
        prompt = G.tokens(w, 10 + i, shape=(w.B, w.N), high=w.vocab)
        dec = R.DecoderGPU(shape, weights, max_rows=w.B * max(w.k, 128))
        sessions.append(R.Session(dec, prompt, w.k, w.gen_tokens, chunk=128, group=w.group, bits=(w.k_bits, w.v_bits)))
    refs = [R.Greedy(se).run() for se in sessions]
    alone = R.VeriCacheLoop(sessions[0], slots=1).run()
    assert np.array_equal(alone, refs[0])
    st = R.Staggered([R.VeriCacheLoop(se, slots=1) for se in sessions])
    got = st.run(timed=True)
    for b in range(2):
        assert np.array_equal(got[b], refs[b]), b
    say(f"rounds {[lp.rounds for lp in st.loops]}")


@pytest.mark.parametrize("graph", [True, False])
def test_adaptive_horizon_equals_greedy(graph):
    """Draft horizons chosen per round by the cost model (HorizonPolicy, horizons 2, 4
    and 8 with buffers for 8): the output still equals greedy, and every horizon is
    drafted at least once."""
    w = SMALL
    _, _, _, dec, sess = _setup(w, std=0.08, chunk=128)
    ref = R.Greedy(sess).run()
    loop = R.VeriCacheLoop(sess, slots=1, graph=graph, horizons=(2, 4, 8))
    got = loop.run()
    assert np.array_equal(got, ref)
    assert all(v > 0 for v in loop.policy.chosen.values()), loop.policy.chosen
    say(f"rounds {loop.rounds}, horizons chosen {loop.policy.chosen}")


@pytest.mark.parametrize("rate", [0.0, 2e9])
def test_prefix_from_file_equals_greedy(tmp_path, rate):
    """The remote-prefix-cache setting: the prompt's full KV is staged every round from
    a file by the library's stager threads (uncapped, and capped at 2 GB/s), the
    generated rows from pinned host memory; the output still equals greedy, and every
    prompt row came through the file (the pinned copy of those rows is cleared)."""
    w = SMALL
    _, _, _, dec, sess = _setup(w, std=0.08, chunk=128)
    ref = R.Greedy(sess).run()
    loop = R.VeriCacheLoop(sess, slots=1, prefix_store=dict(directory=str(tmp_path), n_threads=3,
                                                            chunk_bytes=1 << 14, n_buffers=6, max_bytes_per_s=rate))
    assert all(float(t[:, :, : w.N].abs().max()) == 0 for t in loop.full.host_k)
    got = loop.run()
    assert np.array_equal(got, ref)
    assert loop.full.bytes_from_file > 0
    loop.full.close()
    say(f"rounds {loop.rounds}, {loop.full.bytes_from_file / 2 ** 20:.1f} MiB from the file")


def test_graph_draft_loop_matches_eager():
    """The captured draft loop produces the same drafts as the step-by-step launches
    (std 0.02 model: drafts are mostly accepted, so several rounds and group
    compressions go by)."""
    w = SMALL
    _, _, _, dec, sess = _setup(w, std=0.02, chunk=128)
    a, b = R.VeriCacheLoop(sess, slots=None, graph=True), R.VeriCacheLoop(sess, slots=None, graph=False)
    for _ in range(6):
        a.round()
        b.round()
        assert torch.equal(a.drafts_T, b.drafts_T)
        assert a.out == b.out
    say(f"accept lengths {a.accept_lens}")


def test_round_output_equals_greedy_full_size():
    """4 layers, d_model 2048, 16/4 heads, 16k-token prompts, k = 32, 2-bit KIVI
    drafts, 256 generated tokens per sequence."""
    w = W
    say(f"e2e {w.name}: prefill")
    _, _, _, dec, sess = _setup(w, std=0.02)
    say("greedy")
    ref = R.Greedy(sess).run()
    say("draft-and-verify")
    loop = R.VeriCacheLoop(sess, slots=2)
    got = loop.run()
    say(f"rounds {loop.rounds}, mean accept {np.mean(loop.accept_lens):.2f}")
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M", [1, 4, 40, 128])
def test_gemm_swiglu_equals_separate_calls(M):
    """The gate/up product with SwiGLU in its epilogue equals, bit for bit, the plain
    batch-invariant product into [M, 2F] followed by the activation kernel."""
    say(f"[gemm swiglu] M={M}")
    d, F = 2048, 5504
    x = T(G.normal(W, (22, M), (M, d), 1.0, "bf16"), torch.bfloat16)
    wgu = T(G.normal(W, (23,), (2 * F, d), 0.02, "bf16"), torch.bfloat16)
    gu = torch.empty(M, 2 * F, device=DEV, dtype=torch.bfloat16)
    want = torch.empty(M, F, device=DEV, dtype=torch.bfloat16)
    got = torch.empty_like(want)
    L.vc_gemm_bf16(x, wgu, gu)
    L.vc_swiglu(gu, want)
    L.vc_gemm_bf16_swiglu(x, L.swiglu_interleave(wgu), got)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


@pytest.mark.parametrize("B,k", [(4, 1), (3, 5), (4, 32)])
def test_gemm_rope_equals_separate_calls(B, k):
    """The QKV product with the rotary scatter in its epilogue writes, bit for bit,
    what the plain batch-invariant product followed by the rotary kernel writes
    (queries, and key/value rows including ones that fall outside the cache)."""
    say(f"[gemm rope] B={B} k={k}")
    Hq, Hkv, hd, d = 16, 4, 128, 2048
    M = B * k
    width = (Hq + 2 * Hkv) * hd
    x = T(G.normal(W, (24, B, k), (M, d), 1.0, "bf16"), torch.bfloat16)
    wqkv = T(G.normal(W, (25,), (width, d), 0.02, "bf16"), torch.bfloat16)
    pos = T(G.uniform_ints(W, (26, B, k), (M,), 0, 40000), torch.int32)
    rows = k + 6
    r0 = np.array([(b * 3) % (rows - k + 1) for b in range(B)], np.int64)
    r0[-1] = rows - k + 3                      # the last sequence's last rows fall outside the cache
    row0 = T(r0, torch.int32)
    qkv = torch.empty(M, width, device=DEV, dtype=torch.bfloat16)
    L.vc_gemm_bf16(x, wqkv, qkv)
    outs = []
    for fused in (False, True):
        q = torch.zeros(B, Hq, k, hd, device=DEV, dtype=torch.bfloat16)
        kd = torch.zeros(B, Hkv, rows, hd, device=DEV, dtype=torch.bfloat16)
        vd = torch.zeros_like(kd)
        if fused:
            L.vc_gemm_bf16_rope(x, L.rope_interleave(wqkv, Hq, Hkv, hd), B, k, Hq, Hkv, hd, pos, q, kd, vd, row0)
        else:
            L.vc_rope_qkv(qkv, B, k, Hq, Hkv, hd, pos, q, kd, vd, row0)
        outs.append((q, kd, vd))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
