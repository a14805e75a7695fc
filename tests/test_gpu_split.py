"""GPU parity of the split-stream compressor (vc_split_planes / vc_join_planes)
against the oracle: anchor codes, anchor parameters and residual codes bit exact,
the join restores the full codes, and the existing compressed decode reads the anchor
as an ordinary quantized cache (within the attention tolerance of the oracle's
attention over the anchor's dequantized values)."""
import numpy as np
import pytest
import torch

import lossy_kv_draft_amd as L
from workloads import configs as C, gen as G
from oracle import quant as OQ, split as OS, attention as OA
from gpu_util import assert_close, T, np32, tdtype, oracle_compress, inputs, say

pytestmark = pytest.mark.gpu

CASES = {  # workload, anchor K bits, anchor V bits
    "llama8b_4to2": (C.small(C.LLAMA8B, N=64 * 11), 2, 2),
    "qwen30b_k4v3_to2": (C.small(C.QWEN30B, N=32 * 23), 2, 2),
    "k4v4_to3v2_f32": (C.small(C.E2E, N=32 * 9, k_bits=4, v_bits=4, scale_dtype="f32"), 3, 2),
    "k8v4_to4v4_g16": (C.small(C.E2E, N=16 * 10, k_bits=8, v_bits=4, group=16), 4, 4),
}


def _ckv(w, kb, vb, tail_cap=0):
    return L.Ckv("quant", w.B, w.Hkv, w.d, w.N, k_bits=kb, v_bits=vb, group=w.group, param_dtype=w.scale_dtype,
                 kv_dtype=w.dtype, tail_cap=tail_cap)


def _oracle_split(w, comp, ka, va):
    B, Hkv = comp["k_codes"].shape[:2]
    out = [[OS.split_slice({k: v[b, h] for k, v in comp.items()}, w.d, w.k_bits, w.v_bits, ka, va, w.scale_dtype)
            for h in range(Hkv)] for b in range(B)]
    keys = ["k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"]
    keys += [k for k in ("k_resid", "v_resid") if out[0][0][k] is not None]
    return {k: np.stack([np.stack([out[b][h][k] for h in range(Hkv)]) for b in range(B)]) for k in keys}


def _split_on_gpu(w, ka, va, n):
    K, V = G.full_kv(w, "k"), G.full_kv(w, "v")
    full = _ckv(w, w.k_bits, w.v_bits)
    L.vc_compress(full, T(K, tdtype(w.dtype)), T(V, tdtype(w.dtype)), n_tokens=w.N)
    anchor = _ckv(w, ka, va, tail_cap=1)
    for t in (anchor.k_codes, anchor.v_codes):
        t.fill_(-1)                                  # rows past n stay as they were
    kr, vr = L.split_residuals(full, anchor)
    L.vc_split_planes(full, anchor, kr, vr, n)
    torch.cuda.synchronize()
    return K, V, full, anchor, kr, vr


@pytest.mark.parametrize("name", list(CASES))
def test_split_matches_oracle_bit_exact(name):
    w, ka, va = CASES[name]
    n = w.N - w.group * 2                            # a prefix of the rows
    say(f"[split] {name} B{w.B} Hkv{w.Hkv} N{w.N} n{n} K{w.k_bits}->{ka} V{w.v_bits}->{va} G{w.group}")
    K, V, full, anchor, kr, vr = _split_on_gpu(w, ka, va, n)
    ref = _oracle_split(w, oracle_compress(w, K[:, :, :n], V[:, :, :n]), ka, va)
    u32 = lambda t: t.cpu().numpy().view(np.uint32)
    assert np.array_equal(u32(anchor.k_codes)[:, :, :n], ref["k_codes"])
    assert np.array_equal(u32(anchor.v_codes)[:, :, :n], ref["v_codes"])
    assert (u32(anchor.k_codes)[:, :, n:] == 0xFFFFFFFF).all()
    g = n // w.group
    for key, rows in (("k_scale", g), ("k_zero", g), ("v_scale", n), ("v_zero", n)):
        assert np.array_equal(np32(getattr(anchor, key))[:, :, :rows], ref[key]), key
    if kr is not None:
        assert np.array_equal(u32(kr)[:, :, :n], ref["k_resid"])
    if vr is not None:
        assert np.array_equal(u32(vr)[:, :, :n], ref["v_resid"])


@pytest.mark.parametrize("name", list(CASES))
def test_join_restores_the_full_codes(name):
    w, ka, va = CASES[name]
    K, V, full, anchor, kr, vr = _split_on_gpu(w, ka, va, w.N)
    back = _ckv(w, w.k_bits, w.v_bits)
    back.k_scale, back.k_zero, back.v_scale, back.v_zero = full.k_scale, full.k_zero, full.v_scale, full.v_zero
    L.vc_join_planes(anchor, kr, vr, back, w.N)
    torch.cuda.synchronize()
    assert torch.equal(back.k_codes, full.k_codes) and torch.equal(back.v_codes, full.v_codes)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_on_the_anchor_matches_oracle(name):
    """The drafter's decode over the anchor alone (plus tail rows) against the oracle's
    float64 attention over the anchor's dequantized keys and values."""
    w, ka, va = CASES[name]
    K, V, Q, Kw, Vw = inputs(w)
    _, _, full, anchor, kr, vr = _split_on_gpu(w, ka, va, w.N)
    tail = 3
    dt = tdtype(w.dtype)
    anchor.tail_k = T(Kw[:, :, :tail], dt).contiguous()
    anchor.tail_v = T(Vw[:, :, :tail], dt).contiguous()
    anchor.tail_cap = anchor.tail_len = tail
    anchor.n_main = w.N
    q = T(Q[:, :, tail - 1], dt)
    out = torch.empty(w.B, w.Hq, w.d, device="cuda", dtype=dt)
    L.vc_decode_attn_compressed(anchor, q, out)
    torch.cuda.synchronize()
    ref = _oracle_split(w, oracle_compress(w, K, V), ka, va)
    for b in range(w.B):
        kh = np.stack([OQ.dequantize_k(OQ.unpack_rows(ref["k_codes"][b, h], ka, w.d), ref["k_scale"][b, h],
                                       ref["k_zero"][b, h], w.group) for h in range(w.Hkv)])
        vh = np.stack([OQ.dequantize_v(OQ.unpack_rows(ref["v_codes"][b, h], va, w.d), ref["v_scale"][b, h],
                                       ref["v_zero"][b, h], w.group) for h in range(w.Hkv)])
        o, _ = OA.decode(Q[b, :, tail - 1], kh, vh, w.d ** -0.5, Kw[b, :, :tail], Vw[b, :, :tail])
        assert_close(np32(out[b]), o, w.dtype, f"b={b}")
