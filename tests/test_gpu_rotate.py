"""GPU tests of the channel rotation (vc_hadamard_rows) against the oracle, and of a
drafter with the rotation pre-pass: keys, values and queries rotated, compressed by
the KIVI quantizer and decoded on the matrix cores, the output rotated back."""
import numpy as np
import pytest
import torch

import lossy_kv_draft_amd as L
from oracle import rotate as RO, attention as OA, quant as OQ
from workloads import configs as C, gen as G
from gpu_util import T, np32, tdtype, say

pytestmark = pytest.mark.gpu


def _rows(rows, d, key, dtype):
    """Seeded rows with one outlier channel (x 10), rounded to the storage dtype on the host."""
    x = G.normal(C.TINY, (70,) + key, (rows, d), 1.0, "f32")
    x[:, 5] *= 10.0
    return OQ.bf16_round(x) if dtype == "bf16" else x.astype(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("rows", [1, 5, 1027])
def test_rotation_matches_oracle(dtype, d, rows):
    """Within the float32 arithmetic error (sums of d terms) plus half a unit in the last
    place of the storage type."""
    x = _rows(rows, d, (d, rows), dtype)
    got = np32(L.vc_hadamard_rows(T(x, tdtype(dtype))))
    ref = RO.rotate_rows(x)
    arith = 1e-6 * np.abs(x).sum(-1, keepdims=True) / np.sqrt(d)
    half_ulp = 2.0 ** -8 * np.abs(ref) if dtype == "bf16" else 1e-7 * np.abs(ref)
    excess = (np.abs(got - ref) - arith - half_ulp).max()
    assert excess <= 0, f"max excess {excess}"


@pytest.mark.parametrize("dtype,d,rows", [("f32", 256, 40001), ("bf16", 64, 270001)])
def test_rotation_many_rows(dtype, d, rows):
    """More rows than one pass of the (capped) grid holds, with a ragged last pass; the
    oracle checks every 97th row."""
    x = _rows(rows, d, (d, 1), dtype)
    got = np32(L.vc_hadamard_rows(T(x, tdtype(dtype))))[::97]
    ref = RO.rotate_rows(x[::97])
    tol = (2.0 ** -8 if dtype == "bf16" else 1e-7) * np.abs(ref) + 1e-6 * np.abs(x[::97]).sum(-1, keepdims=True)
    assert (np.abs(got - ref) <= tol).all()


@pytest.mark.parametrize("d", [64, 256])
def test_rotation_bit_exact_on_small_integers(d):
    """Small integers: every butterfly sum is exact in float32 and 1/sqrt(d) is a power of
    two, so the stored result is the correctly rounded exact one."""
    x = np.round(_rows(64, d, (d, 9), "f32") / 4.0).clip(-3, 3).astype(np.float32)
    got = np32(L.vc_hadamard_rows(T(x, torch.bfloat16)))
    assert np.array_equal(got, OQ.bf16_round(RO.rotate_rows(x).astype(np.float32)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rotation_in_place_and_involution(dtype):
    x = _rows(300, 128, (3,), dtype)
    xd = T(x, tdtype(dtype))
    y = L.vc_hadamard_rows(xd, xd)            # in place
    assert y.data_ptr() == xd.data_ptr()
    z = np32(L.vc_hadamard_rows(y))
    tol = 2.0 ** -7 if dtype == "bf16" else 1e-6
    assert np.abs(z - x).max() <= tol * np.abs(x).max()


def test_rotated_drafter_is_closer_to_exact_attention():
    """On keys and values with outlier channels, 2-bit KIVI drafts with the rotation
    pre-pass are closer to exact attention (the oracle's float64 attention over the
    bf16 cache) than the same drafts without it: the pre-pass's purpose."""
    w = C.small(C.LLAMA8B, N=64 * 16, k_bits=2, v_bits=2)
    K, V = OQ.bf16_round(G.full_kv(w, "k")), OQ.bf16_round(G.full_kv(w, "v"))
    Q = OQ.bf16_round(G.full_window_q(w)[:, :, 0])                   # [B, Hq, d]
    dt = torch.bfloat16
    Kd, Vd, Qd = T(K, dt), T(V, dt), T(Q, dt)

    def draft(kd, vd, qd):
        c = L.Ckv("quant", w.B, w.Hkv, w.d, w.N, k_bits=2, v_bits=2, group=w.group, param_dtype=w.scale_dtype,
                  kv_dtype="bf16", tail_cap=1)
        L.vc_compress(c, kd, vd, n_tokens=w.N)
        c.n_main = w.N
        o = torch.empty(w.B, w.Hq, w.d, device="cuda", dtype=dt)
        L.vc_decode_attn_compressed(c, qd, o)
        return o

    plain = np32(draft(Kd, Vd, Qd))
    rot = np32(L.vc_hadamard_rows(draft(L.vc_hadamard_rows(Kd), L.vc_hadamard_rows(Vd), L.vc_hadamard_rows(Qd))))
    exact = np.stack([OA.decode(Q[b], K[b], V[b], w.d ** -0.5)[0] for b in range(w.B)])
    rel = lambda o: np.linalg.norm(o - exact) / np.linalg.norm(exact)
    say(f"relative L2 error vs exact attention: plain {rel(plain):.4f}, rotated {rel(rot):.4f}")
    assert rel(rot) < 0.8 * rel(plain)
