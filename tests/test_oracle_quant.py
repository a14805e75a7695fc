"""Pins of the oracle's quantizer and packer against things other than itself:
hand-derived bit patterns and group examples, torch's bf16 conversion, brute-force
nearest-level search, group-axis perturbations and the 16-bit special case."""
import os
import numpy as np
import pytest
import torch

from oracle import quant as Q
from oracle import attention as A

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _parse_pack():
    rows = []
    for line in open(os.path.join(GOLD, "pack_words.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("=>")
        bits, d, spec = lhs.split()
        bits, d = int(bits), int(d)
        codes = np.zeros(d, np.int64)
        for item in spec.split(","):
            i, v = item.split(":")
            if i == "all":
                codes[:] = int(v)
            else:
                codes[int(i)] = int(v)
        words = [int(x, 16) for x in rhs.split()]
        rows.append((bits, codes, words))
    return rows


@pytest.mark.parametrize("bits,codes,words", _parse_pack())
def test_pack_golden(bits, codes, words):
    assert list(Q.pack_rows(codes[None], bits)[0]) == words
    assert np.array_equal(Q.unpack_rows(np.array([words], np.uint32), bits, len(codes))[0], codes)


def _parse_groups():
    rows = []
    for line in open(os.path.join(GOLD, "quant_groups.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, vals, codes, sz = [p.strip() for p in line.split("|")]
        bits, sd = head.split()
        s, z = (float(x) for x in sz.split())
        rows.append((int(bits), sd, np.array(vals.split(), np.float32),
                     np.array(codes.split(), np.int64), s, z))
    return rows


@pytest.mark.parametrize("bits,sd,vals,codes,s,z", _parse_groups())
def test_quant_golden_groups(bits, sd, vals, codes, s, z):
    G = len(vals)
    # as a V group (one token, G channels) and as a K group (G tokens, one channel)
    qv, sv, zv = Q.quantize_v(vals[None, :], bits, G, sd)
    assert np.array_equal(qv[0], codes) and sv[0, 0] == np.float32(s) and zv[0, 0] == np.float32(z)
    qk, sk, zk = Q.quantize_k(vals[:, None], bits, G, sd)
    assert np.array_equal(qk[:, 0], codes) and sk[0, 0] == np.float32(s) and zk[0, 0] == np.float32(z)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact halfway cases with even and odd kept parts
    u = rng.integers(0x3F000000, 0x40800000, size=5000, dtype=np.uint32)
    halves = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, halves, -halves, np.float32([0.0, -0.0, 1e-40, 3.3e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = Q.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("bits", Q.BITS)
@pytest.mark.parametrize("d", [64, 128])
def test_pack_unpack_roundtrip(bits, d):
    rng = np.random.default_rng(bits * 100 + d)
    codes = rng.integers(0, 1 << bits, size=(37, d))
    words = Q.pack_rows(codes, bits)
    assert words.shape == (37, d * bits // 32) and words.dtype == np.uint32
    assert np.array_equal(Q.unpack_rows(words, bits, d), codes)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("sd", ["f32", "bf16"])
def test_codes_are_nearest_levels(bits, sd):
    """Brute force: each code is the level z + q*s (q in [0, 2^b)) nearest to x,
    skipping elements within 1e-5*s of a tie between two levels."""
    rng = np.random.default_rng(bits + (7 if sd == "bf16" else 0))
    G = 16
    x = (rng.standard_normal((64, G)) * rng.uniform(0.01, 30, size=(64, 1))).astype(np.float32)
    x = Q.bf16_round(x) if sd == "bf16" else x
    q, s, z = Q.quantize_v(x, bits, G, sd)
    lv = z[:, :, None].astype(np.float64) + np.arange(2 ** bits)[None, None, :] * s[:, :, None].astype(np.float64)
    dist = np.abs(x.astype(np.float64)[:, :, None] - np.repeat(lv, G, axis=1))
    best = dist.argmin(axis=-1)
    srt = np.sort(dist, axis=-1)
    clear = (srt[..., 1] - srt[..., 0]) > 1e-5 * np.repeat(s, G, axis=1)
    assert clear.mean() > 0.99
    assert np.array_equal(q[clear], best[clear])
    assert q.min() >= 0 and q.max() <= 2 ** bits - 1


@pytest.mark.parametrize("bits", [2, 3, 4, 8, 16])
def test_fp32_scale_extremes(bits):
    rng = np.random.default_rng(bits)
    k = rng.standard_normal((32 * 4, 8)).astype(np.float32)
    q, s, z = Q.quantize_k(k, bits, 32, "f32")
    g = k.reshape(4, 32, 8)
    qg = q.reshape(4, 32, 8)
    amin = g.argmin(axis=1)
    amax = g.argmax(axis=1)
    for i in range(4):
        for c in range(8):
            assert qg[i, amin[i, c], c] == 0
            assert qg[i, amax[i, c], c] == 2 ** bits - 1
    assert np.array_equal(z, g.min(axis=1))


def test_constant_group_and_zero_scale():
    v = np.full((3, 64), 1.75, np.float32)
    q, s, z = Q.quantize_v(v, 4, 32, "bf16")
    assert np.all(q == 0) and np.all(s == 0) and np.all(z == np.float32(1.75))
    assert np.all(Q.dequantize_v(q, s, z, 32) == 1.75)


def test_group_axes():
    """A spike in K[n, c] changes only K's parameters of (token group n//G, channel c);
    a spike in V[n, c] changes only V's parameters of (token n, channel group c//G)."""
    rng = np.random.default_rng(3)
    G, N, d = 32, 128, 64
    x = rng.standard_normal((N, d)).astype(np.float32)
    y = x.copy()
    n, c = 70, 41
    y[n, c] = 100.0
    _, s0, z0 = Q.quantize_k(x, 4, G, "f32")
    _, s1, z1 = Q.quantize_k(y, 4, G, "f32")
    changed = (s0 != s1) | (z0 != z1)
    assert changed.sum() == 1 and changed[n // G, c]
    _, s0, z0 = Q.quantize_v(x, 4, G, "f32")
    _, s1, z1 = Q.quantize_v(y, 4, G, "f32")
    changed = (s0 != s1) | (z0 != z1)
    assert changed.sum() == 1 and changed[n, c // G]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_dequant_error_bound(bits):
    rng = np.random.default_rng(11)
    k = rng.standard_normal((256, 32)).astype(np.float32)
    q, s, z = Q.quantize_k(k, bits, 64, "f32")
    kh = Q.dequantize_k(q, s, z, 64)
    sr = np.repeat(s, 64, axis=0).astype(np.float64)
    assert np.all(np.abs(kh - k) <= sr * 0.5 * (1 + 1e-5) + 1e-7)


def test_16bit_fp32_params_reduce_to_dense_attention():
    rng = np.random.default_rng(2)
    Hq, Hkv, N, d = 4, 2, 256, 64
    K = rng.standard_normal((Hkv, N, d)).astype(np.float32)
    V = rng.standard_normal((Hkv, N, d)).astype(np.float32)
    q = rng.standard_normal((Hq, d)).astype(np.float32)
    Kh = np.stack([Q.dequantize_k(*Q.quantize_k(K[h], 16, 32, "f32"), 32) for h in range(Hkv)])
    Vh = np.stack([Q.dequantize_v(*Q.quantize_v(V[h], 16, 32, "f32"), 32) for h in range(Hkv)])
    assert np.max(np.abs(Kh - K)) < 1e-4
    o_q, _ = A.decode(q, Kh, Vh, d ** -0.5)
    o_d, _ = A.decode(q, K, V, d ** -0.5)
    assert np.max(np.abs(o_q - o_d)) < 1e-4


def test_compress_slice_layout():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((128, 128)).astype(np.float32)
    v = rng.standard_normal((128, 128)).astype(np.float32)
    c = Q.compress_slice(k, v, 4, 3, 32, "bf16")
    assert c["k_codes"].shape == (128, 16) and c["v_codes"].shape == (128, 12)
    assert c["k_scale"].shape == (4, 128) and c["v_scale"].shape == (128, 4)
    kh, vh = Q.dequantize_slice(c, 128, 4, 3, 32)
    assert np.max(np.abs(kh - k)) < 0.5 and np.max(np.abs(vh - v)) < 1.0
