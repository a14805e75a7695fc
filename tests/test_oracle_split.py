"""Pins of the split-stream oracle (oracle/split.py) against hand-worked packed rows,
the join round trip, the r = 0 identity, the midpoint property of the anchor's
levels and the anchor's error bound."""
import os

import numpy as np
import pytest

from oracle import quant as OQ, split as OS

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "split_words.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        b, a, P, aw, rw = line.split()
        words = lambda s: np.array([int(x, 16) for x in s.split(",")], np.uint32)
        rows.append((int(b), int(a), int(P), words(aw), words(rw)))
    return rows


@pytest.mark.parametrize("case", _golden(), ids=lambda c: f"{c[0]}to{c[1]}")
def test_hand_worked_rows(case):
    b, a, P, aw, rw = case
    codes = np.arange(32) % P
    m, e = OS.split_codes(codes, b, a)
    assert np.array_equal(OQ.pack_rows(m, a), aw)
    assert np.array_equal(OQ.pack_rows(e, b - a), rw)


@pytest.mark.parametrize("b,a", [(4, 2), (3, 2), (4, 3), (8, 4), (8, 2), (2, 2), (4, 4)])
def test_join_restores_every_code(b, a):
    c = np.arange(1 << b)
    m, e = OS.split_codes(c, b, a)
    assert m.max() < (1 << a) and e.max() < (1 << (b - a)) if b > a else (e == 0).all()
    assert np.array_equal(OS.join_codes(m, e, b, a), c)
    # the anchor orders codes like the full codes (most significant bits first)
    assert (np.diff(m) >= 0).all()


def test_no_residual_bits_is_the_identity():
    rng = np.random.default_rng(0)
    s = OQ.bf16_round(rng.uniform(0.01, 2, 50).astype(np.float32))
    z = OQ.bf16_round(rng.normal(0, 3, 50).astype(np.float32))
    sa, za = OS.anchor_params(s, z, 4, 4, "bf16")
    assert np.array_equal(sa, s) and np.array_equal(za, z)


@pytest.mark.parametrize("b,a", [(4, 2), (3, 2), (4, 3)])
def test_anchor_level_is_the_midpoint_of_its_levels(b, a):
    """With dyadic parameters every operation is exact: level m of the anchor is the
    midpoint of full levels m 2^r and m 2^r + 2^r - 1."""
    r = b - a
    for s, z in [(0.25, -1.0), (0.0625, 3.5), (2.0, -40.0)]:
        sa, za = OS.anchor_params(np.float32([s]), np.float32([z]), b, a, "f32")
        for m in range(1 << a):
            lo, hi = z + (m << r) * s, z + ((m << r) + (1 << r) - 1) * s
            assert float(za[0] + m * sa[0]) == (lo + hi) / 2


def test_bf16_anchor_params_are_correctly_rounded():
    """bf16 parameters: s * 2^r is exact; z + s (2^r - 1)/2 is exact in float32 for
    bf16 inputs of nearby magnitude, so the stored zero is the correctly rounded
    exact value."""
    rng = np.random.default_rng(1)
    s = OQ.bf16_round(rng.uniform(0.01, 1, 400).astype(np.float32))
    z = OQ.bf16_round(rng.uniform(-4, 4, 400).astype(np.float32))
    sa, za = OS.anchor_params(s, z, 4, 2, "bf16")
    assert np.array_equal(sa, s * 4)
    exact = z.astype(np.float64) + 1.5 * s.astype(np.float64)
    assert np.array_equal(za, OQ.bf16_round(exact.astype(np.float32)))
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)   # the float32 sum was exact


@pytest.mark.parametrize("kb,vb,ka,va", [(4, 4, 2, 2), (4, 3, 2, 2), (4, 4, 3, 2)])
def test_anchor_dequantization_error_bound(kb, vb, ka, va):
    """Every anchor value is within s (2^r - 1)/2 of the full b-bit value it replaces
    (plus the rounding of the stored zero), hence within s 2^(r-1) + s/2 of the
    original input; joining the two streams gives back the b-bit codes."""
    rng = np.random.default_rng(2)
    N, d, G = 128, 64, 32
    k = rng.normal(0, 1, (N, d)).astype(np.float32)
    v = rng.normal(0, 1, (N, d)).astype(np.float32)
    c = OQ.compress_slice(k, v, kb, vb, G, "f32")
    sp = OS.split_slice(c, d, kb, vb, ka, va, "f32")
    K, V = OQ.dequantize_slice(c, d, kb, vb, G)
    Ka, Va = OQ.dequantize_slice(sp, d, ka, va, G)
    for full, anc, x, s, b, a, ax in [(K, Ka, k, c["k_scale"], kb, ka, 0), (V, Va, v, c["v_scale"], vb, va, 1)]:
        r = b - a
        sfull = np.repeat(s, G, axis=ax).astype(np.float64)
        assert (np.abs(anc - full) <= sfull * ((1 << r) - 1) / 2 * (1 + 1e-6) + 1e-6).all()
        assert (np.abs(anc - x) <= sfull * ((1 << r) - 1) / 2 + sfull / 2 + 1e-5).all()
    if kb > ka:
        km = OQ.unpack_rows(sp["k_codes"], ka, d)
        ke = OQ.unpack_rows(sp["k_resid"], kb - ka, d)
        assert np.array_equal(OS.join_codes(km, ke, kb, ka), c["kq"])
    vm = OQ.unpack_rows(sp["v_codes"], va, d)
    ve = OQ.unpack_rows(sp["v_resid"], vb - va, d)
    assert np.array_equal(OS.join_codes(vm, ve, vb, va), c["vq"])
