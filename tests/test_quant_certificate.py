"""Soundness of the reciprocal certificate the fast compression kernel relies on (host
arithmetic in numpy float32; no GPU, no library code).

The kernel forms a KIVI code from qa = fl(fl(x - z) * r), where r is the hardware
reciprocal of the scale s (within one ulp of 1/s), instead of the correctly rounded
quotient fl(fl(x - z) / s) that defines the code (summary page "VeriCache: Turning
Lossy KV Cache into Lossless LLM Inference", "What the paper found": KIVI-style
per-group min-max quantization).  A code is taken from qa only when qa lies further
than 2^(bits - 20) from every half-integer; the others go to the division.  These tests
check, over random groups of several scales and over points placed on and beside every
half-integer, that a certified code always equals the code from the division, with r
off by one ulp either way, for float32 and bf16 data and parameters.  A margin of zero
must fail the same check (the test can see a wrong certificate).
"""
import numpy as np
import pytest

F32 = np.float32


def _bf16(v):
    u = np.asarray(v, F32).view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.astype(np.uint32).view(F32)


def _cases(rng, bits, trials, n):
    """(x, z, s) float32 triples: random groups plus points on and next to every
    half-integer of each group's code lattice."""
    lev = F32(2 ** bits - 1)
    for _ in range(trials):
        scale = F32(10.0 ** rng.uniform(-6, 4))
        x = (rng.standard_normal(n) * scale).astype(F32)
        for data_bf16 in (False, True):
            xx = _bf16(x) if data_bf16 else x
            mn, mx = xx.min(), xx.max()
            s = F32(F32(mx - mn) / lev)
            for par_bf16 in (False, True):
                ss, zz = (_bf16(s), _bf16(mn)) if par_bf16 else (s, mn)
                if not (ss >= F32(2.0 ** -126) and np.isfinite(ss)):
                    continue
                k = np.arange(-2, 2 ** bits + 2, dtype=F32) + F32(0.5)
                t = (zz + k * ss).astype(F32)
                up = np.nextafter(t, F32(np.inf))
                dn = np.nextafter(t, F32(-np.inf))
                near = np.concatenate([t, up, dn, np.nextafter(up, F32(np.inf)), np.nextafter(dn, F32(-np.inf))])
                if data_bf16:
                    near = np.concatenate([near, _bf16(near)])
                yield np.concatenate([xx, near]).astype(F32), zz, ss


def _mismatches(bits, margin, trials=60, n=4096, seed=11):
    rng = np.random.default_rng(seed)
    lev = F32(2 ** bits - 1)
    checked = bad = 0
    for xa, zz, ss in _cases(rng, bits, trials, n):
        with np.errstate(all="ignore"):
            d = (xa - zz).astype(F32)
            exact = np.clip(np.rint((d / ss).astype(F32)), 0, lev)
            r0 = F32(F32(1.0) / ss)
            for r in (np.nextafter(r0, F32(-np.inf)), r0, np.nextafter(r0, F32(np.inf))):
                qa = (d * F32(r)).astype(F32)
                fr = qa - np.floor(qa)
                ok = np.abs(fr - F32(0.5)) > margin
                checked += int(ok.sum())
                bad += int((np.clip(np.rint(qa[ok]), 0, lev) != exact[ok]).sum())
    return checked, bad


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_certified_codes_equal_division(bits):
    checked, bad = _mismatches(bits, F32(2.0 ** (bits - 20)))
    assert checked > 1_000_000
    assert bad == 0


def test_zero_margin_is_caught():
    _, bad = _mismatches(2, F32(0.0), trials=30)
    assert bad > 0
