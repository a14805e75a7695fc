"""Oracle: split-stream form of a KIVI-quantized cache (most significant bits as an
anchor stream, the rest as a residual stream).

TEST INFRASTRUCTURE (see the package header).

Source: thelatestinai.com listing page for 2604.15409, the Lynx abstract (progressive
split-stream KV transfer): the quantized cache is cut into a high-priority anchor
stream holding the most significant bits and a low-priority residual stream holding
the remaining precision; decoding may start from the anchor alone and is verified
afterwards.  In VeriCache's terms (neuraltrendhub.com summary, "What the paper
found": compressors behind one interface) the anchor is one more compressed cache
to draft from.  The pages give no arithmetic; the reading taken here:

* a b-bit code c of a group with scale s and zero z splits, for an anchor of a bits
  and r = b - a residual bits, into m = c >> r and e = c & (2^r - 1); c = (m << r) | e;
* the anchor is itself an a-bit KIVI cache whose level m stands for the midpoint of
  the 2^r full levels it covers: scale s_a = s * 2^r and zero
  z_a = z + s * (2^r - 1) / 2, each product and sum one IEEE float32 operation,
  rounded to the scale dtype;
* both streams use the library's packing (quant.pack_rows) at their own widths; the
  residual stream keeps the original scales and zeros, so joining restores the
  b-bit cache exactly.

Parity: pinned by a hand-worked packed row (tests/golden/split_words.txt), the join
round trip for every code, the r = 0 identity, and the midpoint property of the
anchor's levels on dyadic parameters.
"""
import numpy as np

from .quant import pack_rows, unpack_rows, to_scale_dtype


def split_codes(codes, bits: int, anchor_bits: int):
    """codes (ints in [0, 2^bits)) -> (anchor codes, residual codes)."""
    r = bits - anchor_bits
    assert 0 <= r and anchor_bits >= 1
    c = np.asarray(codes).astype(np.int64)
    return c >> r, c & ((1 << r) - 1)


def join_codes(anchor, resid, bits: int, anchor_bits: int):
    r = bits - anchor_bits
    return (np.asarray(anchor).astype(np.int64) << r) | np.asarray(resid).astype(np.int64)


def anchor_params(scale, zero, bits: int, anchor_bits: int, scale_dtype: str):
    """(s_a, z_a) of the anchor from the full cache's (s, z) (float32 arrays holding
    scale-dtype values): s_a = fl(s * 2^r), z_a = fl(z + fl(s * (2^r - 1) / 2))."""
    r = bits - anchor_bits
    s = np.asarray(scale, np.float32)
    z = np.asarray(zero, np.float32)
    s_a = np.float32(2.0 ** r) * s
    half_span = np.float32((2.0 ** r - 1.0) / 2.0) * s
    z_a = z + half_span
    return to_scale_dtype(s_a, scale_dtype), to_scale_dtype(z_a, scale_dtype)


def split_slice(c: dict, d: int, k_bits: int, v_bits: int, ka: int, va: int, scale_dtype: str) -> dict:
    """A compress_slice() dict -> the anchor (a compress_slice()-like dict at ka/va
    bits) and the residual words (k_resid, v_resid; None for r = 0)."""
    kq = unpack_rows(c["k_codes"], k_bits, d)
    vq = unpack_rows(c["v_codes"], v_bits, d)
    km, ke = split_codes(kq, k_bits, ka)
    vm, ve = split_codes(vq, v_bits, va)
    ks, kz = anchor_params(c["k_scale"], c["k_zero"], k_bits, ka, scale_dtype)
    vs, vz = anchor_params(c["v_scale"], c["v_zero"], v_bits, va, scale_dtype)
    return dict(k_codes=pack_rows(km, ka), v_codes=pack_rows(vm, va), k_scale=ks, k_zero=kz, v_scale=vs, v_zero=vz,
                k_resid=pack_rows(ke, k_bits - ka) if k_bits > ka else None,
                v_resid=pack_rows(ve, v_bits - va) if v_bits > va else None)
