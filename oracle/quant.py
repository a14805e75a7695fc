"""Oracle: KIVI-style asymmetric group quantization, bit packing, dequantization.

TEST INFRASTRUCTURE (see the package header).

Source: podparley.com episode page "VeriCache: Lossless LLM Inference from Lossy KV
Caches", source 4 (KIVI, "tuning-free asymmetric 2bit quantization for KV cache"),
and the neuraltrendhub.com summary "What the paper found" (KIVI among the
compressors behind the uniform compressor interface).  The pages give the method's
name only; the arithmetic below is the plain reading of "asymmetric" group
quantization with a scale and a zero-point:

* K is quantized per channel: one group = G consecutive tokens of one channel.
* V is quantized per token: one group = G consecutive channels of one token.
* Per group: mn = min, mx = max; s32 = fl32(fl32(mx - mn) / (2^b - 1));
  s = round(s32 -> scale dtype), z = round(mn -> scale dtype);
  code = clamp(rint_half_even(fl32(fl32(x - z) / s)), 0, 2^b - 1), every
  operation in IEEE float32; a group with s == 0 gets all-zero codes.
* Dequantized value: z + code * s.

Packing (a layout of this library, not a fact of the pages): each token row of d
codes is one little-endian bitstream; code c occupies bits b*c .. b*c+b-1 and
32-bit word w holds bits 32w .. 32w+31, so 3-bit codes straddle words.

Parity: pinned by brute-force nearest-level search, hand-written bit patterns
(tests/golden/pack_words.txt), pack/unpack round trips, group-axis perturbation
tests and the 16-bit special case.
"""
import numpy as np

BITS = (2, 3, 4, 8, 16)


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as
    float32.  Written from the format: keep the upper 16 bits of the float32
    pattern after adding half an ulp of the kept part (plus one if the kept
    part is odd, which makes exact halves round to even)."""
    x = np.asarray(x, dtype=np.float32)
    assert np.all(np.isfinite(x)), "non-finite values are outside the oracle's domain"
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    return (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)


def to_scale_dtype(x, scale_dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if scale_dtype == "f32":
        return x.copy()
    if scale_dtype == "bf16":
        return bf16_round(x)
    raise ValueError(scale_dtype)


def _quantize_groups(g: np.ndarray, bits: int, scale_dtype: str):
    """g: float32 [..., n_groups, G] -- the last axis is one group.
    Returns codes (same shape, int64), scale and zero ([..., n_groups], float32
    holding scale-dtype values)."""
    assert bits in BITS
    g = np.asarray(g, dtype=np.float32)
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    levels = np.float32(2 ** bits - 1)
    s32 = (mx - mn).astype(np.float32) / levels          # float32 subtract, float32 divide
    s = to_scale_dtype(s32, scale_dtype)
    z = to_scale_dtype(mn, scale_dtype)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - z[..., None]).astype(np.float32) / s[..., None]   # float32 ops
    q = np.clip(np.rint(t), 0, 2 ** bits - 1)
    q = np.where((s == 0)[..., None], 0, q)
    return q.astype(np.int64), s, z


def quantize_k(k: np.ndarray, bits: int, group: int, scale_dtype: str):
    """Per-channel K quantization of one (batch, kv-head) slice.
    k: [N, d] -> codes [N, d], scale [N/G, d], zero [N/G, d]."""
    N, d = k.shape
    assert N % group == 0
    g = k.reshape(N // group, group, d).transpose(0, 2, 1)      # [N/G, d, G]
    q, s, z = _quantize_groups(g, bits, scale_dtype)
    return q.transpose(0, 2, 1).reshape(N, d), s, z


def quantize_v(v: np.ndarray, bits: int, group: int, scale_dtype: str):
    """Per-token V quantization of one (batch, kv-head) slice.
    v: [N, d] -> codes [N, d], scale [N, d/G], zero [N, d/G]."""
    N, d = v.shape
    assert d % group == 0
    g = v.reshape(N, d // group, group)                         # [N, d/G, G]
    q, s, z = _quantize_groups(g, bits, scale_dtype)
    return q.reshape(N, d), s, z


def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [..., d] (ints in [0, 2^b)) -> uint32 words [..., d*b/32]."""
    codes = np.asarray(codes).astype(np.uint64)
    d = codes.shape[-1]
    assert (d * bits) % 32 == 0
    assert np.all(codes < (1 << bits))
    words = np.zeros(codes.shape[:-1] + (d * bits // 32,), dtype=np.uint64)
    for c in range(d):
        pos = bits * c
        w, off = divmod(pos, 32)
        words[..., w] |= (codes[..., c] << np.uint64(off)) & np.uint64(0xFFFFFFFF)
        if off + bits > 32:                                     # straddles into the next word
            words[..., w + 1] |= codes[..., c] >> np.uint64(32 - off)
    return words.astype(np.uint32)


def unpack_rows(words: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Inverse of pack_rows, read one bit at a time: code c = sum_j bit(b*c+j) << j."""
    words = np.asarray(words).astype(np.uint64)
    codes = np.zeros(words.shape[:-1] + (d,), dtype=np.int64)
    for c in range(d):
        for j in range(bits):
            p = bits * c + j
            bit = (words[..., p // 32] >> np.uint64(p % 32)) & np.uint64(1)
            codes[..., c] |= bit.astype(np.int64) << j
    return codes


def dequantize_k(codes, scale, zero, group: int) -> np.ndarray:
    """float64 [N, d]: z + code * s with the group of token n being n // G."""
    s = np.repeat(np.asarray(scale, np.float64), group, axis=0)
    z = np.repeat(np.asarray(zero, np.float64), group, axis=0)
    return z + np.asarray(codes, np.float64) * s


def dequantize_v(codes, scale, zero, group: int) -> np.ndarray:
    """float64 [N, d]: z + code * s with the group of channel c being c // G."""
    s = np.repeat(np.asarray(scale, np.float64), group, axis=1)
    z = np.repeat(np.asarray(zero, np.float64), group, axis=1)
    return z + np.asarray(codes, np.float64) * s


def compress_slice(k, v, k_bits, v_bits, group, scale_dtype):
    """Quantize and pack one (batch, kv-head) slice.  Returns a dict with the
    packed words and the parameters (the layout of the library's compressed
    cache for one slice)."""
    kq, ks, kz = quantize_k(k, k_bits, group, scale_dtype)
    vq, vs, vz = quantize_v(v, v_bits, group, scale_dtype)
    return dict(k_codes=pack_rows(kq, k_bits), v_codes=pack_rows(vq, v_bits),
                k_scale=ks, k_zero=kz, v_scale=vs, v_zero=vz, kq=kq, vq=vq)


def dequantize_slice(c, d, k_bits, v_bits, group):
    """(K_hat, V_hat) float64 [N, d] from a compress_slice() dict."""
    kq = unpack_rows(c["k_codes"], k_bits, d)
    vq = unpack_rows(c["v_codes"], v_bits, d)
    return (dequantize_k(kq, c["k_scale"], c["k_zero"], group),
            dequantize_v(vq, c["v_scale"], c["v_zero"], group))
