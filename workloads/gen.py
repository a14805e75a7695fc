"""Seeded synthetic inputs shared by the oracle tests, the HIP-path tests and the
benchmark.

This module draws random numbers and stores them; it implements none of the
method's arithmetic.  Every (tensor, batch, head) slice has its own seed, so any
slice of a large workload can be regenerated on its own (the oracle checks
sampled slices of the full-size workloads that way).

Values are drawn in float32 from N(0, 1) and, for bf16 workloads, rounded to the
nearest bf16 (ties to even, via torch's dtype conversion).  Both sides receive the
same rounded values: the GPU as bf16, the oracle as float32/float64 copies of the
same numbers.
"""
from concurrent.futures import ThreadPoolExecutor
import numpy as np
import torch

from .configs import Workload

# tensor codes in the seed sequence
_Q, _K, _V, _QWIN, _KWIN, _VWIN, _OUTLIER, _PROBE, _W = range(1, 10)
_EMB, _LAYER, _NORM, _HEAD, _PROMPT = range(20, 25)


def _rng(w: Workload, *key) -> np.random.Generator:
    return np.random.default_rng([1000 + w.index, *key])


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype and return them as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def outlier_pairs(w: Workload) -> np.ndarray:
    """(kv-head, channel) pairs whose K and V values are multiplied by
    w.outlier_mult: round(frac * Hkv * d) pairs drawn without replacement."""
    n = int(round(w.outlier_frac * w.Hkv * w.d))
    if n == 0:
        return np.zeros((0, 2), dtype=np.int64)
    flat = _rng(w, _OUTLIER).choice(w.Hkv * w.d, size=n, replace=False)
    return np.stack([flat // w.d, flat % w.d], axis=1)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def kv_slice(w: Workload, which: str, b: int, h: int) -> np.ndarray:
    """Full-precision context K or V of (batch b, kv-head h): [N, d] float32 holding
    storage-dtype values."""
    code = {"k": _K, "v": _V}[which]
    x = _normal(_rng(w, code, b, h), (w.N, w.d))
    pairs = outlier_pairs(w)
    for hh, c in pairs:
        if hh == h:
            x[:, c] *= np.float32(w.outlier_mult)
    return to_storage(x, w.dtype)


def window_q(w: Workload, b: int, hq: int) -> np.ndarray:
    """Draft-window queries of (b, q-head hq): [k, d].  Row i is the query of draft
    step i and of verify row i."""
    return to_storage(_normal(_rng(w, _QWIN, b, hq), (w.k, w.d)), w.dtype)


def window_kv(w: Workload, which: str, b: int, h: int) -> np.ndarray:
    """Keys or values of the k window tokens of (b, kv-head h): [k, d]."""
    code = {"k": _KWIN, "v": _VWIN}[which]
    return to_storage(_normal(_rng(w, code, b, h), (w.k, w.d)), w.dtype)


def probes(w: Workload, h: int) -> np.ndarray:
    """Random probe queries of kv-head h for token scoring: [n_probes, d] (bf16 values)."""
    return to_storage(_normal(_rng(w, _PROBE, h), (w.n_probes, w.d)), "bf16")


def projection(w: Workload) -> np.ndarray:
    """Random vocabulary projection W: [vocab, d] (one row per vocabulary entry)."""
    return to_storage(_normal(_rng(w, _W), (w.vocab, w.d)), w.w_dtype)


def _stack(fn, outer, inner, threads=8):
    with ThreadPoolExecutor(threads) as ex:
        rows = list(ex.map(lambda ij: fn(*ij), [(i, j) for i in range(outer) for j in range(inner)]))
    first = rows[0]
    out = np.empty((outer, inner) + first.shape, dtype=first.dtype)
    for idx, r in enumerate(rows):
        out[idx // inner, idx % inner] = r
    return out


def full_kv(w: Workload, which: str) -> np.ndarray:
    """[B, Hkv, N, d] float32 (storage-dtype values)."""
    return _stack(lambda b, h: kv_slice(w, which, b, h), w.B, w.Hkv)


def full_window_q(w: Workload) -> np.ndarray:
    """[B, Hq, k, d]."""
    return _stack(lambda b, h: window_q(w, b, h), w.B, w.Hq)


def full_window_kv(w: Workload, which: str) -> np.ndarray:
    """[B, Hkv, k, d]."""
    return _stack(lambda b, h: window_kv(w, which, b, h), w.B, w.Hkv)


def full_probes(w: Workload) -> np.ndarray:
    """[Hkv, n_probes, d]."""
    return np.stack([probes(w, h) for h in range(w.Hkv)])


def tokens(w: Workload, *key, shape, high) -> np.ndarray:
    """Uniform random token ids in [0, high) (int64)."""
    return _rng(w, _PROMPT, *key).integers(0, high, size=shape, dtype=np.int64)


def uniform_ints(w: Workload, key, shape, low, high) -> np.ndarray:
    return _rng(w, 90, *key).integers(low, high, size=shape, dtype=np.int64)


def normal(w: Workload, key, shape, std=1.0, dtype="f32") -> np.ndarray:
    """Generic seeded N(0, std^2) draw rounded to a storage dtype (model weights,
    test tensors)."""
    x = _normal(_rng(w, 91, *key), shape)
    if std != 1.0:
        x = x * np.float32(std)
    return to_storage(x, dtype)
