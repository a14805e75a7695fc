"""Oracle: orthonormal rotation of each head's channels before quantization.

TEST INFRASTRUCTURE (see the package header).

Source: the neuraltrendhub.com summary "VeriCache: Turning Lossy KV Cache into
Lossless LLM Inference", "What the paper found", names RotateKV and TurboQuant among
the compressors behind the uniform compressor interface, and the pith.science record
of arXiv 2605.17613 lists RotateKV in its references as rotation-based low-bit KV
quantization that spreads outlier channels.  The pages give no rotation; the plainest
reading is a fixed orthonormal Walsh-Hadamard rotation of the d channels of every
key, value and query row: x -> x H / sqrt(d), H the Sylvester Hadamard matrix
(H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]).  The rotation is symmetric and
orthogonal, so it is its own inverse and keeps every dot product: scores are
unchanged when queries and keys are both rotated, and an attention output over
rotated values is rotated back by the same map.

Parity: pinned by a hand-computed example (tests/golden/hadamard_d4.txt), the
library Hadamard matrix, orthogonality, the involution, dot-product preservation and
the spread of a single outlier channel.
"""
import numpy as np


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1, int64."""
    assert d >= 1 and d & (d - 1) == 0, "d must be a power of two"
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_rows(x) -> np.ndarray:
    """x [..., d] -> x H / sqrt(d) in float64 (rows rotated independently)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    return (x @ hadamard(d).astype(np.float64)) / np.sqrt(d)
