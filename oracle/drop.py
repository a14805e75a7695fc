"""Oracle: token dropping by accumulated attention from probe queries, top-k
selection and gather.

TEST INFRASTRUCTURE (see the package header).

Source: podparley.com episode page, source 3 ("H2O: Heavy-Hitter Oracle"): keep
the tokens that collect the most attention; neuraltrendhub.com summary, "Original
abstract": token dropping is one of the compressor families.  Reading taken where
the pages are silent:

* score_n = sum over probes p of softmax_n(P_p . K_n * sm_scale), per (batch,
  kv-head), computed in float64;
* n_keep = ceil(keep_ratio * N); the n_keep largest scores are kept, equal scores
  going to the lower token index; kept indices are stored ascending and the K/V
  rows are gathered unchanged.

Parity: pinned by brute-force ranking on small inputs, by the invariant
sum_n score_n = number of probes, by the equal-keys and heavy-hitter cases, and by
keep-all reducing to the dense cache bit for bit.
"""
import math
import numpy as np


def n_keep(N: int, keep_ratio: float) -> int:
    return min(N, max(1, int(math.ceil(keep_ratio * N - 1e-9))))


def scores(K: np.ndarray, P: np.ndarray, sm_scale: float) -> np.ndarray:
    """K [N, d] keys of one (batch, kv-head); P [n_probes, d] probes.
    Returns accumulated attention [N] (float64)."""
    K = np.asarray(K, np.float64)
    P = np.asarray(P, np.float64)
    acc = np.zeros(K.shape[0])
    for p in range(P.shape[0]):
        s = (K @ P[p]) * sm_scale
        e = np.exp(s - s.max())
        acc += e / e.sum()
    return acc


def select(score: np.ndarray, keep: int) -> np.ndarray:
    """Indices of the `keep` largest scores, ties to the lower index, ascending.
    Works in the precision of `score` (pass float32 scores to reproduce a float32
    decision)."""
    score = np.asarray(score)
    order = np.lexsort((np.arange(score.shape[0]), -score.astype(np.float64)))
    return np.sort(order[:keep]).astype(np.int32)


def gather(x: np.ndarray, idx: np.ndarray) -> np.ndarray:
    return np.asarray(x)[np.asarray(idx, np.int64)]
