"""Oracle: draft/target tokens from attention outputs through a fixed random
vocabulary projection, greedy argmax.

TEST INFRASTRUCTURE (see the package header).

Source: neuraltrendhub.com summary "What the paper found" (greedy decoding output
must equal full-KV inference).  For the attention-only workloads there is no model,
so the token of a row is read from its attention output through a fixed random
projection W [V, d], one row per vocabulary entry (a reading; the pages do not
describe one):

* u = mean over the Hq q-heads of the row's attention output (float64);
* logits_v = u . W_v; token = argmax, equal logits going to the lowest index.

Parity: pinned by planted ties (lowest index wins) and by np.argmax's documented
first-occurrence rule.
"""
import numpy as np


def head_mean(o: np.ndarray) -> np.ndarray:
    """o [..., Hq, d] -> u [..., d] (float64)."""
    return np.asarray(o, np.float64).mean(axis=-2)


def logits(u: np.ndarray, W: np.ndarray) -> np.ndarray:
    """u [..., d], W [V, d] -> [..., V] (float64)."""
    return np.asarray(u, np.float64) @ np.asarray(W, np.float64).T


def argmax_lowest(x: np.ndarray) -> np.ndarray:
    """Argmax over the last axis; among equal maxima the lowest index."""
    x = np.asarray(x)
    m = x.max(axis=-1, keepdims=True)
    hit = x == m
    return np.argmax(hit, axis=-1).astype(np.int32)


def tokens_from_outputs(o: np.ndarray, W: np.ndarray) -> np.ndarray:
    """o [B, Hq, k, d] attention outputs -> tokens [B, k]."""
    u = head_mean(np.moveaxis(np.asarray(o), 2, 1))     # [B, k, d]
    return argmax_lowest(logits(u, W))
