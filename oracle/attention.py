"""Oracle: single-token decode attention (drafting) and causal window attention
(verification), float64.

TEST INFRASTRUCTURE (see the package header).

Source: "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference"
(neuraltrendhub.com summary), "What the paper found" and "Original abstract": the
target model runs on the compressed KV cache to draft tokens one at a time and on
the full KV cache to verify the drafted window.  The pages do not spell out
attention itself; this is standard scaled dot-product softmax attention with
grouped KV heads:

* q-head h reads kv-head floor(h / (Hq / Hkv)) (contiguous grouping);
* scores s_n = (q . k_n) * sm_scale, p = softmax(s), o = sum_n p_n v_n,
  lse = log sum_n exp(s_n) (natural log);
* verify row i of a k-row window sees the context [0, N) and window rows [0, i].

Parity: pinned by closed forms (one key, equal keys, one dominant key, equal-score
LSE), by the GQA head map, by agreement with torch's scaled_dot_product_attention
(a library routine) and, for verify, by causality and by its reduction to decode.
"""
import numpy as np


def _softmax_attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, sm_scale: float):
    """One query row q [d] over keys/vals [n, d]: returns (o [d], lse)."""
    s = (keys @ q) * sm_scale
    m = np.max(s)
    e = np.exp(s - m)
    l = np.sum(e)
    return (e @ vals) / l, m + np.log(l)


def decode(q, K, V, sm_scale, tail_k=None, tail_v=None):
    """One batch element.  q [Hq, d]; K, V [Hkv, n, d] (dequantized or gathered
    keys/values, any float type); optional full-precision tail rows
    tail_k/tail_v [Hkv, t, d] appended after the n cached tokens.
    Returns o [Hq, d] float64 and lse [Hq] float64."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if tail_k is not None and tail_k.shape[1] > 0:
        K = np.concatenate([K, np.asarray(tail_k, np.float64)], axis=1)
        V = np.concatenate([V, np.asarray(tail_v, np.float64)], axis=1)
    Hq, d = q.shape
    Hkv = K.shape[0]
    assert Hq % Hkv == 0
    grp = Hq // Hkv
    o = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    for h in range(Hq):
        g = h // grp
        o[h], lse[h] = _softmax_attend(q[h], K[g], V[g], sm_scale)
    return o, lse


def verify(q, Kc, Vc, Kw, Vw, sm_scale):
    """One batch element, row-by-row definition.  q [Hq, k, d]; context Kc, Vc
    [Hkv, N, d]; window Kw, Vw [Hkv, k, d].  Row i attends to the N context rows
    and window rows 0..i.  Returns o [Hq, k, d], lse [Hq, k] (float64)."""
    q = np.asarray(q, np.float64)
    Hq, k, d = q.shape
    o = np.zeros((Hq, k, d))
    lse = np.zeros((Hq, k))
    Kw = np.asarray(Kw)
    Vw = np.asarray(Vw)
    for i in range(k):
        o[:, i], lse[:, i] = decode(q[:, i], Kc, Vc, sm_scale, Kw[:, : i + 1], Vw[:, : i + 1])
    return o, lse


def verify_masked(q, Kc, Vc, Kw, Vw, sm_scale):
    """Same as verify(), written as one masked score matrix per head (used to
    cross-check the row loop)."""
    q = np.asarray(q, np.float64)
    Hq, k, d = q.shape
    Hkv, N, _ = Kc.shape
    grp = Hq // Hkv
    K = np.concatenate([np.asarray(Kc, np.float64), np.asarray(Kw, np.float64)], axis=1)
    V = np.concatenate([np.asarray(Vc, np.float64), np.asarray(Vw, np.float64)], axis=1)
    allowed = np.zeros((k, N + k), dtype=bool)
    allowed[:, :N] = True
    allowed[:, N:] = np.tril(np.ones((k, k), dtype=bool))
    o = np.zeros((Hq, k, d))
    lse = np.zeros((Hq, k))
    for h in range(Hq):
        g = h // grp
        S = (q[h] @ K[g].T) * sm_scale
        S = np.where(allowed, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        L = E.sum(axis=1, keepdims=True)
        o[h] = (E @ V[g]) / L
        lse[h] = (m + np.log(L))[:, 0]
    return o, lse
