"""Oracle: greedy verification by longest matching prefix.

TEST INFRASTRUCTURE (see the package header).

Source: neuraltrendhub.com summary "What the paper found": drafted tokens are
verified against the full KV cache so that greedy output is identical to full-KV
inference; podparley.com episode page, source 2 (Leviathan et al., speculative
decoding): the longest prefix on which draft and target agree is accepted, and the
target's token at the first disagreement is committed in its place.

Window convention (a reading; the pages do not fix it): the k verify rows take
inputs [last committed token, d_1 .. d_{k-1}] and row i's greedy token is the
target t_{i+1}.  With drafts d[0..k) and targets t[0..k):

* a = first i with d[i] != t[i], or k if none;
* committed tokens = d[0:a] followed by t[a] when a < k; n_commit = a + (a < k);
* the full cache grows by min(a + 1, k) rows (the rows of the verified inputs).

Parity: pinned by brute force over all string pairs of length <= 5 on a 3-letter
alphabet against os.path.commonprefix (a library routine).
"""
import numpy as np


def accept_row(draft, target):
    """One sequence.  Returns (accept_len, n_commit, commit list)."""
    k = len(draft)
    a = 0
    while a < k and draft[a] == target[a]:
        a += 1
    commit = list(draft[:a])
    if a < k:
        commit.append(target[a])
    return a, len(commit), commit


def accept(draft: np.ndarray, target: np.ndarray):
    """Batched: draft, target int [B, k] -> accept_len [B], n_commit [B],
    commit [B, k] (entries past n_commit are -1)."""
    draft = np.asarray(draft)
    target = np.asarray(target)
    B, k = draft.shape
    acc = np.zeros(B, np.int32)
    nc = np.zeros(B, np.int32)
    com = np.full((B, k), -1, np.int32)
    for b in range(B):
        a, n, c = accept_row(list(draft[b]), list(target[b]))
        acc[b], nc[b] = a, n
        com[b, :n] = c
    return acc, nc, com


def cache_advance(accept_len: int, k: int) -> int:
    return min(accept_len + 1, k)
