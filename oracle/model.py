"""Oracle: a small Llama-style pre-norm decoder in float64, its greedy full-KV
decoding, and the VeriCache draft-and-verify round.

TEST INFRASTRUCTURE (see the package header).

Source for the round: "VeriCache: Turning Lossy KV Cache into Lossless LLM
Inference" (neuraltrendhub.com summary), "What the paper found" and "Original
abstract": the target model drafts with the compressed KV cache, the drafts are
verified against the full KV cache and the output equals greedy full-KV decoding.
Greedy prefix acceptance: oracle.accept.

The model itself is not on the pages (they evaluate trained models); this is a
plain reading of a Llama-style decoder, random-initialised:
  x = E[token]; per layer: h = rmsnorm(x) ; q, k, v = h Wqkv^T ; rotary(q, k) ;
  x += attention(q, k, v) Wo^T ; h = rmsnorm(x) ; x += (silu(h Wg^T) * h Wu^T) Wd^T ;
  logits = rmsnorm(x) Whead^T.
Rotary embedding: pairs (j, j + hd/2) rotated by pos * theta^(-2j/hd).

The compressed draft cache of one layer and sequence holds KIVI-quantized groups of
G committed tokens (dequantized here) followed by a full-precision tail (committed
tokens that do not fill a group yet, then the round's draft tokens).  After each
round the committed rows' keys/values -- as computed by the verify pass -- replace
the draft rows in the tail, and every full group of G committed tail rows is
quantized into the compressed part (a reading; the pages do not describe the
cache update).

Parity: the model functions are pinned by torch's rms_norm and silu and by rotary
invariants; the round by the pages' own invariant -- output identical to greedy
full-KV decoding -- for the compressed drafter, an adversarial random drafter and a
perfect (full-KV) drafter.  The decoder's weights are random: parity of the model
itself against a trained model is unpinned by construction.
"""
from dataclasses import dataclass, field
import numpy as np

from . import attention as A
from . import quant as Q
from . import accept as AC
from .logits import argmax_lowest


def rmsnorm(x, w, eps=1e-5):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def rope(x, pos, theta=10000.0):
    """x [n, H, hd], pos [n] -> rotated copy (float64)."""
    x = np.asarray(x, np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-2.0 * np.arange(half) / hd)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]          # [n, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x):
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


@dataclass
class Config:
    layers: int
    d_model: int
    Hq: int
    Hkv: int
    hd: int
    ffn: int
    vocab: int
    theta: float = 10000.0
    eps: float = 1e-5


@dataclass
class Weights:
    E: np.ndarray                 # [V, dm]
    wqkv: list                    # [(Hq + 2 Hkv) hd, dm] per layer
    wo: list                      # [dm, Hq hd]
    wgu: list                     # [2F, dm]: gate rows then up rows
    wd: list                      # [dm, F]
    n1: list                      # [dm]
    n2: list                      # [dm]
    nf: np.ndarray                # [dm]
    head: np.ndarray              # [V, dm]


class Decoder:
    """Forward passes over explicit per-layer key/value arrays (float64)."""

    def __init__(self, cfg: Config, w: Weights):
        self.c = cfg
        self.w = w
        self.scale = cfg.hd ** -0.5

    def _qkv(self, l, h, pos):
        c = self.c
        qkv = h @ np.asarray(self.w.wqkv[l], np.float64).T
        n = h.shape[0]
        q = qkv[:, : c.Hq * c.hd].reshape(n, c.Hq, c.hd)
        k = qkv[:, c.Hq * c.hd:(c.Hq + c.Hkv) * c.hd].reshape(n, c.Hkv, c.hd)
        v = qkv[:, (c.Hq + c.Hkv) * c.hd:].reshape(n, c.Hkv, c.hd)
        return rope(q, pos, c.theta), rope(k, pos, c.theta), v

    def _mlp(self, l, x):
        c = self.c
        h = rmsnorm(x, self.w.n2[l], c.eps)
        gu = h @ np.asarray(self.w.wgu[l], np.float64).T
        return x + (silu(gu[:, : c.ffn]) * gu[:, c.ffn:]) @ np.asarray(self.w.wd[l], np.float64).T

    def logits(self, x):
        return rmsnorm(x, self.w.nf, self.c.eps) @ np.asarray(self.w.head, np.float64).T

    def forward_full(self, tokens, pos0, kv):
        """n consecutive tokens of one sequence at positions pos0.. attending causally
        to the full cache kv[l] = (K [Hkv, L, hd], V) with L = pos0 rows.  Returns the
        logits [n, V] and the new rows' (K, V) per layer [Hkv, n, hd] (not appended)."""
        c = self.c
        n = len(tokens)
        pos = np.arange(pos0, pos0 + n)
        x = np.asarray(self.w.E, np.float64)[np.asarray(tokens)]
        new = []
        for l in range(c.layers):
            h = rmsnorm(x, self.w.n1[l], c.eps)
            q, k, v = self._qkv(l, h, pos)
            Kc, Vc = kv[l]
            kw, vw = k.transpose(1, 0, 2), v.transpose(1, 0, 2)
            o, _ = A.verify(q.transpose(1, 0, 2), Kc, Vc, kw, vw, self.scale)       # [Hq, n, hd]
            x = x + o.transpose(1, 0, 2).reshape(n, c.Hq * c.hd) @ np.asarray(self.w.wo[l], np.float64).T
            x = self._mlp(l, x)
            new.append((kw, vw))
        return self.logits(x), new

    def forward_draft(self, token, pos, ckv):
        """One token at position pos attending to the compressed cache ckv[l] =
        (K_hat [Hkv, m, hd], V_hat, tail_K [Hkv, t, hd], tail_V); its own key/value
        row is appended to the tail (in place).  Returns logits [V]."""
        c = self.c
        x = np.asarray(self.w.E, np.float64)[[token]]
        for l in range(c.layers):
            h = rmsnorm(x, self.w.n1[l], c.eps)
            q, k, v = self._qkv(l, h, np.array([pos]))
            Kh, Vh, tk, tv = ckv[l]
            tk = np.concatenate([tk, k.transpose(1, 0, 2)], axis=1)
            tv = np.concatenate([tv, v.transpose(1, 0, 2)], axis=1)
            ckv[l] = (Kh, Vh, tk, tv)
            o, _ = A.decode(q[0], Kh, Vh, self.scale, tk, tv)                        # [Hq, hd]
            x = x + o.reshape(1, c.Hq * c.hd) @ np.asarray(self.w.wo[l], np.float64).T
            x = self._mlp(l, x)
        return self.logits(x)[0]


def random_weights(cfg: Config, rng: np.random.Generator, std=0.02) -> Weights:
    def n(*shape):
        return rng.standard_normal(shape) * std

    L = cfg.layers
    return Weights(
        E=n(cfg.vocab, cfg.d_model),
        wqkv=[n((cfg.Hq + 2 * cfg.Hkv) * cfg.hd, cfg.d_model) for _ in range(L)],
        wo=[n(cfg.d_model, cfg.Hq * cfg.hd) for _ in range(L)],
        wgu=[n(2 * cfg.ffn, cfg.d_model) for _ in range(L)],
        wd=[n(cfg.d_model, cfg.ffn) for _ in range(L)],
        n1=[1.0 + n(cfg.d_model) for _ in range(L)],
        n2=[1.0 + n(cfg.d_model) for _ in range(L)],
        nf=1.0 + n(cfg.d_model),
        head=n(cfg.vocab, cfg.d_model))


# ---------------------------------------------------------------- decoding

def prefill(dec: Decoder, prompt):
    """Runs the prompt; returns (full cache per layer, first greedy token)."""
    c = dec.c
    empty = [(np.zeros((c.Hkv, 0, c.hd)), np.zeros((c.Hkv, 0, c.hd))) for _ in range(c.layers)]
    lg, new = dec.forward_full(list(prompt), 0, empty)
    return [(k, v) for k, v in new], int(argmax_lowest(lg[-1]))


def greedy(dec: Decoder, prompt, T):
    """Greedy full-KV decoding: the first T generated tokens."""
    kv, tok = prefill(dec, prompt)
    out = [tok]
    pos = len(prompt)
    while len(out) < T:
        lg, new = dec.forward_full([tok], pos, kv)
        kv = [(np.concatenate([K, nk], 1), np.concatenate([V, nv], 1)) for (K, V), (nk, nv) in zip(kv, new)]
        tok = int(argmax_lowest(lg[0]))
        out.append(tok)
        pos += 1
    return out


@dataclass
class RoundStats:
    rounds: int = 0
    accept_lens: list = field(default_factory=list)


def vericache(dec: Decoder, prompt, T, k, bits=(2, 2), group=8, scale_dtype="f32", drafter="compressed",
              rng=None, stats: RoundStats = None):
    """Draft-and-verify decoding until T tokens are committed; returns them.

    drafter: "compressed" (the target model on the compressed cache), "adversarial"
    (uniform random tokens) or "perfect" (the target model on the full cache)."""
    c = dec.c
    kv, tok = prefill(dec, prompt)
    L = len(prompt)
    kb, vb = bits

    def compress_rows(K, V):
        """Dequantized KIVI copy of [Hkv, G*n, hd] rows, group by group."""
        Kh = np.zeros_like(K)
        Vh = np.zeros_like(V)
        for h in range(c.Hkv):
            for g0 in range(0, K.shape[1], group):
                cs = Q.compress_slice(K[h, g0:g0 + group].astype(np.float32), V[h, g0:g0 + group].astype(np.float32),
                                      kb, vb, group, scale_dtype)
                Kh[h, g0:g0 + group], Vh[h, g0:g0 + group] = Q.dequantize_slice(cs, c.hd, kb, vb, group)
        return Kh, Vh

    # compressed cache: whole groups of the prompt, the rest in the tail
    n_main = (L // group) * group
    ccache = []
    for K, V in kv:
        Kh, Vh = compress_rows(K[:, :n_main], V[:, :n_main])
        ccache.append([Kh, Vh, K[:, n_main:].copy(), V[:, n_main:].copy()])
    out = [tok]
    while len(out) < T:
        # ---- draft k tokens
        if drafter == "adversarial":
            drafts = [int(x) for x in rng.integers(0, c.vocab, size=k)]
        else:
            drafts = []
            cur = tok
            if drafter == "compressed":
                work = [tuple(x) for x in ccache]
                for i in range(k):
                    lg = dec.forward_draft(cur, L + i, work)
                    cur = int(argmax_lowest(lg))
                    drafts.append(cur)
            else:
                work = [(K, V) for K, V in kv]
                for i in range(k):
                    lg, new = dec.forward_full([cur], L + i, work)
                    work = [(np.concatenate([K, nk], 1), np.concatenate([V, nv], 1))
                            for (K, V), (nk, nv) in zip(work, new)]
                    cur = int(argmax_lowest(lg[0]))
                    drafts.append(cur)
        # ---- verify the window [tok, d_1 .. d_{k-1}] against the full cache
        window = [tok] + drafts[: k - 1]
        lg, new = dec.forward_full(window, L, kv)
        targets = [int(t) for t in argmax_lowest(lg)]
        a, n_commit, commit = AC.accept_row(drafts, targets)
        if stats is not None:
            stats.rounds += 1
            stats.accept_lens.append(a)
        adv = AC.cache_advance(a, k)
        # ---- commit: full cache and compressed tail take the verified rows
        kv = [(np.concatenate([K, nk[:, :adv]], 1), np.concatenate([V, nv[:, :adv]], 1))
              for (K, V), (nk, nv) in zip(kv, new)]
        for l, (nk, nv) in enumerate(new):
            Kh, Vh, tk, tv = ccache[l]
            tk = np.concatenate([tk, nk[:, :adv]], 1)
            tv = np.concatenate([tv, nv[:, :adv]], 1)
            full = (tk.shape[1] // group) * group
            if full:
                Kn, Vn = compress_rows(tk[:, :full], tv[:, :full])
                Kh, Vh = np.concatenate([Kh, Kn], 1), np.concatenate([Vh, Vn], 1)
                tk, tv = tk[:, full:], tv[:, full:]
            ccache[l] = [Kh, Vh, tk, tv]
        L += adv
        out.extend(commit)
        tok = commit[-1]
    return out[:T]
