"""End-to-end draft-and-verify rounds of a decoder on one GPU, sequencing the
library's kernels (every arithmetic step runs in libvc.so; this module only issues
calls, keeps lengths and owns device/pinned memory through torch).

The round follows "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference"
(neuraltrendhub.com summary, "What the paper found" and "Original abstract"):
  * the full KV cache of every layer lives in pinned host memory and is staged to the
    device layer by layer on a side stream while the model drafts k tokens on the
    compressed (KIVI-quantized) cache; the device holds R layer slots (a ring), so
    layers past the first R are staged while the verify pass runs the earlier ones;
  * the k-row window [last committed token, d_1 .. d_{k-1}] is verified against the
    full cache; the longest prefix on which drafts and greedy targets agree is
    committed, plus the target at the first disagreement;
  * the verified rows' keys/values are appended to the host full cache and to the
    compressed cache's tail; whole groups of the tail are quantized into the
    compressed part.
Greedy full-KV decoding with the same kernels is the reference the output must equal.
"""
from dataclasses import dataclass
import sys
import time
import numpy as np
import torch

from . import _lib as L

BF16 = torch.bfloat16


@dataclass
class ModelShape:
    layers: int
    d_model: int
    Hq: int
    Hkv: int
    hd: int
    ffn: int
    vocab: int
    theta: float = 10000.0
    eps: float = 1e-5


class DecoderGPU:
    """Random-initialised Llama-style decoder: bf16 weights on the device."""

    def __init__(self, shape: ModelShape, weights: dict, max_rows: int, device="cuda"):
        self.s = shape
        self.w = weights
        self.dev = device
        s = shape
        z = dict(device=device, dtype=BF16)
        self.max_rows = max_rows
        self.x = torch.empty(max_rows, s.d_model, **z)
        self.h = torch.empty(max_rows, s.d_model, **z)
        self.qkv = torch.empty(max_rows, (s.Hq + 2 * s.Hkv) * s.hd, **z)
        self.q = torch.empty(max_rows * s.Hq * s.hd, **z)
        self.attn = torch.empty(max_rows * s.Hq * s.hd, **z)
        self.rows = torch.empty(max_rows, s.Hq * s.hd, **z)
        self.gu = torch.empty(max_rows, 2 * s.ffn, **z)
        self.act = torch.empty(max_rows, s.ffn, **z)
        self.logits = torch.empty(max_rows, s.vocab, device=device, dtype=torch.float32)
        # gate/up rows interleaved in blocks of 8 for the product fused with SwiGLU, and
        # the q/k rows of each head with their rotation partners for the product fused
        # with the rotary embedding (copies of the weights in the layouts those read)
        self.wgu_i = [L.swiglu_interleave(t) for t in weights["wgu"]]
        self.wqkv_r = [L.rope_interleave(t, s.Hq, s.Hkv, s.hd) for t in weights["wqkv"]]

    def forward(self, tokens, B, k, attend, head=True):
        """tokens: int32 [B*k] (row b*k + i = token i of sequence b).  attend(l, M)
        runs layer l's attention on self.qkv[:M] and leaves its output as rows
        [M, Hq*hd] in self.rows[:M].  Returns float32 logits [M, vocab] (a view of
        self.logits), or None when head is False: prompt chunks, whose projections
        use the many-row GEMM (the decode and verify passes use the batch-invariant
        one, so that verify rows equal one-row greedy steps bit for bit)."""
        s, w = self.s, self.w
        M = B * k
        x, h = self.x[:M], self.h[:M]
        mm = L.vc_gemm_bf16 if head else L.vc_gemm_bf16_wide
        L.vc_embed(w["E"], tokens, x)
        for l in range(s.layers):
            L.vc_rmsnorm(x, w["n1"][l], h, eps=s.eps)
            # steps of up to 32 rows: the batch-invariant product with the rotary scatter in
            # its epilogue (bit for bit the two calls; the verify pass keeps them apart,
            # where the layer's full cache is waited for after the projection)
            rope = getattr(attend, "rope", None) if head and M <= 32 else None
            if rope is not None:
                t = rope(l, M)
                L.vc_gemm_bf16_rope(h, self.wqkv_r[l], t["B"], t["k"], s.Hq, s.Hkv, s.hd, t["pos"], t["q"], t["K"],
                                    t["V"], t["row0"], theta=s.theta)
            else:
                mm(h, w["wqkv"][l], self.qkv[:M])
            attend(l, M)
            mm(self.rows[:M], w["wo"][l], x, R=x)
            L.vc_rmsnorm(x, w["n2"][l], h, eps=s.eps)
            if head:  # the batch-invariant product with SwiGLU in its epilogue (bit for bit the two calls)
                L.vc_gemm_bf16_swiglu(h, self.wgu_i[l], self.act[:M])
            else:
                mm(h, w["wgu"][l], self.gu[:M])
                L.vc_swiglu(self.gu[:M], self.act[:M])
            mm(self.act[:M], w["wd"][l], x, R=x)
        if not head:
            return None
        L.vc_rmsnorm(x, w["nf"], h, eps=s.eps)
        L.vc_gemm_bf16(h, w["head"], self.logits[:M])
        return self.logits[:M]


def _i32(x, device):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=device)


def _round_up(x, m):
    return (x + m - 1) // m * m


class FullCache:
    """Per-layer device full KV [B, Hkv, rows, hd] (bf16), resident."""

    def __init__(self, shape: ModelShape, B, rows, device="cuda", layers=None):
        n = shape.layers if layers is None else layers
        self.k = [torch.zeros(B, shape.Hkv, rows, shape.hd, dtype=BF16, device=device) for _ in range(n)]
        self.v = [torch.zeros_like(t) for t in self.k]
        self.rows = rows

    def clone(self):
        c = FullCache.__new__(FullCache)
        c.k, c.v, c.rows = [t.clone() for t in self.k], [t.clone() for t in self.v], self.rows
        return c

    # the hooks of a forward pass over a resident cache
    def begin(self, n_rows, lo, hi):
        pass

    def acquire(self, l):
        return self.k[l], self.v[l]

    def release(self, l):
        pass


class HostFullKV:
    """The full KV of every layer in pinned host memory, staged into `slots` device
    buffers (layer l uses slot l % slots) on a side stream.

    A forward pass over it calls begin(n_rows, lo, hi) once, then acquire(l) before
    and release(l) after layer l's attention:
      begin    stages rows [0, n_rows) of layers [0, slots) (these copies overlap
               whatever the compute stream does next, e.g. drafting);
      acquire  makes the compute stream wait for layer l's rows;
      release  writes rows [lo, hi) of the slot back to the host (the pass's new
               keys/values) and stages layer l + slots into the freed slot."""

    def __init__(self, src: FullCache, slots: int, device="cuda"):
        n = len(src.k)
        self.layers, self.slots = n, max(1, min(slots, n))
        self.host_k = [torch.empty(t.shape, dtype=BF16, pin_memory=True) for t in src.k]
        self.host_v = [torch.empty(t.shape, dtype=BF16, pin_memory=True) for t in src.v]
        for l in range(n):
            self.host_k[l].copy_(src.k[l])
            self.host_v[l].copy_(src.v[l])
        self.slot_k = [torch.zeros_like(src.k[0]) for _ in range(self.slots)]
        self.slot_v = [torch.zeros_like(src.v[0]) for _ in range(self.slots)]
        self.rows = src.rows
        self.stream = torch.cuda.Stream()
        self.staged = [torch.cuda.Event() for _ in range(n)]
        self.freed = [torch.cuda.Event() for _ in range(n)]
        self.n_rows = self.lo = self.hi = 0
        self.bytes_staged = 0

    def _stage(self, l):
        j = l % self.slots
        L.vc_stage_full_kv(self.host_k[l], self.host_v[l], self.slot_k[j], self.slot_v[j], 0, self.n_rows,
                           copy_stream=self.stream, done=self.staged[l])
        self.bytes_staged += 2 * self.host_k[l][:, :, : self.n_rows].numel() * 2

    def begin(self, n_rows, lo, hi):
        self.n_rows, self.lo, self.hi = n_rows, lo, hi
        for l in range(self.slots):
            self._stage(l)

    def acquire(self, l):
        torch.cuda.current_stream().wait_event(self.staged[l])
        j = l % self.slots
        return self.slot_k[j], self.slot_v[j]

    def release(self, l):
        j = l % self.slots
        self.freed[l].record()
        self.stream.wait_event(self.freed[l])
        L.vc_stage_full_kv_d2h(self.slot_k[j], self.slot_v[j], self.host_k[l], self.host_v[l], self.lo, self.hi,
                               copy_stream=self.stream)
        if l + self.slots < self.layers:
            self._stage(l + self.slots)


class FileFullKV(HostFullKV):
    """The remote-prefix-cache setting (summary page, "What the paper found" and
    "Original abstract"): the full KV of the prompt (rows [0, prefix_rows)) lives in a
    store off the host's pinned memory -- a file here, read by the library's stager
    threads, optionally capped at a link rate -- and is staged from there every
    round; rows written after the prompt (the generated tokens) stay in pinned host
    memory as in HostFullKV.  The file holds, per layer, K then V, each
    [B, Hkv, prefix_rows, hd] bf16; it is unlinked at creation and lives as long as
    its descriptor.  The prompt rows of the pinned copy are cleared, so every prompt
    row a verify pass reads has come through the file."""

    def __init__(self, src: FullCache, slots: int, prefix_rows: int, device="cuda", directory=None,
                 n_threads=8, chunk_bytes=16 << 20, n_buffers=16, max_bytes_per_s=0.0):
        import os
        import tempfile
        super().__init__(src, slots, device)
        P = int(prefix_rows)
        assert 0 < P <= src.rows
        self.P = P
        if directory is None:
            directory = tempfile.gettempdir()
        fd, path = tempfile.mkstemp(prefix="vc_prefix_", dir=directory)
        os.unlink(path)
        self.fd = fd
        self.layer_bytes = 2 * src.k[0][:, :, :P].numel() * 2
        with os.fdopen(os.dup(fd), "wb") as f:   # the prefix store, written once by the prefill
            for l in range(self.layers):
                for t in (self.host_k[l], self.host_v[l]):
                    f.write(t[:, :, :P].contiguous().view(torch.int16).numpy().tobytes())
                    t[:, :, :P].zero_()
        self.stager = L.FileStager(n_threads, chunk_bytes, n_buffers, max_bytes_per_s)
        self.file_done = [torch.cuda.Event() for _ in range(self.layers)]
        self.tickets = [None] * self.layers
        self.bytes_from_file = 0

    def _stage(self, l):
        j = l % self.slots
        P, n = self.P, self.n_rows
        off = l * self.layer_bytes
        self.tickets[l] = self.stager.stage(self.fd, off, off + self.layer_bytes // 2, self.slot_k[j], self.slot_v[j],
                                            P, 0, min(P, n), copy_stream=self.stream, done=self.file_done[l])
        self.bytes_from_file += 2 * self.slot_k[j][:, :, : min(P, n)].numel() * 2
        L.vc_stage_full_kv(self.host_k[l], self.host_v[l], self.slot_k[j], self.slot_v[j], min(P, n), max(P, n),
                           copy_stream=self.stream, done=self.staged[l])
        self.bytes_staged += 2 * self.host_k[l][:, :, : n].numel() * 2

    def acquire(self, l):
        self.stager.wait(self.tickets[l])
        self.tickets[l] = None
        torch.cuda.current_stream().wait_event(self.file_done[l])
        return super().acquire(l)

    def release(self, l):
        assert self.lo >= self.P, "rows of the prompt are never rewritten"
        super().release(l)

    def close(self):
        import os
        for t in self.tickets:
            if t is not None:
                self.stager.wait(t)
        self.tickets = [None] * self.layers
        self.stager.close()
        if self.fd is not None:
            os.close(self.fd)
            self.fd = None

    def __del__(self, _finalizing=sys.is_finalizing):
        if not _finalizing() and getattr(self, "fd", None) is not None:
            try:
                self.close()
            except Exception:
                pass


def attend_full(dec: DecoderGPU, cache, B, k, pos, row0, ctx_len, ctx_lens, split_tokens, ws, after=None):
    """Attention callback over a full cache (FullCache or HostFullKV): rotary + scatter
    of the rows' keys/values into the cache at rows row0[b] + i, then causal verify
    attention over rows [0, row0[b] + i].  after(l, K, V) runs before the layer's
    cache is released."""
    s = dec.s
    roped = {}

    def rope(l, M):
        """The rotary scatter's destinations, for a projection that applies it (the
        layer's cache is acquired here, before the projection writes into it)."""
        K, V = cache.acquire(l)
        q = dec.q[: M * s.Hq * s.hd].view(B, s.Hq, k, s.hd)
        roped[l] = (q, K, V)
        return dict(B=B, k=k, pos=pos, q=q, K=K, V=V, row0=row0)

    def attend(l, M):
        if l in roped:
            q, K, V = roped.pop(l)
        else:
            K, V = cache.acquire(l)
            q = dec.q[: M * s.Hq * s.hd].view(B, s.Hq, k, s.hd)
            L.vc_rope_qkv(dec.qkv[:M], B, k, s.Hq, s.Hkv, s.hd, pos, q, K, V, row0, theta=s.theta)
        out = dec.attn[: M * s.Hq * s.hd].view(B, s.Hq, k, s.hd)
        L.vc_verify_attn_full(q, K, V, ctx_len, out, ctx_lens=ctx_lens, split_tokens=split_tokens, ws=ws)
        if after is not None:
            after(l, K, V)
        cache.release(l)
        L.vc_heads_to_rows(out, dec.rows[:M])
    attend.rope = rope
    return attend


def attend_draft(dec: DecoderGPU, ckvs, B, pos, tail_row, main_lens, tail_lens, ws):
    """Attention callback of one draft step: rotary + append of the token's key/value
    to the compressed cache's tail, then decode attention over compressed rows + tail."""
    s = dec.s
    roped = set()

    def rope(l, M):
        """The rotary scatter's destinations (the compressed cache's tail), for a
        projection that applies it."""
        ckv = ckvs[l]
        roped.add(l)
        q = dec.q[: M * s.Hq * s.hd].view(B, s.Hq, 1, s.hd)
        return dict(B=B, k=1, pos=pos, q=q, K=ckv.tail_k, V=ckv.tail_v, row0=tail_row)

    def attend(l, M):
        ckv = ckvs[l]
        q = dec.q[: M * s.Hq * s.hd].view(B, s.Hq, 1, s.hd)
        if l in roped:
            roped.discard(l)
        else:
            L.vc_rope_qkv(dec.qkv[:M], B, 1, s.Hq, s.Hkv, s.hd, pos, q, ckv.tail_k, ckv.tail_v, tail_row,
                          theta=s.theta)
        out = dec.rows[:M].view(B, s.Hq, s.hd)
        L.vc_decode_attn_compressed(ckv, q.view(B, s.Hq, s.hd), out, main_lens=main_lens, tail_lens=tail_lens, ws=ws)
    attend.rope = rope
    return attend


class Session:
    """Prompt state shared by the greedy reference and the draft-and-verify loop.

    The prompt's first N0 - 1 tokens run through the verify kernel in chunks (causal
    attention over the rows before the chunk plus the chunk itself); the last prompt
    token then runs as a one-row step, like every later greedy step, and gives the
    first generated token."""

    def __init__(self, dec: DecoderGPU, prompt: np.ndarray, k: int, gen: int, chunk=512, group=32, bits=(2, 2),
                 device="cuda"):
        self.dec, self.k, self.gen, self.group, self.bits = dec, k, gen, group, bits
        s = dec.s
        self.B, self.N0 = prompt.shape
        B, N0 = self.B, self.N0
        assert N0 >= 1 and B * max(k, chunk) <= dec.max_rows
        self.rows = _round_up(N0 + gen + 2 * k, 32)
        self.split = L.vc_verify_split_tokens(B, s.Hkv, self.rows)
        self.device = device
        self.ver_ws = L.workspace(L.vc_verify_workspace_bytes(B, s.Hq, s.Hkv, s.hd, max(k, chunk), self.rows,
                                                              self.split), device)
        self.cache = FullCache(s, B, self.rows, device)
        tok = torch.as_tensor(prompt.astype(np.int32), device=device)
        for c0 in range(0, N0 - 1, chunk):
            c = min(chunk, N0 - 1 - c0)
            toks = tok[:, c0:c0 + c].contiguous().view(-1)
            pos = (torch.arange(c, device=device, dtype=torch.int32) + c0).repeat(B)
            row0 = torch.full((B,), c0, dtype=torch.int32, device=device)
            dec.forward(toks, B, c, attend_full(dec, self.cache, B, c, pos, row0, c0, None, self.split, self.ver_ws),
                        head=False)
        self.first = greedy_step(dec, self.cache, tok[:, N0 - 1].contiguous(), N0 - 1, self.split, self.ver_ws)
        self.first_logits = dec.logits[:B].clone()   # of the last prompt position
        torch.cuda.synchronize()


def greedy_step(dec: DecoderGPU, cache, tok, L_ctx: int, split, ws):
    """One greedy full-KV step of every sequence (all at context length L_ctx): the
    tokens' keys/values go to cache row L_ctx; returns the next tokens (int32 [B])."""
    B = tok.numel()
    pos = torch.full((B,), L_ctx, dtype=torch.int32, device=tok.device)
    cache.begin(L_ctx, L_ctx, L_ctx + 1)
    lg = dec.forward(tok, B, 1, attend_full(dec, cache, B, 1, pos, pos, L_ctx, None, split, ws))
    nxt = torch.empty(B, dtype=torch.int32, device=tok.device)
    L.vc_argmax_rows(lg, nxt)
    return nxt


class Greedy:
    """Greedy full-KV decoding from a session's prompt: the output reference, and the
    baselines of the throughput figures -- full KV resident on the device
    (slots=None) or staged from pinned host memory every step (slots=R).

    With the cache resident and graph=True one step is captured once as a HIP graph
    (its launches replayed without host overhead): positions come from a device
    buffer and the attention reads per-sequence lengths, with the cache's row count
    as the bound -- the same arithmetic as the uncaptured step (splits sit at
    absolute positions)."""

    def __init__(self, sess: Session, slots=None, graph=True):
        self.sess = sess
        res = sess.cache.clone()
        self.cache = res if slots is None else HostFullKV(res, slots, sess.device)
        if slots is not None:
            del res
        self.tok = sess.first.clone()
        self.out = [self.tok]
        self.L = sess.N0
        self.graph = None
        if graph and slots is None:
            dec, B = sess.dec, sess.B
            self.g_tok = self.tok.clone()
            self.g_L = torch.full((B,), self.L, dtype=torch.int32, device=sess.device)
            self.g_next = torch.empty(B, dtype=torch.int32, device=sess.device)
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph):
                lg = dec.forward(self.g_tok, B, 1, attend_full(dec, self.cache, B, 1, self.g_L, self.g_L,
                                                               sess.rows - 1, self.g_L, sess.split, sess.ver_ws))
                L.vc_argmax_rows(lg, self.g_next)
                self.g_tok.copy_(self.g_next)

    def step(self):
        sess = self.sess
        if self.graph is not None:
            self.g_L.fill_(self.L)
            self.graph.replay()
            self.tok = self.g_next.clone()
        else:
            self.tok = greedy_step(sess.dec, self.cache, self.tok, self.L, sess.split, sess.ver_ws)
        self.out.append(self.tok)
        self.L += 1

    def run(self, n=None):
        n = self.sess.gen if n is None else n
        while len(self.out) < n:
            self.step()
        torch.cuda.synchronize()
        return torch.stack(self.out[:n], 1).cpu().numpy()


class HorizonPolicy:
    """Adaptive draft horizon from a cost model (summary page, "What the paper found":
    the draft horizon is extended to exploit long acceptance runs): each round drafts
    with the horizon k of `horizons` that maximises the estimated commits per second,
    E[min(a + 1, k)] / T(k).  a is a sequence's accepted draft count; a round drafted
    with horizon kr reveals min(a, kr - 1), which fixes min(a + 1, k) for every
    k <= kr, so E[min(a + 1, k)] is the mean over the recent rounds drafted with a
    horizon of at least k.  T(k) is the mean wall time of the recent rounds drafted with
    k.  Every horizon is tried once, the longest first, and the longest is drafted again
    every `explore` rounds so that its statistics stay current."""

    def __init__(self, horizons, explore=8, memory=64):
        self.h = sorted(set(int(k) for k in horizons))
        self.explore, self.memory = explore, memory
        self.times = {k: [] for k in self.h}
        self.obs = []                       # (horizon, accepted counts of the active sequences)
        self.rounds = 0
        self.chosen = {k: 0 for k in self.h}

    def choose(self):
        untried = [k for k in reversed(self.h) if not self.times[k]]
        if untried:
            return untried[0]
        if self.rounds % self.explore == 0:
            return self.h[-1]
        best, kb = -1.0, self.h[-1]
        for k in self.h:
            seen = [np.minimum(a + 1, k) for kr, a in self.obs if kr >= k and len(a)]
            if not seen:
                continue
            rate = float(np.mean(np.concatenate(seen))) / float(np.mean(self.times[k][-16:]))
            if rate > best:
                best, kb = rate, k
        return kb

    def update(self, k, seconds, accepted):
        self.rounds += 1
        self.chosen[k] += 1
        self.times[k].append(seconds)
        self.obs.append((k, np.asarray(accepted, np.int64)))
        del self.obs[:-self.memory]


class VeriCacheLoop:
    """Draft-and-verify decoding.  slots=R keeps the full KV in pinned host memory and
    stages it through R device slots (R = layers: every layer staged during
    drafting); slots=None keeps it resident on the device (no PCIe traffic; for
    separating transfer time from compute).

    graph=True captures the k draft steps once as a HIP graph: their inputs
    (positions, tail rows, lengths, the first token) live in static device buffers
    refreshed before each replay, and the compressed caches' descriptors carry fixed
    bounds (capacity and tail capacity) while the kernels read the per-sequence
    lengths."""

    def __init__(self, sess: Session, slots=2, graph=True, horizons=None, prefix_store=None):
        """prefix_store: None, or the keyword arguments of FileFullKV (without src,
        slots, prefix_rows) to stage the prompt's full KV from a file instead of
        pinned host memory (needs slots)."""
        self.sess = sess
        # draft horizons: the session's k alone, or several (each at most k), one chosen
        # per round by HorizonPolicy; buffers are sized for k
        hs = sorted(set(int(h) for h in horizons)) if horizons else [sess.k]
        assert 1 <= hs[0] and hs[-1] <= sess.k
        self.policy = HorizonPolicy(hs) if len(hs) > 1 else None   # one horizon: drafted every round
        self.horizons = hs
        dec, s, B, dev = sess.dec, sess.dec.s, sess.B, sess.device
        G, k = sess.group, sess.k
        kb, vb = sess.bits
        N0 = sess.N0
        res = sess.cache.clone()
        if prefix_store is not None:
            assert slots is not None, "the prefix store is staged through device slots"
            self.full = FileFullKV(res, slots, N0, dev, **prefix_store)
        else:
            self.full = res if slots is None else HostFullKV(res, slots, dev)
        # compressed caches: whole groups of the prompt + the rest in the tail
        cap = _round_up(N0 + sess.gen + 2 * k + G, max(32, G))
        self.tail_cap = G + 2 * k
        self.ckvs = []
        n_main = (N0 // G) * G
        for l in range(s.layers):
            c = L.Ckv("quant", B, s.Hkv, s.hd, cap, k_bits=kb, v_bits=vb, group=G, param_dtype="bf16", kv_dtype="bf16",
                      tail_cap=self.tail_cap, device=dev)
            if n_main:
                L.vc_compress(c, sess.cache.k[l], sess.cache.v[l], n_tokens=n_main)
            L.vc_copy_kv_rows(sess.cache.k[l], sess.cache.v[l], _i32(np.full(B, n_main), dev), c.tail_k, c.tail_v,
                              _i32(np.zeros(B), dev), _i32(np.full(B, N0 - n_main), dev), max(N0 - n_main, 1))
            self.ckvs.append(c)
        del res
        self.win = FullCache(s, B, k, dev)          # each layer's window keys/values of the verify pass
        self.n_main = np.full(B, n_main, np.int64)
        self.ctail = np.full(B, N0 - n_main, np.int64)
        self.Lb = np.full(B, N0, np.int64)
        self.tok = sess.first.clone()
        self.out = [[int(t)] for t in sess.first.cpu().numpy()]
        self.dec_ws = L.workspace(L.vc_decode_workspace_bytes(self.ckvs[0], s.Hq), dev)
        self.drafts_T = torch.empty(k, B, dtype=torch.int32, device=dev)
        self.targets = torch.empty(B * k, dtype=torch.int32, device=dev)
        self.acc = torch.empty(B, dtype=torch.int32, device=dev)
        self.nc = torch.empty(B, dtype=torch.int32, device=dev)
        self.com_flat = torch.empty(B * k, dtype=torch.int32, device=dev)
        self.rounds = 0
        self.accept_lens = []
        self.ev = {n: torch.cuda.Event(enable_timing=True) for n in ("start", "drafted", "verified", "end")}
        self.phase_ms = {"draft": 0.0, "verify": 0.0, "update": 0.0}
        # the draft loop's inputs, refreshed every round
        for c in self.ckvs:
            c.n_main, c.tail_len = cap, self.tail_cap
        i32 = dict(dtype=torch.int32, device=dev)
        self.g_tok = torch.empty(B, **i32)
        self.g_pos, self.g_trow, self.g_tlen = (torch.empty(k, B, **i32) for _ in range(3))
        self.g_main = torch.empty(B, **i32)
        self.graphs = {}
        if graph:
            self._set_draft_inputs()
            for h in hs:
                self.graphs[h] = torch.cuda.CUDAGraph()
                with torch.cuda.graph(self.graphs[h]):
                    self._draft_steps(h)

    def _set_draft_inputs(self):
        k = self.sess.k
        i_col = np.arange(k)[:, None]
        cpu = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
        self.g_tok.copy_(self.tok)
        self.g_pos.copy_(cpu(self.Lb[None, :] + i_col))
        self.g_trow.copy_(cpu(self.ctail[None, :] + i_col))
        self.g_tlen.copy_(cpu(self.ctail[None, :] + i_col + 1))
        self.g_main.copy_(cpu(self.n_main))

    def _draft_steps(self, kr):
        dec, B = self.sess.dec, self.sess.B
        cur = self.g_tok
        for i in range(kr):
            attend = attend_draft(dec, self.ckvs, B, self.g_pos[i], self.g_trow[i], self.g_main, self.g_tlen[i],
                                  self.dec_ws)
            lg = dec.forward(cur, B, 1, attend)
            L.vc_argmax_rows(lg, self.drafts_T[i])
            cur = self.drafts_T[i]

    def done(self):
        return min(len(o) for o in self.out) >= self.sess.gen

    def round(self, timed=False):
        """One draft-and-verify round of every sequence; returns the tokens committed."""
        sess, dec, s = self.sess, self.sess.dec, self.sess.dec.s
        B, G, dev = sess.B, sess.group, sess.device
        k = self.policy.choose() if self.policy else self.horizons[-1]    # this round's horizon
        t_round = time.perf_counter()
        maxL = int(self.Lb.max())
        if timed:
            self.ev["start"].record()
        # the draft steps' inputs first: their small host-to-device copies must not queue
        # behind the staging copies
        self._set_draft_inputs()
        # ---- staging of the first slots' layers starts now, overlapping the drafts
        self.full.begin(maxL, int(self.Lb.min()), maxL + k)
        # ---- k draft steps on the compressed cache
        if self.graphs:
            self.graphs[k].replay()
        else:
            self._draft_steps(k)
        if timed:
            self.ev["drafted"].record()
        drafts = self.drafts_T.t().contiguous()                    # [B, k]
        # ---- verify the window [last committed, d_1 .. d_{k-1}] against the full cache
        window = torch.cat([self.tok.view(B, 1), drafts[:, : k - 1]], 1).contiguous().view(-1)
        vpos = _i32(self.Lb[:, None] + np.arange(k)[None, :], dev).view(-1)
        row0 = _i32(self.Lb, dev)
        zeros, kk = _i32(np.zeros(B), dev), _i32(np.full(B, k), dev)

        def keep_window(l, K, V):
            L.vc_copy_kv_rows(K, V, row0, self.win.k[l], self.win.v[l], zeros, kk, k)

        attend = attend_full(dec, self.full, B, k, vpos, row0, maxL, row0, sess.split, sess.ver_ws, after=keep_window)
        lg = dec.forward(window, B, k, attend)
        targets = self.targets[: B * k]
        com = self.com_flat[: B * k].view(B, k)
        L.vc_argmax_rows(lg, targets)
        L.vc_accept(drafts[:, :k].contiguous(), targets.view(B, k), self.acc, self.nc, com)
        if timed:
            self.ev["verified"].record()
        acc, nc, com = self.acc.cpu().numpy(), self.nc.cpu().numpy(), com.cpu().numpy()  # the round's one sync
        # a sequence that already has its tokens stays where it is (its rows are still
        # computed, within the cache, and discarded)
        active = np.array([len(o) < sess.gen for o in self.out])
        nc = np.where(active, nc, 0)
        adv = np.where(active, np.minimum(acc + 1, k), 0)
        # ---- compressed tails take the verified rows; whole groups are quantized
        dst0, cnt = _i32(self.ctail, dev), _i32(adv, dev)
        for l in range(s.layers):
            c = self.ckvs[l]
            L.vc_copy_kv_rows(self.win.k[l], self.win.v[l], zeros, c.tail_k, c.tail_v, dst0, cnt, k)
        new_tail = self.ctail + adv
        full = (new_tail // G) * G
        if full.any():
            rest = new_tail - full
            for b in np.nonzero(full)[0]:
                for l in range(s.layers):
                    c = self.ckvs[l]
                    L.vc_compress(c.batch_view(b), c.tail_k[b:b + 1], c.tail_v[b:b + 1], n_tokens=int(full[b]),
                                  dst_begin=int(self.n_main[b]))
            s0, rc = _i32(full, dev), _i32(rest, dev)
            for l in range(s.layers):
                c = self.ckvs[l]
                L.vc_copy_kv_rows(c.tail_k, c.tail_v, s0, c.tail_k, c.tail_v, zeros, rc, G)
            self.n_main = self.n_main + full
            new_tail = rest
        self.ctail = new_tail
        self.Lb = self.Lb + adv
        for b in range(B):
            self.out[b].extend(int(t) for t in com[b, : nc[b]])
        self.tok = torch.as_tensor(np.array([self.out[b][-1] for b in range(B)], np.int32), device=dev)
        if timed:
            self.ev["end"].record()
            self.ev["end"].synchronize()
            e = self.ev
            self.phase_ms["draft"] += e["start"].elapsed_time(e["drafted"])
            self.phase_ms["verify"] += e["drafted"].elapsed_time(e["verified"])
            self.phase_ms["update"] += e["verified"].elapsed_time(e["end"])
        self.rounds += 1
        self.accept_lens.extend(int(a) for a in acc[active])
        if self.policy:
            # the round's whole cost, its cache update included, is charged to its own
            # horizon: wait for the update's device work before reading the clock
            torch.cuda.current_stream().synchronize()
            self.policy.update(k, time.perf_counter() - t_round, acc[active])
        return int(nc.sum())

    def run(self, timed=False):
        while not self.done():
            self.round(timed)
        torch.cuda.synchronize()
        return np.array([o[: self.sess.gen] for o in self.out], np.int32)


class Staggered:
    """Several independent batches decoded at once, each by its own VeriCacheLoop
    (its own decoder buffers, caches and staging stream) driven by its own host thread
    on its own compute stream, so that one batch's drafting overlaps another's full-KV
    staging and verification (summary page, "What the paper found": the drafting,
    staging and verification of different batches are staggered across the GPU and
    the host link).  Each loop's HIP graph is captured when the loop is built, before
    any thread starts; the threads share nothing but the device."""

    def __init__(self, loops):
        self.loops = list(loops)
        self.streams = [torch.cuda.Stream() for _ in self.loops]

    def run(self, timed=False):
        import threading
        errors = []

        def drive(loop, stream):
            try:
                with torch.cuda.stream(stream):
                    while not loop.done():
                        loop.round(timed)
                stream.synchronize()
            except BaseException as e:  # re-raised in the calling thread
                errors.append(e)

        threads = [threading.Thread(target=drive, args=(lp, st)) for lp, st in zip(self.loops, self.streams)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        if errors:
            raise errors[0]
        torch.cuda.synchronize()
        return [np.array([o[: lp.sess.gen] for o in lp.out], np.int32) for lp in self.loops]


def random_weights(shape: ModelShape, seed_fn, std=0.02, device="cuda"):
    """bf16 weights of a random-initialised decoder; seed_fn(key, shape, std) returns
    a float32 numpy draw of N(0, std^2) for an integer key tuple.  Projections are
    stored [out_features, in_features]; wgu holds the gate rows, then the up rows."""
    s = shape
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(BF16).to(device)
    w = dict(E=t(seed_fn((0,), (s.vocab, s.d_model), std)),
             head=t(seed_fn((1,), (s.vocab, s.d_model), std)),
             nf=t(1.0 + seed_fn((2,), (s.d_model,), std)))
    w["wqkv"] = [t(seed_fn((3, l), ((s.Hq + 2 * s.Hkv) * s.hd, s.d_model), std)) for l in range(s.layers)]
    w["wo"] = [t(seed_fn((4, l), (s.d_model, s.Hq * s.hd), std)) for l in range(s.layers)]
    w["wgu"] = [t(seed_fn((5, l), (2 * s.ffn, s.d_model), std)) for l in range(s.layers)]
    w["wd"] = [t(seed_fn((6, l), (s.d_model, s.ffn), std)) for l in range(s.layers)]
    w["n1"] = [t(1.0 + seed_fn((7, l), (s.d_model,), std)) for l in range(s.layers)]
    w["n2"] = [t(1.0 + seed_fn((8, l), (s.d_model,), std)) for l in range(s.layers)]
    return w


def weights_to(w: dict, device):
    return {k: ([x.to(device) for x in v] if isinstance(v, list) else v.to(device)) for k, v in w.items()}
