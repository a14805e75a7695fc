"""Shapes of the five synthetic workloads.

The VeriCache pages (neuraltrendhub.com summary, "What the paper found" and the
abstract; pith.science record of arXiv 2605.17613, abstract) measure on real
models and datasets.  None of those are available here, so every workload is a
seeded synthetic stand-in with the shapes below.  This module holds shapes only:
no arithmetic of the method.
"""
from dataclasses import dataclass, replace, field
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # 1..5, also the seed offset
    dtype: str                 # "f32" or "bf16": KV / query / output storage type
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int                     # context tokens held in the (compressed and full) cache
    k: int                     # draft window / verify rows
    method: str = "quant"      # "quant" (KIVI-style) or "drop" (accumulated-attention top-k)
    k_bits: int = 4
    v_bits: int = 4
    group: int = 32
    scale_dtype: str = "bf16"
    keep_ratio: float = 1.0
    n_probes: int = 0
    outlier_frac: float = 0.0  # fraction of (kv-head, channel) pairs scaled by outlier_mult
    outlier_mult: float = 10.0
    vocab: int = 0             # random projection W [d, vocab] for argmax, 0 = none
    w_dtype: str = "f32"
    # end-to-end decoder (last workload only)
    layers: int = 0
    d_model: int = 0
    ffn: int = 0
    gen_tokens: int = 0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def group_size(self) -> int:
        return self.Hq // self.Hkv


# Tiny attention layer, fp32, 2-bit K per-channel / 2-bit V per-token, group 32,
# fp32 scale and zero-point, k = 8, random 64x1000 projection.
TINY = Workload(name="tiny_fp32", index=1, dtype="f32", B=1, Hq=8, Hkv=2, d=64,
                N=512, k=8, k_bits=2, v_bits=2, group=32, scale_dtype="f32",
                vocab=1000, w_dtype="f32")

# Llama-3-8B-shaped layer: B8, 32/8 heads, d128, N32768, 1% outlier channels x10,
# 4-bit K and V, group 64, draft window 32.
LLAMA8B = Workload(name="llama8b_n32k_4bit", index=2, dtype="bf16", B=8, Hq=32, Hkv=8,
                   d=128, N=32768, k=32, k_bits=4, v_bits=4, group=64,
                   scale_dtype="bf16", outlier_frac=0.01)

# Token-dropping draft: B4, 32/8 heads, d128, N131072, keep 25% by accumulated
# attention from 64 random probe queries, verify window 40.
DROP = Workload(name="drop25_n128k", index=3, dtype="bf16", B=4, Hq=32, Hkv=8, d=128,
                N=131072, k=40, method="drop", keep_ratio=0.25, n_probes=64,
                k_bits=16, v_bits=16)

# Qwen3-30B-A3B-shaped attention: B16, 32/4 heads, d128, N65536, K 4-bit / V 3-bit,
# group 32, bf16 scales, verify window 40, 128x151936 bf16 projection.
QWEN30B = Workload(name="qwen30b_n64k_k4v3", index=4, dtype="bf16", B=16, Hq=32, Hkv=4,
                   d=128, N=65536, k=40, k_bits=4, v_bits=3, group=32,
                   scale_dtype="bf16", vocab=151936, w_dtype="bf16")

# End-to-end round on a random-init 4-layer decoder.
E2E = Workload(name="decoder4l_n16k_2bit", index=5, dtype="bf16", B=4, Hq=16, Hkv=4,
               d=128, N=16384, k=32, k_bits=2, v_bits=2, group=32, scale_dtype="bf16",
               vocab=32000, w_dtype="bf16", layers=4, d_model=2048, ffn=5504,
               gen_tokens=256)

ALL = {w.index: w for w in (TINY, LLAMA8B, DROP, QWEN30B, E2E)}


def small(w: Workload, **kw) -> Workload:
    """A reduced copy of a workload for parity tests: same method, bits, group,
    dtype and head ratio, with fewer batches/heads/tokens."""
    base = dict(B=min(w.B, 2), Hkv=min(w.Hkv, 2))
    base["Hq"] = base["Hkv"] * w.group_size
    base.update(kw)
    return w.with_(**base)
