"""Plain CPU oracle of the VeriCache draft-and-verify hot path.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import this package; the library and its Python binding never
do, and the two share no code (only the seeded input generators in ``workloads``
serve both sides).

What it computes, and where the pages say so:

* Drafting with a compressed KV cache and verifying against the full KV cache so
  that greedy output equals full-KV greedy decoding -- "VeriCache: Turning Lossy
  KV Cache into Lossless LLM Inference" (neuraltrendhub.com summary), "What the
  paper found" and "Original abstract".
* Compressors: KIVI-style asymmetric low-bit quantization (podparley.com episode
  page, source 4, "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache")
  and token dropping by accumulated attention (same list, source 3, "H2O:
  Heavy-Hitter Oracle").
* Greedy verification by longest matching prefix (same list, source 2, "Fast
  Inference from Transformers via Speculative Decoding").

Precision: attention, scores and logits in float64.  Quantization decisions (the
integer codes) are taken in IEEE float32, the precision the kernels take them in,
so that codes can be compared bit for bit.

Parity status of each function is stated in its module header.
"""
from . import quant, attention, drop, accept, logits, rotate, split  # noqa: F401
