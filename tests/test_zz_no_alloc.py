"""vc_decode_attn_compressed_noalloc (no workspace argument; the split partials in the
library's own device array) against vc_decode_attn_compressed through the C ABI: two
calls in a row, the second on a smaller cache, each equal to the existing entry
point's output and log-sum-exp bit for bit (same kernels, same splits); the array's
size limit is enforced before anything is enqueued."""
import numpy as np
import pytest
import torch

import lossy_kv_draft_amd as L
from workloads import configs as C
from gpu_util import T, inputs, oracle_compress, upload_quant, say

pytestmark = pytest.mark.gpu


def _cache(w, tail):
    K, V, Q, Kw, Vw = inputs(w)
    comp = oracle_compress(w, K, V)
    ckv = L.Ckv("quant", w.B, w.Hkv, w.d, w.N, k_bits=w.k_bits, v_bits=w.v_bits, group=w.group,
                param_dtype=w.scale_dtype, kv_dtype=w.dtype, tail_cap=max(tail, 1))
    upload_quant(ckv, comp, w.N)
    ckv.n_main, ckv.tail_len = w.N, tail
    if tail:
        ckv.tail_k[:, :, :tail] = T(Kw[:, :, :tail], torch.bfloat16)
        ckv.tail_v[:, :, :tail] = T(Vw[:, :, :tail], torch.bfloat16)
    return ckv, T(Q[:, :, max(tail - 1, 0)], torch.bfloat16)


def _both(ckv, q, main_lens=None):
    B, Hq, d = q.shape
    outs = []
    for fn in ("noalloc", "ws"):
        o = torch.full((B, Hq, d), float("nan"), device="cuda", dtype=torch.bfloat16)
        lse = torch.full((B, Hq), float("nan"), device="cuda")
        if fn == "noalloc":
            L.vc_decode_attn_compressed_noalloc(ckv, q, o, lse=lse, main_lens=main_lens)
        else:
            L.vc_decode_attn_compressed(ckv, q, o, lse=lse, main_lens=main_lens)
        outs.append((o, lse))
    torch.cuda.synchronize()
    return outs


def test_noalloc_decode_equals_the_workspace_entry_point_on_two_calls():
    big = C.small(C.LLAMA8B, N=64 * 37)                     # 4/4-bit G64, matrix-core kernel
    small = C.small(C.E2E, B=1, Hkv=2, N=32 * 9)            # 2/2-bit G32, fewer rows and sequences
    for w, tail in ((big, 5), (small, 3)):
        say(f"[noalloc] {w.name} B{w.B} N{w.N} tail {tail}")
        ckv, q = _cache(w, tail)
        (o1, l1), (o2, l2) = _both(ckv, q)
        assert not torch.isnan(o1.float()).any() and not torch.isnan(l1).any()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_decode_generic_and_ragged():
    """The generic kernel (float32 parameters, a capacity not a multiple of 32) and
    per-sequence lengths, after a larger call has left its partials in the array."""
    w = C.small(C.E2E, N=16 * 13, k_bits=3, v_bits=2, group=16, scale_dtype="f32")
    ckv, q = _cache(w, 4)
    lens = torch.tensor([16 * 13, 16 * 5], dtype=torch.int32, device="cuda")
    (o1, l1), (o2, l2) = _both(ckv, q, main_lens=lens)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_rejects_partials_beyond_the_array():
    """B 128 x Hkv 8 x 16 q-heads per kv-head needs more than the 8 MiB array (one
    split per (sequence, kv-head): 8 MiB of outputs plus their maxima and sums):
    rejected with VC_ERR_WORKSPACE, nothing written."""
    ckv = L.Ckv("quant", 128, 8, 128, 32, k_bits=4, v_bits=4, group=32, tail_cap=1)
    ckv.n_main = 32
    q = torch.zeros(128, 128, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full((128, 128, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.VcError) as e:
        L.vc_decode_attn_compressed_noalloc(ckv, q, out)
    assert e.value.status == L._lib.VC_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
