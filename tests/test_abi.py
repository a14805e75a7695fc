"""The C-ABI library: it loads without a GPU, exports every entry point declared in
include/vc.h, and rejects bad arguments on the host before anything is enqueued
(these calls never reach a kernel launch)."""
import ctypes
import os
import re

import pytest
import torch

import lossy_kv_draft_amd as L

INC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def declared():
    text = "".join(open(os.path.join(INC, f)).read() for f in sorted(os.listdir(INC)) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(vc_\w+)\s*\(", text))


def test_header_and_binding_agree():
    assert declared() == set(L.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared():
        assert hasattr(lib, name), name


def test_keep_count_and_split_tokens():
    assert L.vc_drop_keep_count(0.25, 131072) == 32768
    assert L.vc_drop_keep_count(0.25, 10) == 3
    assert L.vc_drop_keep_count(1.0, 7) == 7
    # without a device the library assumes 512 resident workgroups
    for B, H, rows in [(1, 2, 32800), (4, 4, 64), (8, 8, 32800), (16, 4, 65576), (4, 8, 131112), (8, 8, 1)]:
        c = L.vc_verify_split_tokens(B, H, rows)
        S = max(1, 512 // (B * H))                # splits per (sequence, kv-head) that fit
        assert c % 64 == 0 and c >= 64
        assert -(-rows // c) <= S                 # at most S splits
        assert c == 64 or -(-rows // (c - 64)) > S  # and the smallest such multiple of 64


def _ckv(**kw):
    a = dict(k_bits=2, v_bits=2, group=32, param_dtype="f32", kv_dtype="f32", tail_cap=4, device="cpu")
    a.update(kw)
    return L.Ckv("quant", 1, 2, 64, 512, **a)


def _bad(fn, *a, status=L._lib.VC_ERR_INVALID_ARG, **k):
    with pytest.raises(L.VcError) as e:
        fn(*a, **k)
    assert e.value.status == status, str(e.value)
    assert L.vc_last_error() != ""
    return str(e.value)


def test_decode_rejects_bad_arguments():
    q = torch.zeros(1, 8, 64)
    out = torch.zeros(1, 8, 64)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    c = _ckv()
    c.k_bits = 5
    assert "bits" in _bad(L.vc_decode_attn_compressed, c, q, out, ws=ws, stream=0)
    c = _ckv()
    c.n_main = 100  # not a multiple of the group
    _bad(L.vc_decode_attn_compressed, c, q, out, ws=ws, stream=0)
    c = _ckv()
    c.n_main = 512
    _bad(L.vc_decode_attn_compressed, c, torch.zeros(1, 7, 64), torch.zeros(1, 7, 64), ws=ws, stream=0)
    _bad(L.vc_decode_attn_compressed, c, q, out, ws=torch.zeros(8, dtype=torch.uint8), stream=0,
         status=L._lib.VC_ERR_WORKSPACE)
    c.tail_len = 5  # beyond tail_cap
    _bad(L.vc_decode_attn_compressed, c, q, out, ws=ws, stream=0)


def test_compress_rejects_misaligned_rows():
    c = _ckv()
    k = torch.zeros(1, 2, 512, 64)
    _bad(L.vc_compress, c, k, k, src_begin=16, n_tokens=32, stream=0)
    _bad(L.vc_compress, c, k, k, n_tokens=48, stream=0)
    _bad(L.vc_compress, c, k, k, dst_begin=512, n_tokens=32, stream=0)


def test_verify_accept_stage_reject_bad_arguments():
    q = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)
    kc = torch.zeros(1, 2, 100, 64, dtype=torch.bfloat16)
    out = torch.zeros_like(q)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    _bad(L.vc_verify_attn_full, q, kc, kc, 97, out, ws=ws, stream=0)          # ctx + k > rows
    _bad(L.vc_verify_attn_full, q, kc, kc, 10, out, ws=ws, split_tokens=100, stream=0)
    _bad(L.vc_verify_attn_full, q.float(), kc.float(), kc.float(), 10, out.float(), ws=ws, stream=0,
         sm_scale=-1.0)
    _bad(L.vc_verify_attn_full, torch.zeros(1, 8, 4, 96, dtype=torch.bfloat16),
         torch.zeros(1, 2, 100, 96, dtype=torch.bfloat16), torch.zeros(1, 2, 100, 96, dtype=torch.bfloat16), 10,
         torch.zeros(1, 8, 4, 96, dtype=torch.bfloat16), ws=ws, stream=0, status=L._lib.VC_ERR_UNSUPPORTED)
    d = torch.zeros(2, 2000, dtype=torch.int32)
    _bad(L.vc_accept, d, d, d[:, 0], d[:, 0], d, stream=0)                    # k > 1024
    hk = torch.zeros(1, 2, 8, 4)
    _bad(L.vc_stage_full_kv, hk, hk, torch.zeros(1, 2, 4, 4), torch.zeros(1, 2, 4, 4), 0, 8, copy_stream=0)


def test_drop_rejects_bad_arguments():
    s = torch.zeros(1, 2, 10)
    _bad(L.vc_drop_select, s, 11, torch.zeros(1, 2, 11, dtype=torch.int32), stream=0)
    _bad(L.vc_drop_select, s, 0, torch.zeros(1, 2, 1, dtype=torch.int32), stream=0)
    k = torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16)
    _bad(L.vc_drop_scores, k, torch.zeros(2, 65, 64, dtype=torch.bfloat16), torch.zeros(1, 2, 10),
         ws=torch.zeros(1 << 16, dtype=torch.uint8), stream=0)


def test_hadamard_rejects_unsupported_widths():
    x = torch.zeros(3, 96, dtype=torch.bfloat16)
    assert "d = 64, 128 or 256" in _bad(L.vc_hadamard_rows, x, stream=0, status=L._lib.VC_ERR_UNSUPPORTED)
    y = torch.zeros(0, 128)
    assert L.vc_hadamard_rows(y, stream=0).shape == (0, 128)    # no rows: nothing launched
    z = torch.zeros(4 * 128 + 2, dtype=torch.bfloat16)[2:].view(4, 128)   # 4-byte offset
    assert "aligned" in _bad(L.vc_hadamard_rows, z, stream=0)


def test_file_stager_rejects_bad_arguments():
    """Checked before any HIP call: bad sizes, a NULL stager, a bad descriptor."""
    h = ctypes.c_void_p()
    lib = L._lib.lib
    for args in [(0, 1 << 20, 4, 0.0), (4, 1 << 20, 2, 0.0), (2, 100, 4, 0.0), (2, 1 << 20, 4, -1.0)]:
        assert lib.vc_file_stager_create(*args, ctypes.byref(h)) == L._lib.VC_ERR_INVALID_ARG
        assert h.value is None and L.vc_last_error() != ""
    t = ctypes.c_int64()
    assert lib.vc_stage_full_kv_file(None, 3, 0, 0, 1, 1, 1, 1, 64, 2, 10, 10, 0, 10, None, None,
                                     ctypes.byref(t)) == L._lib.VC_ERR_INVALID_ARG
    assert lib.vc_file_stager_wait(None, 1) == L._lib.VC_ERR_INVALID_ARG
    assert lib.vc_file_stager_destroy(None) == L._lib.VC_OK


def test_split_planes_rejects_bad_arguments():
    full = _ckv(k_bits=4, v_bits=4)
    anchor = _ckv(k_bits=2, v_bits=2)
    r = torch.zeros(1, 2, 512, 4, dtype=torch.int32)
    assert "exceed" in _bad(L.vc_split_planes, anchor, full, r, r, 64, stream=0)       # anchor wider than full
    _bad(L.vc_split_planes, full, anchor, r, r, 48, stream=0)                          # not a whole group
    _bad(L.vc_split_planes, full, anchor, None, r, 64, stream=0)                       # residual missing
    _bad(L.vc_split_planes, full, full, r, r, 64, stream=0)                            # shares arrays
    wide = _ckv(k_bits=16, v_bits=4)
    _bad(L.vc_split_planes, wide, anchor, r, r, 64, stream=0, status=L._lib.VC_ERR_UNSUPPORTED)
    other = _ckv(k_bits=2, v_bits=2, group=64)
    _bad(L.vc_join_planes, other, r, r, full, 64, stream=0)                            # group differs


def test_rmsnorm_rejects_bad_arguments():
    bf = torch.bfloat16
    _bad(L.vc_rmsnorm, torch.zeros(4, 250, dtype=bf), torch.zeros(250, dtype=bf), torch.zeros(4, 250, dtype=bf),
         stream=0)                                                                     # d not a multiple of 8
    _bad(L.vc_rmsnorm, torch.zeros(4, 256, dtype=bf), torch.zeros(256, dtype=bf), torch.zeros(4, 256, dtype=bf),
         eps=0.0, stream=0)


def test_gemm_swiglu_rejects_bad_arguments():
    bf = torch.bfloat16
    x = torch.zeros(4, 256, dtype=bf)
    act = torch.zeros(4, 60, dtype=bf)
    _bad(L.vc_gemm_bf16_swiglu, x, torch.zeros(120, 256, dtype=bf), act, stream=0)       # F = 60 not a multiple of 8
    _bad(L.vc_gemm_bf16_swiglu, torch.zeros(4, 250, dtype=bf), torch.zeros(128, 250, dtype=bf),
         torch.zeros(4, 64, dtype=bf), stream=0)                                         # K not a multiple of 32


def test_gemm_rope_rejects_bad_arguments():
    bf = torch.bfloat16
    x = torch.zeros(4, 256, dtype=bf)
    w = torch.zeros(24 * 8, 256, dtype=bf)
    q = torch.zeros(4, 16, 1, 8, dtype=bf)
    kv = torch.zeros(4, 4, 10, 8, dtype=bf)
    i32 = torch.zeros(4, dtype=torch.int32)
    _bad(L.vc_gemm_bf16_rope, x, w, 4, 1, 16, 4, 8, i32, q, kv, kv, i32, stream=0)          # hd not a multiple of 16
    _bad(L.vc_gemm_bf16_rope, x, w, 4, 1, 16, 4, 16, i32, q, kv, kv, i32, theta=1.0, stream=0)


def _layout_bytes(method, B, Hkv, d, cap, kb, vb, G, pdt, kvdt, tail_cap):
    """The array sizes the header's layouts give, written out per array."""
    pb = {"f32": 4, "bf16": 2}[pdt]
    eb = {"f32": 4, "bf16": 2}[kvdt]
    z = dict.fromkeys(L.CKV_ARRAYS, 0)
    if method == "quant":
        z["k_codes"] = B * Hkv * cap * (d * kb // 32) * 4
        z["v_codes"] = B * Hkv * cap * (d * vb // 32) * 4
        z["k_scale"] = z["k_zero"] = B * Hkv * (cap // G) * d * pb
        z["v_scale"] = z["v_zero"] = B * Hkv * cap * (d // G) * pb
    else:
        z["k_kept"] = z["v_kept"] = B * Hkv * cap * d * eb
        z["kept_idx"] = B * Hkv * cap * 4
    z["tail_k"] = z["tail_v"] = B * Hkv * tail_cap * d * eb
    return z


@pytest.mark.parametrize("bits", [2, 3, 4, 8, 16])
@pytest.mark.parametrize("pdt", ["f32", "bf16"])
def test_ckv_sizes_match_the_layouts(bits, pdt):
    for G, d, cap, tail in [(32, 128, 1024, 70), (64, 128, 32768, 0), (16, 64, 48, 5), (128, 128, 256, 1)]:
        kb, vb = bits, {2: 3, 3: 2, 4: 8, 8: 4, 16: 2}[bits]
        c = L.Ckv("quant", 3, 2, d, cap, k_bits=kb, v_bits=vb, group=G, param_dtype=pdt, kv_dtype="bf16",
                  tail_cap=tail, device="cpu")
        want = _layout_bytes("quant", 3, 2, d, cap, kb, vb, G, pdt, "bf16", tail)
        assert L.vc_ckv_sizes(c) == want
        for name in L.CKV_ARRAYS:  # the binding allocates exactly those bytes
            t = getattr(c, name)
            assert (0 if t is None else t.numel() * t.element_size()) == want[name], name


@pytest.mark.parametrize("kvdt", ["f32", "bf16"])
def test_ckv_sizes_drop(kvdt):
    c = L.Ckv("drop", 4, 8, 128, 32768, keep_ratio=0.25, kv_dtype=kvdt, tail_cap=40, device="cpu")
    want = _layout_bytes("drop", 4, 8, 128, 32768, 0, 0, 1, "f32", kvdt, 40)
    assert L.vc_ckv_sizes(c) == want
    assert c.k_codes is None and c.k_kept.shape == (4, 8, 32768, 128) and c.kept_idx.dtype == torch.int32


def test_ckv_sizes_reject_invalid_descriptors():
    c = _ckv()
    for field, value in [("k_bits", 5), ("group", 48), ("capacity", 500), ("B", 0), ("tail_cap", -1),
                         ("param_dtype", "f16")]:
        bad = _ckv()
        setattr(bad, field, value)
        if field == "param_dtype":
            st = bad.struct()
            st.param_dtype = 7
            out = (ctypes.c_size_t * len(L.CKV_ARRAYS))()
            assert L._lib.lib.vc_ckv_sizes(ctypes.byref(st), out) == L._lib.VC_ERR_INVALID_ARG
            continue
        _bad(L.vc_ckv_sizes, bad)
    assert L.vc_ckv_sizes(c)["k_codes"] == 2 * 512 * 4 * 4


def test_workspace_size_query_equals_the_per_call_sizes():
    c = _ckv(kv_dtype="bf16", param_dtype="bf16")
    assert L.vc_workspace_size(L.VC_OP_DECODE, ckv=c, Hq=8) == L.vc_decode_workspace_bytes(c, 8) > 0
    for args in [(8, 32, 8, 128, 32, 32768, 0), (16, 32, 4, 128, 40, 65536, 0), (1, 8, 2, 64, 8, 512, 256)]:
        B, Hq, Hkv, d, k, n, sp = args
        got = L.vc_workspace_size(L.VC_OP_VERIFY, B=B, Hq=Hq, Hkv=Hkv, d=d, k=k, max_len=n, split_tokens=sp)
        assert got == L.vc_verify_workspace_bytes(B, Hq, Hkv, d, k, n, sp) > 0
    assert L.vc_workspace_size(L.VC_OP_LOGITS, rows=640, vocab=151936) == L.vc_logits_workspace_bytes(640, 151936)
    dr = L.Ckv("drop", 2, 2, 128, 1024, keep_ratio=0.25, tail_cap=0, device="cpu")
    assert (L.vc_workspace_size(L.VC_OP_COMPRESS, ckv=dr, n_tokens=4096, n_probes=64)
            == L.vc_compress_workspace_bytes(dr, 4096, 64) > 0)
    assert L.vc_workspace_size(99, rows=1, vocab=1) == 0
    assert L.vc_workspace_size(L.VC_OP_DECODE) == 0           # no descriptor

