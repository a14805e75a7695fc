"""ctypes declarations of include/vc.h and thin wrappers taking torch tensors."""
import atexit
import copy
import ctypes
import os
import sys
import weakref

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvc.so")

VC_OK, VC_ERR_INVALID_ARG, VC_ERR_UNSUPPORTED, VC_ERR_WORKSPACE, VC_ERR_HIP, VC_ERR_IO = range(6)
VC_F32, VC_BF16 = 0, 1
VC_QUANT_KIVI, VC_DROP_TOPK = 1, 2

_STATUS = {1: "VC_ERR_INVALID_ARG", 2: "VC_ERR_UNSUPPORTED", 3: "VC_ERR_WORKSPACE", 4: "VC_ERR_HIP", 5: "VC_ERR_IO"}


class VcError(RuntimeError):
    def __init__(self, status, fn, msg):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python lossy_kv_draft_amd/build.py)")
lib = ctypes.CDLL(LIB_PATH)

c_i32, c_i64, c_f32, c_sz, c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class vc_ckv(ctypes.Structure):
    _fields_ = [("method", c_i32), ("k_bits", c_i32), ("v_bits", c_i32), ("group", c_i32),
                ("param_dtype", c_i32), ("kv_dtype", c_i32), ("keep_ratio", c_f32),
                ("B", c_i32), ("Hkv", c_i32), ("d", c_i32), ("capacity", c_i64), ("n_main", c_i64),
                ("k_codes", c_p), ("v_codes", c_p), ("k_scale", c_p), ("k_zero", c_p),
                ("v_scale", c_p), ("v_zero", c_p), ("k_kept", c_p), ("v_kept", c_p),
                ("kept_idx", c_p), ("tail_k", c_p), ("tail_v", c_p),
                ("tail_cap", c_i64), ("tail_len", c_i64), ("flags", c_i32)]


VC_CKV_DECODE_F32 = 1
# vc_ckv_array: order of the sizes vc_ckv_sizes reports
CKV_ARRAYS = ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero", "k_kept", "v_kept", "kept_idx",
              "tail_k", "tail_v")
VC_OP_COMPRESS, VC_OP_DECODE, VC_OP_VERIFY, VC_OP_LOGITS = 1, 2, 3, 4


class vc_ws_query(ctypes.Structure):
    _fields_ = [("ckv", ctypes.POINTER(vc_ckv)), ("n_tokens", c_i64), ("n_probes", c_i32), ("Hq", c_i32),
                ("B", c_i32), ("Hkv", c_i32), ("d", c_i32), ("k", c_i32), ("max_len", c_i64),
                ("split_tokens", c_i32), ("rows", c_i64), ("vocab", c_i32)]


_P = ctypes.POINTER(vc_ckv)
# name -> (restype, argtypes); every symbol declared in include/vc.h
_DECLS = {
    "vc_ckv_sizes": (c_i32, [_P, ctypes.POINTER(c_sz)]),
    "vc_workspace_size": (c_sz, [c_i32, ctypes.POINTER(vc_ws_query)]),
    "vc_compress": (c_i32, [_P, c_p, c_p, c_i64, c_i64, c_i64, c_i64, c_p, c_i32, c_f32, c_p, c_sz, c_p]),
    "vc_compress_workspace_bytes": (c_sz, [_P, c_i64, c_i32]),
    "vc_drop_keep_count": (c_i64, [c_f32, c_i64]),
    "vc_drop_scores": (c_i32, [c_p, c_i32, c_p, c_i32, c_i32, c_i64, c_i32, c_i32, c_f32, c_p, c_p, c_sz, c_p]),
    "vc_drop_scores_workspace_bytes": (c_sz, [c_i32, c_i32, c_i64, c_i32]),
    "vc_drop_select": (c_i32, [c_p, c_i32, c_i32, c_i64, c_i64, c_p, c_p, c_sz, c_p]),
    "vc_drop_select_workspace_bytes": (c_sz, [c_i32, c_i32, c_i64]),
    "vc_gather_rows": (c_i32, [c_p, c_i32, c_i32, c_i32, c_i64, c_i32, c_p, c_i64, c_p, c_i64, c_p]),
    "vc_decode_attn_compressed": (c_i32, [_P, c_p, c_i32, c_f32, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "vc_decode_workspace_bytes": (c_sz, [_P, c_i32]),
    "vc_decode_attn_compressed_noalloc": (c_i32, [_P, c_p, c_i32, c_f32, c_p, c_p, c_p, c_p, c_p]),
    "vc_verify_attn_full": (c_i32, [c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, c_i64, c_p,
                                    c_i32, c_f32, c_p, c_p, c_p, c_sz, c_p]),
    "vc_verify_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, c_i32]),
    "vc_verify_split_tokens": (c_i32, [c_i32, c_i32, c_i64]),
    "vc_head_mean": (c_i32, [c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, c_i64, c_i64, c_p, c_p]),
    "vc_logits_argmax": (c_i32, [c_p, c_i32, c_i64, c_i32, c_p, c_i32, c_i32, c_p, c_p, c_sz, c_p]),
    "vc_logits_workspace_bytes": (c_sz, [c_i64, c_i32]),
    "vc_accept": (c_i32, [c_p, c_p, c_i32, c_i32, c_p, c_p, c_p, c_p]),
    "vc_hadamard_rows": (c_i32, [c_p, c_i32, c_i64, c_i32, c_p, c_p]),
    "vc_stage_full_kv": (c_i32, [c_p, c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i64, c_i64, c_i64, c_i64,
                                 c_p, c_p]),
    "vc_stage_full_kv_d2h": (c_i32, [c_p, c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i64, c_i64, c_i64, c_i64,
                                     c_p, c_p]),
    "vc_split_planes": (c_i32, [_P, _P, c_p, c_p, c_i64, c_p]),
    "vc_join_planes": (c_i32, [_P, c_p, c_p, _P, c_i64, c_p]),
    "vc_file_stager_create": (c_i32, [c_i32, c_sz, c_i32, ctypes.c_double, ctypes.POINTER(c_p)]),
    "vc_file_stager_destroy": (c_i32, [c_p]),
    "vc_stage_full_kv_file": (c_i32, [c_p, c_i32, c_i64, c_i64, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i64, c_i64,
                                      c_i64, c_i64, c_p, c_p, ctypes.POINTER(c_i64)]),
    "vc_file_stager_wait": (c_i32, [c_p, c_i64]),
    "vc_last_error": (ctypes.c_char_p, []),
    # vc_model.h
    "vc_gemm_bf16": (c_i32, [c_p, c_i64, c_p, c_i64, c_i64, c_i32, c_i32, c_p, c_i64, c_i32, c_p, c_p]),
    "vc_gemm_bf16_wide": (c_i32, [c_p, c_i64, c_p, c_i64, c_i64, c_i32, c_i32, c_p, c_i64, c_i32, c_p, c_p]),
    "vc_gemm_bf16_swiglu": (c_i32, [c_p, c_i64, c_p, c_i64, c_i64, c_i32, c_i32, c_p, c_i64, c_p]),
    "vc_gemm_bf16_rope": (c_i32, [c_p, c_i64, c_p, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_p, c_p, c_p,
                                  c_p, c_i64, c_p, c_p]),
    "vc_rmsnorm": (c_i32, [c_p, c_p, c_i64, c_i32, c_f32, c_p, c_p]),
    "vc_rope_qkv": (c_i32, [c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_p, c_p, c_p, c_p, c_i64, c_p, c_p]),
    "vc_swiglu": (c_i32, [c_p, c_i64, c_i32, c_p, c_p]),
    "vc_embed": (c_i32, [c_p, c_i32, c_i32, c_p, c_i64, c_p, c_p]),
    "vc_heads_to_rows": (c_i32, [c_p, c_i32, c_i32, c_i32, c_i32, c_p, c_p]),
    "vc_argmax_rows": (c_i32, [c_p, c_i64, c_i32, c_p, c_p]),
    "vc_copy_kv_rows": (c_i32, [c_p, c_p, c_i64, c_p, c_p, c_p, c_i64, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                c_p]),
}
EXPORTS = tuple(_DECLS)
for _n, (_r, _a) in _DECLS.items():
    _f = getattr(lib, _n)
    _f.restype, _f.argtypes = _r, _a


def vc_last_error() -> str:
    return lib.vc_last_error().decode()


def _check(status, fn):
    if status != VC_OK:
        raise VcError(status, fn, vc_last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    return s.cuda_stream if hasattr(s, "cuda_stream") else s


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return VC_F32
    if t == torch.bfloat16:
        return VC_BF16
    raise TypeError(f"unsupported dtype {t}")


_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Zero-filled device workspace (the library restores the parts that must be zero)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


class Ckv:
    """Device storage of one layer's compressed KV cache plus its vc_ckv descriptor.

    method "quant": packed codes and group parameters; method "drop": kept rows and
    their source positions.  Both carry a full-precision tail of tail_cap rows."""

    def __init__(self, method, B, Hkv, d, capacity, *, k_bits=4, v_bits=4, group=32, param_dtype="bf16",
                 kv_dtype="bf16", keep_ratio=1.0, tail_cap=0, flags=0, device="cuda"):
        self.method = {"quant": VC_QUANT_KIVI, "drop": VC_DROP_TOPK}[method]
        self.B, self.Hkv, self.d, self.capacity = B, Hkv, d, capacity
        self.k_bits, self.v_bits, self.group = k_bits, v_bits, group
        self.param_dtype, self.kv_dtype, self.keep_ratio = param_dtype, kv_dtype, keep_ratio
        self.tail_cap = tail_cap
        self.flags = flags
        self.n_main = 0
        self.tail_len = 0
        for name in CKV_ARRAYS:
            setattr(self, name, None)
        # byte sizes from the library (vc_ckv_sizes); the shapes below are the views
        # the header's layouts give those bytes
        sizes = vc_ckv_sizes(self)
        kvt, pt = _TORCH[kv_dtype], _TORCH[param_dtype]
        shapes = {
            "k_codes": (torch.int32, (B, Hkv, capacity, d * k_bits // 32)),
            "v_codes": (torch.int32, (B, Hkv, capacity, d * v_bits // 32)),
            "k_scale": (pt, (B, Hkv, capacity // group, d)), "k_zero": (pt, (B, Hkv, capacity // group, d)),
            "v_scale": (pt, (B, Hkv, capacity, d // group)), "v_zero": (pt, (B, Hkv, capacity, d // group)),
            "k_kept": (kvt, (B, Hkv, capacity, d)), "v_kept": (kvt, (B, Hkv, capacity, d)),
            "kept_idx": (torch.int32, (B, Hkv, capacity)),
            "tail_k": (kvt, (B, Hkv, tail_cap, d)), "tail_v": (kvt, (B, Hkv, tail_cap, d)),
        }
        for name in CKV_ARRAYS:
            nbytes = sizes[name]
            if nbytes:
                dt, shape = shapes[name]
                setattr(self, name, torch.zeros(nbytes, dtype=torch.uint8, device=device).view(dt).view(shape))

    def struct(self) -> vc_ckv:
        return vc_ckv(self.method, self.k_bits, self.v_bits, self.group,
                      VC_F32 if self.param_dtype == "f32" else VC_BF16,
                      VC_F32 if self.kv_dtype == "f32" else VC_BF16, self.keep_ratio,
                      self.B, self.Hkv, self.d, self.capacity, self.n_main,
                      _ptr(self.k_codes), _ptr(self.v_codes), _ptr(self.k_scale), _ptr(self.k_zero),
                      _ptr(self.v_scale), _ptr(self.v_zero), _ptr(self.k_kept), _ptr(self.v_kept),
                      _ptr(self.kept_idx), _ptr(self.tail_k), _ptr(self.tail_v), self.tail_cap, self.tail_len,
                      self.flags)

    def batch_view(self, b: int) -> "Ckv":
        """Descriptor of sequence b alone (B = 1) over the same device storage."""
        v = copy.copy(self)
        v.B = 1
        for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero", "k_kept", "v_kept", "kept_idx",
                     "tail_k", "tail_v"):
            t = getattr(self, name)
            setattr(v, name, None if t is None else t[b:b + 1])
        return v

    def stored_bytes(self, n_main=None) -> int:
        """Bytes of the compressed rows [0, n_main) over all sequences and heads."""
        n = self.n_main if n_main is None else n_main
        bh = self.B * self.Hkv
        if self.method == VC_QUANT_KIVI:
            pb = 4 if self.param_dtype == "f32" else 2
            codes = bh * n * self.d * (self.k_bits + self.v_bits) // 8
            params = bh * (n // self.group) * self.d * 2 * pb + bh * n * (self.d // self.group) * 2 * pb
            return codes + params
        eb = 4 if self.kv_dtype == "f32" else 2
        return bh * n * self.d * 2 * eb


def vc_ckv_sizes(ckv: "Ckv") -> dict:
    """Byte size of every array of the descriptor (vc_ckv_sizes), by array name."""
    out = (c_sz * len(CKV_ARRAYS))()
    _check(lib.vc_ckv_sizes(ctypes.byref(ckv.struct()), out), "vc_ckv_sizes")
    return dict(zip(CKV_ARRAYS, (int(x) for x in out)))


def vc_workspace_size(op: int, *, ckv=None, n_tokens=0, n_probes=0, Hq=0, B=0, Hkv=0, d=0, k=0, max_len=0,
                      split_tokens=0, rows=0, vocab=0) -> int:
    c = ckv.struct() if ckv is not None else None
    q = vc_ws_query(ctypes.pointer(c) if c is not None else None, n_tokens, n_probes, Hq, B, Hkv, d, k, max_len,
                    split_tokens, rows, vocab)
    return lib.vc_workspace_size(op, ctypes.byref(q))


def vc_compress_workspace_bytes(ckv: Ckv, n_tokens: int, n_probes: int) -> int:
    return lib.vc_compress_workspace_bytes(ctypes.byref(ckv.struct()), n_tokens, n_probes)


def vc_compress(ckv: Ckv, k_src, v_src, *, src_begin=0, n_tokens=None, dst_begin=0, probes=None,
                sm_scale=None, ws=None, stream=None):
    src_rows = k_src.shape[2]
    n = src_rows - src_begin if n_tokens is None else n_tokens
    P = 0 if probes is None else probes.shape[1]
    scale = (ckv.d ** -0.5) if sm_scale is None else sm_scale
    c = ckv.struct()
    if ws is None:
        ws = workspace(lib.vc_compress_workspace_bytes(ctypes.byref(c), n, P), k_src.device)
    _check(lib.vc_compress(ctypes.byref(c), _ptr(k_src), _ptr(v_src), src_rows, src_begin, n, dst_begin,
                           _ptr(probes), P, scale, _ptr(ws), ws.numel(), _stream(stream)), "vc_compress")


def vc_drop_keep_count(keep_ratio: float, N: int) -> int:
    return lib.vc_drop_keep_count(keep_ratio, N)


def vc_drop_scores_workspace_bytes(B, Hkv, N, n_probes) -> int:
    return lib.vc_drop_scores_workspace_bytes(B, Hkv, N, n_probes)


def vc_drop_scores(k, probes, scores, *, sm_scale=None, ws=None, stream=None):
    B, Hkv, N, d = k.shape
    P = probes.shape[1]
    if ws is None:
        ws = workspace(lib.vc_drop_scores_workspace_bytes(B, Hkv, N, P), k.device)
    _check(lib.vc_drop_scores(_ptr(k), _dt(k.dtype), _ptr(probes), B, Hkv, N, d, P,
                              d ** -0.5 if sm_scale is None else sm_scale, _ptr(scores), _ptr(ws), ws.numel(),
                              _stream(stream)), "vc_drop_scores")


def vc_drop_select(scores, n_keep, kept_idx, *, ws=None, stream=None):
    B, Hkv, N = scores.shape
    if ws is None:
        ws = workspace(lib.vc_drop_select_workspace_bytes(B, Hkv, N), scores.device)
    _check(lib.vc_drop_select(_ptr(scores), B, Hkv, N, n_keep, _ptr(kept_idx), _ptr(ws), ws.numel(),
                              _stream(stream)), "vc_drop_select")


def vc_gather_rows(src, idx, n, dst, *, stream=None):
    B, Hkv, src_rows, d = src.shape
    _check(lib.vc_gather_rows(_ptr(src), _dt(src.dtype), B, Hkv, src_rows, d, _ptr(idx), n, _ptr(dst),
                              dst.shape[2], _stream(stream)), "vc_gather_rows")


def vc_decode_workspace_bytes(ckv: Ckv, Hq: int) -> int:
    return lib.vc_decode_workspace_bytes(ctypes.byref(ckv.struct()), Hq)


def vc_decode_attn_compressed(ckv: Ckv, q, out, *, lse=None, sm_scale=None, main_lens=None, tail_lens=None,
                              ws=None, stream=None):
    B, Hq, d = q.shape
    c = ckv.struct()
    if ws is None:
        ws = workspace(lib.vc_decode_workspace_bytes(ctypes.byref(c), Hq), q.device)
    _check(lib.vc_decode_attn_compressed(ctypes.byref(c), _ptr(q), Hq, d ** -0.5 if sm_scale is None else sm_scale,
                                         _ptr(main_lens), _ptr(tail_lens), _ptr(out), _ptr(lse), _ptr(ws),
                                         ws.numel(), _stream(stream)), "vc_decode_attn_compressed")


VC_DECODE_NOALLOC_SCRATCH_BYTES = 8 << 20


def vc_decode_attn_compressed_noalloc(ckv: Ckv, q, out, *, lse=None, sm_scale=None, main_lens=None, tail_lens=None,
                                      stream=None):
    """vc_decode_attn_compressed with the split partials in the library's own device
    array (no workspace argument, nothing allocated)."""
    B, Hq, d = q.shape
    _check(lib.vc_decode_attn_compressed_noalloc(ctypes.byref(ckv.struct()), _ptr(q), Hq,
                                                 d ** -0.5 if sm_scale is None else sm_scale, _ptr(main_lens),
                                                 _ptr(tail_lens), _ptr(out), _ptr(lse), _stream(stream)),
           "vc_decode_attn_compressed_noalloc")


def vc_verify_split_tokens(B: int, Hkv: int, cache_rows: int) -> int:
    return lib.vc_verify_split_tokens(B, Hkv, cache_rows)


def vc_verify_workspace_bytes(B, Hq, Hkv, d, k, max_len, split_tokens=0) -> int:
    return lib.vc_verify_workspace_bytes(B, Hq, Hkv, d, k, max_len, split_tokens)


def vc_verify_attn_full(q, k_cache, v_cache, ctx_len, out, *, lse=None, ctx_lens=None, split_tokens=0,
                        sm_scale=None, ws=None, stream=None):
    B, Hq, k, d = q.shape
    Hkv, rows = k_cache.shape[1], k_cache.shape[2]
    if ws is None:
        ws = workspace(lib.vc_verify_workspace_bytes(B, Hq, Hkv, d, k, ctx_len, split_tokens), q.device)
    _check(lib.vc_verify_attn_full(_ptr(q), _ptr(k_cache), _ptr(v_cache), _dt(q.dtype), B, Hq, Hkv, d, k, rows,
                                   ctx_len, _ptr(ctx_lens), split_tokens,
                                   d ** -0.5 if sm_scale is None else sm_scale, _ptr(out), _ptr(lse), _ptr(ws),
                                   ws.numel(), _stream(stream)), "vc_verify_attn_full")


def vc_hadamard_rows(x, out=None, *, stream=None):
    """Rows of x [..., d] (contiguous, bf16 or f32) rotated by H / sqrt(d) into out
    (default: a new tensor; out may be x).  Returns out."""
    assert x.is_contiguous()
    if out is None:
        out = torch.empty_like(x)
    assert out.is_contiguous() and out.shape == x.shape and out.dtype == x.dtype
    d = x.shape[-1]
    _check(lib.vc_hadamard_rows(_ptr(x), _dt(x.dtype), x.numel() // d if d else 0, d, _ptr(out), _stream(stream)),
           "vc_hadamard_rows")
    return out


def vc_head_mean(o, u, *, k=None, stream=None):
    """o: [B, Hq, k, d] (verify layout) or [B, Hq, d] (decode layout) -> u float32 [B*k, d]."""
    if o.dim() == 3:
        B, Hq, d = o.shape
        kk, sb, sh, si = 1, o.stride(0), o.stride(1), 0
    else:
        B, Hq, kk, d = o.shape
        sb, sh, si = o.stride(0), o.stride(1), o.stride(2)
    _check(lib.vc_head_mean(_ptr(o), _dt(o.dtype), B, Hq, kk, d, sb, sh, si, _ptr(u), _stream(stream)),
           "vc_head_mean")


def vc_logits_workspace_bytes(R, V) -> int:
    return lib.vc_logits_workspace_bytes(R, V)


def vc_logits_argmax(u, W, tokens, *, ws=None, stream=None):
    R, K = u.shape
    V = W.shape[0]
    if ws is None:
        ws = workspace(lib.vc_logits_workspace_bytes(R, V), u.device)
    _check(lib.vc_logits_argmax(_ptr(u), _dt(u.dtype), R, K, _ptr(W), _dt(W.dtype), V, _ptr(tokens), _ptr(ws),
                                ws.numel(), _stream(stream)), "vc_logits_argmax")


def vc_accept(draft, target, accept_len, n_commit, commit, *, stream=None):
    B, k = draft.shape
    _check(lib.vc_accept(_ptr(draft), _ptr(target), B, k, _ptr(accept_len), _ptr(n_commit), _ptr(commit),
                         _stream(stream)), "vc_accept")


def _ensure_event(ev, stream):
    """torch creates the HIP event behind a torch.cuda.Event on its first record;
    record it once so that a valid handle is passed to the library."""
    if ev is not None and not ev.cuda_event:
        ev.record(torch.cuda.current_stream() if stream is None else stream)


def vc_stage_full_kv(host_k, host_v, dev_k, dev_v, tok_begin, tok_end, *, copy_stream=None, done=None):
    B, Hkv, host_rows, d = host_k.shape
    _ensure_event(done, copy_stream)
    _check(lib.vc_stage_full_kv(_ptr(host_k), _ptr(host_v), _ptr(dev_k), _ptr(dev_v), B, Hkv, d,
                                host_k.element_size(), host_rows, dev_k.shape[2], tok_begin, tok_end,
                                _stream(copy_stream), None if done is None else done.cuda_event),
           "vc_stage_full_kv")


def vc_stage_full_kv_d2h(dev_k, dev_v, host_k, host_v, tok_begin, tok_end, *, copy_stream=None, done=None):
    B, Hkv, host_rows, d = host_k.shape
    _ensure_event(done, copy_stream)
    _check(lib.vc_stage_full_kv_d2h(_ptr(dev_k), _ptr(dev_v), _ptr(host_k), _ptr(host_v), B, Hkv, d,
                                    host_k.element_size(), host_rows, dev_k.shape[2], tok_begin, tok_end,
                                    _stream(copy_stream), None if done is None else done.cuda_event),
           "vc_stage_full_kv_d2h")


def split_residuals(full: "Ckv", anchor: "Ckv"):
    """Zeroed residual arrays (k_resid, v_resid) for splitting `full` into `anchor`
    (None where the widths are equal)."""
    def one(b, a):
        r = b - a
        if r <= 0:
            return None
        return torch.zeros(full.B, full.Hkv, full.capacity, full.d * r // 32, dtype=torch.int32,
                           device=full.k_codes.device)
    return one(full.k_bits, anchor.k_bits), one(full.v_bits, anchor.v_bits)


def vc_split_planes(full: "Ckv", anchor: "Ckv", k_resid, v_resid, n_tokens, *, stream=None):
    _check(lib.vc_split_planes(ctypes.byref(full.struct()), ctypes.byref(anchor.struct()), _ptr(k_resid),
                               _ptr(v_resid), n_tokens, _stream(stream)), "vc_split_planes")


def vc_join_planes(anchor: "Ckv", k_resid, v_resid, full: "Ckv", n_tokens, *, stream=None):
    _check(lib.vc_join_planes(ctypes.byref(anchor.struct()), _ptr(k_resid), _ptr(v_resid),
                              ctypes.byref(full.struct()), n_tokens, _stream(stream)), "vc_join_planes")


_LIVE_STAGERS = weakref.WeakSet()


@atexit.register
def _close_live_stagers():
    """Joins the reader threads of every stager still open before the interpreter and
    the HIP runtime shut down (a worker must not be inside a HIP call then)."""
    for st in list(_LIVE_STAGERS):
        try:
            st.close()
        except Exception:
            pass


class FileStager:
    """vc_file_stager: reader threads and pinned bounce buffers that stage full-KV rows
    from a file (the remote prefix cache stand-in) to the device.  Closed by close(),
    by the garbage collector, or at interpreter exit, whichever comes first."""

    def __init__(self, n_threads=8, chunk_bytes=16 << 20, n_buffers=16, max_bytes_per_s=0.0):
        h = c_p()
        _check(lib.vc_file_stager_create(n_threads, chunk_bytes, n_buffers, float(max_bytes_per_s),
                                         ctypes.byref(h)), "vc_file_stager_create")
        self.handle = h.value
        _LIVE_STAGERS.add(self)

    def stage(self, fd, k_offset, v_offset, dev_k, dev_v, file_rows, tok_begin, tok_end, *, copy_stream=None,
              done=None):
        """Rows [tok_begin, tok_end) of the [B, Hkv, file_rows, d] K and V stored at the two
        byte offsets of fd -> the same rows of dev_k, dev_v.  Returns the ticket."""
        B, Hkv, dev_rows, d = dev_k.shape
        assert dev_v.shape == dev_k.shape and dev_k.is_contiguous() and dev_v.is_contiguous()
        _ensure_event(done, copy_stream)
        t = c_i64()
        _check(lib.vc_stage_full_kv_file(self.handle, fd, k_offset, v_offset, _ptr(dev_k), _ptr(dev_v), B, Hkv, d,
                                         dev_k.element_size(), file_rows, dev_rows, tok_begin, tok_end,
                                         _stream(copy_stream), None if done is None else done.cuda_event,
                                         ctypes.byref(t)), "vc_stage_full_kv_file")
        return t.value

    def wait(self, ticket):
        _check(lib.vc_file_stager_wait(self.handle, ticket), "vc_file_stager_wait")

    def close(self):
        if self.handle:
            h, self.handle = self.handle, None
            _LIVE_STAGERS.discard(self)
            _check(lib.vc_file_stager_destroy(h), "vc_file_stager_destroy")

    def __del__(self, _finalizing=sys.is_finalizing):
        if _finalizing():   # the HIP runtime may already be gone: leave it to the OS
            return
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- vc_model.h

def vc_gemm_bf16(A, W, C, *, R=None, stream=None):
    """C[M, N] = A[M, K] @ W[N, K]^T (+ R); A, W bf16 2-D views with unit column stride."""
    M, K = A.shape
    N = W.shape[0]
    _check(lib.vc_gemm_bf16(_ptr(A), A.stride(0), _ptr(W), W.stride(0), M, N, K, _ptr(C), C.stride(0),
                            _dt(C.dtype), _ptr(R), _stream(stream)), "vc_gemm_bf16")


def swiglu_interleave(wgu):
    """[2F, K] gate-then-up rows -> the layout vc_gemm_bf16_swiglu reads (blocks of 8
    gate rows followed by the same 8 up rows); a copy of the weights, no arithmetic."""
    F2, K = wgu.shape
    return wgu.view(2, F2 // 16, 8, K).transpose(0, 1).reshape(F2, K).contiguous()


def vc_gemm_bf16_swiglu(A, Wi, act, *, stream=None):
    """act[M, F] = swiglu(A @ Wgu^T) with Wi = swiglu_interleave(Wgu); equal bit for bit to
    vc_gemm_bf16 into [M, 2F] followed by vc_swiglu."""
    M, K = A.shape
    F = Wi.shape[0] // 2
    _check(lib.vc_gemm_bf16_swiglu(_ptr(A), A.stride(0), _ptr(Wi), Wi.stride(0), M, F, K, _ptr(act), act.stride(0),
                                   _stream(stream)), "vc_gemm_bf16_swiglu")


def rope_interleave(wqkv, Hq, Hkv, hd):
    """[(Hq + 2 Hkv) hd, K] QKV projection -> the layout vc_gemm_bf16_rope reads (in each
    q and k head, tiles of 8 elements followed by their 8 rotation partners); a copy of
    the weights, no arithmetic."""
    K = wqkv.shape[1]
    nqk = (Hq + Hkv) * hd
    qk = wqkv[:nqk].view(Hq + Hkv, 2, hd // 16, 8, K).permute(0, 2, 1, 3, 4).reshape(nqk, K)
    return torch.cat([qk, wqkv[nqk:]]).contiguous()


def vc_gemm_bf16_rope(A, Wr, B, k, Hq, Hkv, hd, pos, q_out, k_dst, v_dst, row0, *, theta=10000.0, stream=None):
    """vc_rope_qkv(A @ Wqkv^T, ...) in one launch, Wr = rope_interleave(Wqkv, Hq, Hkv, hd)."""
    assert k_dst.shape == v_dst.shape and k_dst.is_contiguous() and v_dst.is_contiguous() and q_out.is_contiguous()
    _check(lib.vc_gemm_bf16_rope(_ptr(A), A.stride(0), _ptr(Wr), Wr.stride(0), B, k, A.shape[1], Hq, Hkv, hd, theta,
                                 _ptr(pos), _ptr(q_out), _ptr(k_dst), _ptr(v_dst), k_dst.shape[2], _ptr(row0),
                                 _stream(stream)), "vc_gemm_bf16_rope")


def vc_gemm_bf16_wide(A, W, C, *, R=None, stream=None):
    """vc_gemm_bf16 for many rows (prompt processing; not batch invariant)."""
    M, K = A.shape
    N = W.shape[0]
    _check(lib.vc_gemm_bf16_wide(_ptr(A), A.stride(0), _ptr(W), W.stride(0), M, N, K, _ptr(C), C.stride(0),
                                 _dt(C.dtype), _ptr(R), _stream(stream)), "vc_gemm_bf16_wide")


def vc_rmsnorm(x, w, y, *, eps=1e-5, stream=None):
    M, d = x.shape
    _check(lib.vc_rmsnorm(_ptr(x), _ptr(w), M, d, eps, _ptr(y), _stream(stream)), "vc_rmsnorm")


def vc_rope_qkv(qkv, B, k, Hq, Hkv, hd, pos, q_out, k_dst, v_dst, row0, *, theta=10000.0, stream=None):
    _check(lib.vc_rope_qkv(_ptr(qkv), B, k, Hq, Hkv, hd, theta, _ptr(pos), _ptr(q_out), _ptr(k_dst), _ptr(v_dst),
                           k_dst.shape[2], _ptr(row0), _stream(stream)), "vc_rope_qkv")


def vc_swiglu(gu, out, *, stream=None):
    M, F2 = gu.shape
    _check(lib.vc_swiglu(_ptr(gu), M, F2 // 2, _ptr(out), _stream(stream)), "vc_swiglu")


def vc_embed(E, tokens, x, *, stream=None):
    V, d = E.shape
    _check(lib.vc_embed(_ptr(E), V, d, _ptr(tokens), tokens.numel(), _ptr(x), _stream(stream)), "vc_embed")


def vc_heads_to_rows(o, out, *, stream=None):
    B, H, k, hd = o.shape
    _check(lib.vc_heads_to_rows(_ptr(o), B, H, k, hd, _ptr(out), _stream(stream)), "vc_heads_to_rows")


def vc_argmax_rows(logits, tokens, *, stream=None):
    R, V = logits.shape
    _check(lib.vc_argmax_rows(_ptr(logits), R, V, _ptr(tokens), _stream(stream)), "vc_argmax_rows")


def vc_copy_kv_rows(src_k, src_v, src_row0, dst_k, dst_v, dst_row0, count, max_count, *, stream=None):
    B, Hkv, src_rows, d = src_k.shape
    _check(lib.vc_copy_kv_rows(_ptr(src_k), _ptr(src_v), src_rows, _ptr(src_row0), _ptr(dst_k), _ptr(dst_v),
                               dst_k.shape[2], _ptr(dst_row0), _ptr(count), max_count, B, Hkv, d,
                               src_k.element_size(), _stream(stream)), "vc_copy_kv_rows")
