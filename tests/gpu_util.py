"""Helpers of the GPU parity tests: seeded inputs on the device and the oracle's
results for the same inputs.  Oracle values are computed here from the seeded
inputs only; nothing computed by the HIP path is ever fed to the oracle."""
import numpy as np
import torch

from workloads import configs as C, gen as G
from oracle import quant as OQ

DEV = "cuda"
TOL = {"f32": 1e-4, "bf16": 2e-2}      # max-abs on attention outputs
# log-sum-exp: float32 on both storage types; with bf16 KV the probabilities enter the
# products (and their sum) rounded to bf16, 8 significant bits: the sum's relative
# error is at most 2^-8, so ln of it is off by at most ln(1 + 2^-8) < 3.9e-3
LSE_TOL = {"f32": 1e-4, "bf16": 4e-3}


def storage_half_ulp(ref, dtype):
    """Half a unit in the last place of the output storage type at |ref|: the bf16
    rounding of the stored result adds up to this much on top of the arithmetic
    error (a value of 28 in an outlier channel has a bf16 half-ulp of 0.0625)."""
    if dtype != "bf16":
        return 0.0
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def max_excess(got, ref, dtype):
    """max over elements of |got - ref| - (TOL + storage half-ulp); <= 0 passes."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    return float((err - TOL[dtype] - storage_half_ulp(ref, dtype)).max())


def assert_close(got, ref, dtype, what=""):
    ex = max_excess(got, ref, dtype)
    err = float(np.abs(np.asarray(got, np.float64) - ref).max())
    assert ex <= 0, f"{what} max-abs error {err:.4g} exceeds {TOL[dtype]} + storage half-ulp"


def tdtype(s):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[s]


def T(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def np32(t):
    return t.detach().float().cpu().numpy()


def oracle_compress(w, K, V):
    """Per-slice oracle quantization of [B, Hkv, N, d] K and V."""
    B, Hkv = K.shape[:2]
    out = [[OQ.compress_slice(K[b, h], V[b, h], w.k_bits, w.v_bits, w.group, w.scale_dtype) for h in range(Hkv)]
           for b in range(B)]
    stack = lambda key: np.stack([np.stack([out[b][h][key] for h in range(Hkv)]) for b in range(B)])
    return {k: stack(k) for k in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero")}


def oracle_dequant(w, comp):
    """Dequantized float64 K_hat, V_hat [B, Hkv, N, d] from oracle_compress() output."""
    B, Hkv, N = comp["k_codes"].shape[:3]
    d = w.d
    kh = np.zeros((B, Hkv, N, d))
    vh = np.zeros((B, Hkv, N, d))
    for b in range(B):
        for h in range(Hkv):
            c = {k: v[b, h] for k, v in comp.items()}
            kh[b, h], vh[b, h] = OQ.dequantize_slice(c, d, w.k_bits, w.v_bits, w.group)
    return kh, vh


def upload_quant(ckv, comp, n_rows, row0=0):
    """Copy oracle-packed rows into a Ckv's device arrays at rows [row0, row0 + n_rows)."""
    G_ = ckv.group
    ckv.k_codes[:, :, row0:row0 + n_rows] = T(comp["k_codes"].view(np.int32), torch.int32)
    ckv.v_codes[:, :, row0:row0 + n_rows] = T(comp["v_codes"].view(np.int32), torch.int32)
    pt = tdtype(ckv.param_dtype)
    ckv.k_scale[:, :, row0 // G_:(row0 + n_rows) // G_] = T(comp["k_scale"], pt)
    ckv.k_zero[:, :, row0 // G_:(row0 + n_rows) // G_] = T(comp["k_zero"], pt)
    ckv.v_scale[:, :, row0:row0 + n_rows] = T(comp["v_scale"], pt)
    ckv.v_zero[:, :, row0:row0 + n_rows] = T(comp["v_zero"], pt)


def inputs(w):
    """Seeded K, V [B,Hkv,N,d], window Q [B,Hq,k,d], window K, V [B,Hkv,k,d] (float32 arrays)."""
    return (G.full_kv(w, "k"), G.full_kv(w, "v"), G.full_window_q(w), G.full_window_kv(w, "k"),
            G.full_window_kv(w, "v"))


def say(msg):
    print(msg, flush=True)
