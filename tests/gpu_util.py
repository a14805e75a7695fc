"""Helpers of the GPU parity tests: seeded inputs on the device and the oracle's
results for the same inputs.  Oracle values are computed here from the seeded
inputs only; nothing computed by the HIP path is ever fed to the oracle."""
import numpy as np
import torch

from workloads import configs as C, gen as G
from oracle import quant as OQ

DEV = "cuda"
TOL = {"f32": 1e-4, "bf16": 2e-2}      # max-abs on attention outputs
LSE_TOL = {"f32": 1e-4, "bf16": 2e-3}  # log-sum-exp is float32 on both storage types


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
