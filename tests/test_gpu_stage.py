"""GPU: full-KV staging from pinned host memory to the device and back (bytes
exact), ordered by an event on a side stream."""
import numpy as np
import pytest
import torch

import lossy_kv_draft_amd as L
from workloads import configs as C, gen as G

pytestmark = pytest.mark.gpu


def test_stage_rows_h2d_and_d2h():
    w = C.small(C.E2E, N=1000)
    K = torch.from_numpy(G.full_kv(w, "k")).to(torch.bfloat16).pin_memory()
    V = torch.from_numpy(G.full_kv(w, "v")).to(torch.bfloat16).pin_memory()
    dk = torch.zeros(w.B, w.Hkv, 1200, w.d, dtype=torch.bfloat16, device="cuda")
    dv = torch.zeros_like(dk)
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    L.vc_stage_full_kv(K, V, dk, dv, 100, 900, copy_stream=side, done=ev)
    torch.cuda.current_stream().wait_event(ev)
    got_k = dk.cpu()
    assert torch.equal(got_k[:, :, 100:900], K[:, :, 100:900])
    assert torch.all(got_k[:, :, :100] == 0) and torch.all(got_k[:, :, 900:] == 0)
    assert torch.equal(dv.cpu()[:, :, 100:900], V[:, :, 100:900])
    # device rows back to a pinned host copy
    hk = torch.zeros_like(K).pin_memory()
    hv = torch.zeros_like(V).pin_memory()
    dk[:, :, 950:960] = 3.0
    torch.cuda.synchronize()
    L.vc_stage_full_kv_d2h(dk, dv, hk, hv, 950, 960, copy_stream=side, done=ev)
    ev.synchronize()
    assert torch.all(hk[:, :, 950:960] == 3.0) and torch.all(hk[:, :, :950] == 0)
