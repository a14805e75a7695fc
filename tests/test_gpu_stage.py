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


# ---------------------------------------------------------------- staging from a file

def _prefix_file(tmp_path, arrays):
    """The arrays' bytes one after another in a file; returns (fd, byte offsets)."""
    import os
    path = tmp_path / "prefix.bin"
    offs, pos = [], 0
    with open(path, "wb") as f:
        for a in arrays:
            offs.append(pos)
            f.write(a.tobytes())
            pos += a.nbytes
    return os.open(path, os.O_RDONLY), offs


@pytest.mark.parametrize("dtype,chunk,n_threads,rows", [("bf16", 4096, 3, (3, 77)), ("f32", 4096, 8, (0, 400)),
                                                         ("bf16", 1 << 20, 2, (0, 1000)), ("f32", 8192, 4, (5, 5))])
def test_stage_from_file_bytes_exact(tmp_path, dtype, chunk, n_threads, rows):
    """Rows [lo, hi) of K and V stored in a file land on the same device rows, byte for
    byte (ranges cut into chunks that do not divide them), other rows untouched."""
    import os
    w = C.small(C.E2E, N=1000)
    K, V = G.full_kv(w, "k"), G.full_kv(w, "v")
    if dtype == "bf16":   # bf16 bit patterns carried as int16
        K, V = (torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy() for a in (K, V))
    fd, (_, ok, ov) = _prefix_file(tmp_path, [np.zeros(3, np.uint8), K, V])   # offsets not aligned
    tdt = torch.int16 if dtype == "bf16" else torch.float32
    dk = torch.full((w.B, w.Hkv, 1200, w.d), 7, dtype=tdt, device="cuda")
    dv = torch.full_like(dk, 7)
    st = L.FileStager(n_threads=n_threads, chunk_bytes=chunk, n_buffers=2 * n_threads)
    side, ev = torch.cuda.Stream(), torch.cuda.Event()
    lo, hi = rows
    t = st.stage(fd, ok, ov, dk, dv, w.N, lo, hi, copy_stream=side, done=ev)
    st.wait(t)
    torch.cuda.current_stream().wait_event(ev)
    gk, gv = dk.cpu().numpy(), dv.cpu().numpy()
    assert np.array_equal(gk[:, :, lo:hi], K[:, :, lo:hi]) and np.array_equal(gv[:, :, lo:hi], V[:, :, lo:hi])
    assert (gk[:, :, :lo] == 7).all() and (gk[:, :, hi:] == 7).all() and (gv[:, :, hi:] == 7).all()
    st.close()
    os.close(fd)


def test_stage_from_file_rate_cap_and_read_error(tmp_path):
    """A byte-rate cap holds (8 MiB at 256 MiB/s takes at least 31 ms); a read past the
    end of the file is reported (VC_ERR_IO) for its ticket only, and the stager goes on
    serving later calls."""
    import os
    import time
    K = np.arange(8 * 1024 * 1024 // 4, dtype=np.float32).reshape(1, 1, 8192, 256)
    fd, (ok,) = _prefix_file(tmp_path, [K])
    dk = torch.zeros(1, 1, 8192, 256, device="cuda")
    dv = torch.zeros_like(dk)
    st = L.FileStager(n_threads=4, chunk_bytes=1 << 20, n_buffers=8, max_bytes_per_s=256 * 2 ** 20)
    t0 = time.perf_counter()
    t = st.stage(fd, ok, ok, dk, dv, 8192, 0, 4096)          # K and V both from the same 4 MiB
    st.wait(t)
    torch.cuda.synchronize()
    took = time.perf_counter() - t0
    assert took >= 8 / 256 - 1e-3, took
    assert np.array_equal(dk.cpu().numpy()[:, :, :4096], K[:, :, :4096])
    assert np.array_equal(dv.cpu().numpy()[:, :, :4096], K[:, :, :4096])
    st.close()
    st = L.FileStager(n_threads=2, chunk_bytes=1 << 16, n_buffers=4)
    bad = st.stage(fd, ok, ok + 4 * 2 ** 20, dk, dv, 8192, 0, 8192)   # V runs 4 MiB past the end
    with pytest.raises(L.VcError) as e:
        st.wait(bad)
    assert e.value.status == L.VC_ERR_IO and "end of the file" in str(e.value)
    torch.cuda.synchronize()
    dk.zero_()
    st.wait(st.stage(fd, ok, ok, dk, dv, 8192, 100, 200))
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy()[:, :, 100:200], K[:, :, 100:200])
    st.close()
    os.close(fd)
