"""Benchmark of the VeriCache draft-and-verify hot path on one MI355X.

One step = one kernel-level draft-and-verify round over one batch of synthetic
inputs resident in HBM:
  draft   k single-token decode-attention calls over the compressed cache (draft
          step i attends to the compressed context plus window rows 0..i),
  verify  causal window attention of the k rows over the full bf16 cache,
  tokens  head mean + greedy argmax through a fixed random vocabulary projection
          for the draft and the verify rows, then longest-prefix acceptance.
Staging of the full KV from pinned host memory (PCIe) and compression are measured
separately (they are not part of `value`).

value = compressed decode-attention HBM GB/s (algorithmic bytes of the k decode
calls / their time; the k calls are replayed from one HIP graph, as the end-to-end
rounds do).  verify TFLOP/s is reported beside it, and "e2e" holds the
accepted tokens/s of whole draft-and-verify rounds of a random-init 4-layer decoder
after a 32k-token prompt (full KV staged from pinned host memory every round),
beside greedy full-KV decoding with the KV resident and with it staged every step.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed decode-attn HBM GB/s; verify-attn TFLOP/s; accepted tok/s @32k ctx"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llama8b", choices=["llama8b", "qwen30b", "drop", "tiny"])
    p.add_argument("--copies", type=int, default=3, help="compressed-cache copies rotated across draft calls")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-stage", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-e2e", action="store_true", help="skip the end-to-end decoder rounds")
    p.add_argument("--no-remote-prefix", action="store_true",
                   help="skip the end-to-end rounds with the prompt's full KV staged from a file")
    p.add_argument("--e2e-ctx", type=int, default=32768, help="prompt length of the end-to-end rounds")
    p.add_argument("--e2e-gen", type=int, default=256, help="tokens generated per sequence")
    p.add_argument("--e2e-slots", type=int, default=2, help="device layer slots of the staged full KV")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="first run a plain device copy of this many MiB (3 times): the reference dispatch that "
                        "scales hardware traffic counters to bytes")
    return p.parse_args()


# Committed counter summaries of the decode kernel per workload, and the sources whose
# hash they record (a summary taken on other sources is not reported).
TRAFFIC = {
    "llama8b_n32k_4bit": ("decode_mfma_llama8b_n32k_hbm_traffic.txt",
                          ("decode_mfma.hip", "decode_common.h", "decode.hip", "common.h")),
    "drop25_n128k": ("decode_dense_drop25_n128k_hbm_traffic.txt",
                     ("verify.hip", "decode_common.h", "decode.hip", "common.h")),
}


def source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "lossy_kv_draft_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per decode launch from the committed counter summary, if it was
    taken on the current decode sources and this workload; else None."""
    if workload_name not in TRAFFIC:
        return None
    fname, files = TRAFFIC[workload_name]
    try:
        with open(os.path.join(ROOT, "profiles", fname)) as fh:
            kv = dict(line[2:].split(":", 1) for line in fh if line.startswith("# ") and ":" in line)
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != source_hash(files) or kv.get("workload") != workload_name:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def decode_bytes(w, n_ctx, tail):
    """Algorithmic bytes of one decode call: the compressed rows it must read (codes
    and group parameters, or the kept bf16 rows), the tail rows, the queries and the
    outputs."""
    bh = w.B * w.Hkv
    eb = 4 if w.dtype == "f32" else 2
    if w.method == "quant":
        pb = 4 if w.scale_dtype == "f32" else 2
        main = bh * n_ctx * w.d * (w.k_bits + w.v_bits) // 8
        main += bh * (n_ctx // w.group) * w.d * 2 * pb + bh * n_ctx * (w.d // w.group) * 2 * pb
    else:
        main = bh * n_ctx * w.d * 2 * eb
    return main + bh * tail * w.d * 2 * eb + 2 * w.B * w.Hq * w.d * eb


def verify_flops(w, n_ctx):
    """4 * B * Hq * d * sum_i (N + i + 1): QK^T and PV over the visible keys."""
    return 4.0 * w.B * w.Hq * w.d * sum(n_ctx + i + 1 for i in range(w.k))


def verify_bytes(w, n_ctx):
    eb = 4 if w.dtype == "f32" else 2
    return w.B * w.Hkv * (n_ctx + w.k) * w.d * 2 * eb + 2 * w.B * w.Hq * w.k * w.d * eb


def workload(name):
    from workloads import configs as C
    w = {"llama8b": C.LLAMA8B, "qwen30b": C.QWEN30B, "drop": C.DROP, "tiny": C.TINY}[name]
    # A projection for the greedy tokens: the Llama-3-8B-shaped and token-dropping
    # layers name none, so they use a Llama-3 sized vocabulary (128256).
    if w.vocab == 0:
        w = w.with_(vocab=128256, w_dtype="bf16")
    return w


def setup(w, copies):
    import torch
    import lossy_kv_draft_amd as L
    from workloads import gen as G
    dev = "cuda"
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    rows = w.N + w.k
    t0 = time.time()
    kc = torch.empty(w.B, w.Hkv, rows, w.d, dtype=dt, device=dev)
    vc = torch.empty_like(kc)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        for b in range(w.B):
            for which, dst in (("k", kc), ("v", vc)):
                rows_b = list(ex.map(lambda h: G.kv_slice(w, which, b, h), range(w.Hkv)))
                dst[b, :, :w.N] = torch.from_numpy(np.stack(rows_b)).to(dev, dt)
    kc[:, :, w.N:] = torch.from_numpy(G.full_window_kv(w, "k")).to(dev, dt)
    vc[:, :, w.N:] = torch.from_numpy(G.full_window_kv(w, "v")).to(dev, dt)
    q = torch.from_numpy(G.full_window_q(w)).to(dev, dt)
    Wp = torch.from_numpy(G.projection(w)).to(dev, torch.float32 if w.w_dtype == "f32" else torch.bfloat16)
    print(f"[bench] inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    ckvs = []
    comp_ms = None
    for c in range(copies):
        if w.method == "quant":
            ckv = L.Ckv("quant", w.B, w.Hkv, w.d, w.N, k_bits=w.k_bits, v_bits=w.v_bits, group=w.group,
                        param_dtype=w.scale_dtype, kv_dtype=w.dtype, tail_cap=w.k)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            L.vc_compress(ckv, kc, vc, n_tokens=w.N)
            e1.record()
            torch.cuda.synchronize()
            comp_ms = e0.elapsed_time(e1)
            ckv.n_main = w.N
        else:
            keep = L.vc_drop_keep_count(w.keep_ratio, w.N)
            ckv = L.Ckv("drop", w.B, w.Hkv, w.d, keep, keep_ratio=w.keep_ratio, kv_dtype=w.dtype, tail_cap=w.k)
            probes = torch.from_numpy(G.full_probes(w)).to(dev, torch.bfloat16)
            ksrc = kc[:, :, :w.N].contiguous()
            vsrc = vc[:, :, :w.N].contiguous()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            L.vc_compress(ckv, ksrc, vsrc, probes=probes)
            e1.record()
            torch.cuda.synchronize()
            comp_ms = e0.elapsed_time(e1)
            del ksrc, vsrc
            ckv.n_main = keep
        ckv.tail_k.copy_(kc[:, :, w.N:])
        ckv.tail_v.copy_(vc[:, :, w.N:])
        ckvs.append(ckv)
    st = dict(w=w, kc=kc, vc=vc, q=q, W=Wp, ckvs=ckvs, dt=dt, comp_ms=comp_ms)
    st["dec_ws"] = L.workspace(L.vc_decode_workspace_bytes(ckvs[0], w.Hq))
    st["ver_ws"] = L.workspace(L.vc_verify_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.k, w.N))
    R = w.B * w.k
    st["lg_ws"] = L.workspace(L.vc_logits_workspace_bytes(R, w.vocab))
    st["qrows"] = [q[:, :, i].contiguous() for i in range(w.k)]
    # draft outputs [k, B, Hq, d]: step i writes slice i; read as [B, Hq, k, d] by stride
    st["dec_all"] = torch.empty(w.k, w.B, w.Hq, w.d, dtype=dt, device=dev)
    st["dec_out"] = [st["dec_all"][i] for i in range(w.k)]
    st["out_v"] = torch.empty(w.B, w.Hq, w.k, w.d, dtype=dt, device=dev)
    st["u_d"] = torch.empty(R, w.d, device=dev)
    st["u_v"] = torch.empty(R, w.d, device=dev)
    st["tok_d"] = torch.empty(R, dtype=torch.int32, device=dev)
    st["tok_v"] = torch.empty(R, dtype=torch.int32, device=dev)
    st["acc"] = torch.empty(w.B, dtype=torch.int32, device=dev)
    st["nc"] = torch.empty(w.B, dtype=torch.int32, device=dev)
    st["com"] = torch.empty(w.B, w.k, dtype=torch.int32, device=dev)
    return st


def draft_calls(st, dec_ev=None):
    """The k draft decode calls of one round (step i sees i + 1 tail rows).  dec_ev:
    list of (start, end) event pairs around each decode launch."""
    import lossy_kv_draft_amd as L
    w = st["w"]
    for i in range(w.k):
        ckv = st["ckvs"][i % len(st["ckvs"])]
        ckv.tail_len = i + 1
        if dec_ev:
            dec_ev[i][0].record()
        L.vc_decode_attn_compressed(ckv, st["qrows"][i], st["dec_out"][i], ws=st["dec_ws"])
        if dec_ev:
            dec_ev[i][1].record()


def capture_draft(st):
    """The k draft calls captured once as a HIP graph (their arguments, tail lengths
    included, are fixed per step), replayed in every timed round: host launch gaps
    between the calls are gone."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        draft_calls(st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        draft_calls(st)
    torch.cuda.synchronize()
    return g


def run_step(st, ev=None, graph=None):
    """One round.  ev: 4 events (start, after draft, after verify, after tokens);
    graph: the captured draft calls (else they are launched one by one)."""
    import lossy_kv_draft_amd as L
    w = st["w"]
    if ev:
        ev[0].record()
    if graph is not None:
        graph.replay()
    else:
        draft_calls(st)
    if ev:
        ev[1].record()
    L.vc_verify_attn_full(st["q"], st["kc"], st["vc"], w.N, st["out_v"], ws=st["ver_ws"])
    if ev:
        ev[2].record()
    L.vc_head_mean(st["dec_all"].permute(1, 2, 0, 3), st["u_d"])
    L.vc_head_mean(st["out_v"], st["u_v"])
    L.vc_logits_argmax(st["u_d"], st["W"], st["tok_d"], ws=st["lg_ws"])
    L.vc_logits_argmax(st["u_v"], st["W"], st["tok_v"], ws=st["lg_ws"])
    L.vc_accept(st["tok_d"].view(w.B, w.k), st["tok_v"].view(w.B, w.k), st["acc"], st["nc"], st["com"])
    if ev:
        ev[3].record()


def measure_rotation(st):
    """The rotation pre-pass (vc_hadamard_rows) over the layer's full K: one read and
    one write of every row; HBM-bound."""
    import torch
    import lossy_kv_draft_amd as L
    x = st["kc"]
    y = torch.empty_like(x)
    for _ in range(2):
        L.vc_hadamard_rows(x, y)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        L.vc_hadamard_rows(x, y)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 5 * 1e3
    nbytes = 2 * x.numel() * x.element_size()
    return {"rows": int(x.numel() // x.shape[-1]), "d": int(x.shape[-1]), "us": round(us, 2),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 /
                                                                                   HBM_PEAK_GBS, 4)}


def measure_split_stream(st, anchor_bits=2):
    """The split-stream compressor on the layer's compressed cache: vc_split_planes
    (anchor of the top `anchor_bits` bits plus residual), and the draft decode over the
    anchor alone against the decode over the full-width cache (same query, same
    tail)."""
    import torch
    import lossy_kv_draft_amd as L
    w = st["w"]
    full = st["ckvs"][0]
    if w.method != "quant" or min(full.k_bits, full.v_bits) <= anchor_bits:
        return None
    anchor = L.Ckv("quant", w.B, w.Hkv, w.d, w.N, k_bits=anchor_bits, v_bits=anchor_bits, group=w.group,
                   param_dtype=w.scale_dtype, kv_dtype=w.dtype, tail_cap=w.k)
    anchor.tail_k, anchor.tail_v = full.tail_k, full.tail_v
    anchor.n_main = full.n_main
    kr, vr = L.split_residuals(full, anchor)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    split_us = timed(lambda: L.vc_split_planes(full, anchor, kr, vr, w.N), 5)
    full.tail_len = anchor.tail_len = w.k
    q, out = st["qrows"][w.k - 1], st["dec_out"][w.k - 1]
    full_us = timed(lambda: L.vc_decode_attn_compressed(full, q, out, ws=st["dec_ws"]), 20)
    anchor_us = timed(lambda: L.vc_decode_attn_compressed(anchor, q, out, ws=st["dec_ws"]), 20)
    moved = full.stored_bytes(w.N) + anchor.stored_bytes(w.N) + sum(t.numel() * 4 for t in (kr, vr) if t is not None)
    anchor_bytes = decode_bytes(w.with_(k_bits=anchor_bits, v_bits=anchor_bits), w.N, w.k)
    return {"anchor_bits": anchor_bits, "split_us": round(split_us, 2),
            "split_GBps": round(moved / (split_us * 1e-6) / 1e9, 1),
            "decode_full_us": round(full_us, 2), "decode_anchor_us": round(anchor_us, 2),
            "decode_anchor_GBps": round(anchor_bytes / (anchor_us * 1e-6) / 1e9, 1),
            "anchor_speedup": round(full_us / anchor_us, 3)}


def measure_stage(st):
    """Full-KV swap-in: H2D copy of the whole context of one layer from pinned host
    memory on a side stream, alone and overlapped with the k draft decodes."""
    import torch
    import lossy_kv_draft_amd as L
    w = st["w"]
    hk = torch.empty(st["kc"].shape, dtype=st["dt"], pin_memory=True)
    hv = torch.empty(st["vc"].shape, dtype=st["dt"], pin_memory=True)
    hk.copy_(st["kc"])
    hv.copy_(st["vc"])
    dk = torch.empty_like(st["kc"])
    dv = torch.empty_like(st["vc"])
    side = torch.cuda.Stream()
    nbytes = 2 * w.B * w.Hkv * w.N * w.d * hk.element_size()
    done = torch.cuda.Event()

    def stage():
        L.vc_stage_full_kv(hk, hv, dk, dv, 0, w.N, copy_stream=side, done=done)

    def draft():
        draft_calls(st)

    res = {}
    for name, fn in (("stage_alone", lambda: (stage(), done.synchronize())),
                     ("draft_alone", lambda: (draft(), torch.cuda.synchronize())),
                     ("overlapped", lambda: (stage(), draft(), torch.cuda.current_stream().wait_event(done),
                                             torch.cuda.synchronize()))):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        res[name] = min(ts) * 1e3
    ok = torch.equal(dk[:, :, :w.N], st["kc"][:, :, :w.N])
    return {"bytes": nbytes, "h2d_GBps": round(nbytes / (res["stage_alone"] * 1e-3) / 1e9, 2),
            "stage_ms": round(res["stage_alone"], 3), "draft_ms": round(res["draft_alone"], 3),
            "overlapped_ms": round(res["overlapped"], 3),
            "overlap_hidden_frac": round((res["stage_alone"] + res["draft_alone"] - res["overlapped"]) /
                                         min(res["stage_alone"], res["draft_alone"]), 3),
            "copy_exact": bool(ok)}


def e2e_rounds(ctx, gen, slots, remote=True):
    """Draft-and-verify decoding of the random-init 4-layer decoder (d_model 2048,
    16/4 heads, SwiGLU 5504, vocab 32000, batch 4, 2-bit KIVI drafts, k = 32) after a
    prompt of `ctx` tokens: accepted tokens/s with the full KV staged from pinned host
    memory every round, beside greedy full-KV decoding with the full KV resident and
    with it staged every step.  The draft-and-verify output is checked against the
    resident greedy output."""
    import torch
    from workloads import configs as C, gen as G
    from lossy_kv_draft_amd import round as R
    w = C.E2E.with_(N=ctx, gen_tokens=gen, name=f"decoder4l_n{ctx // 1024}k_2bit")
    shape = R.ModelShape(layers=w.layers, d_model=w.d_model, Hq=w.Hq, Hkv=w.Hkv, hd=w.d, ffn=w.ffn, vocab=w.vocab)
    seed = lambda key, shp, s: G.normal(w, key, shp, s, "f32")
    weights = R.weights_to(R.random_weights(shape, seed, std=0.02, device="cpu"), "cuda")
    prompt = G.tokens(w, 0, shape=(w.B, w.N), high=w.vocab)
    chunk = 512
    dec = R.DecoderGPU(shape, weights, max_rows=w.B * max(w.k, chunk))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sess = R.Session(dec, prompt, w.k, gen, chunk=chunk, group=w.group, bits=(w.k_bits, w.v_bits))
    prefill_s = time.perf_counter() - t0

    def timed(fn):
        torch.cuda.synchronize()
        t = time.perf_counter()
        out = fn()
        torch.cuda.synchronize()
        return out, time.perf_counter() - t

    note = lambda m: print(f"[bench] e2e: {m}", file=sys.stderr, flush=True)
    note(f"prefill done in {prefill_s:.1f}s; greedy baselines")
    g = R.Greedy(sess)
    g.run(4)                                                    # warm-up
    g = R.Greedy(sess)
    ref, t_res = timed(lambda: g.run())
    n_staged = 8
    gs = R.Greedy(sess, slots=slots)
    gs.run(2)
    _, t_st = timed(lambda: gs.run(2 + n_staged))
    del gs
    note("draft-and-verify")
    warm = R.VeriCacheLoop(sess, slots=slots)
    warm.round()
    del warm
    loop = R.VeriCacheLoop(sess, slots=slots)
    got, t_vc = timed(lambda: loop.run(timed=True))
    ok = bool(np.array_equal(got, ref))
    note("cost model calibration")
    calib = cost_calibration(R, sess, w, timed)
    # the same batch with the draft horizon chosen per round by the cost model
    note("adaptive horizon")
    horizons = tuple(h for h in (4, 8, 16, 32) if h <= w.k)
    ada = R.VeriCacheLoop(sess, slots=slots, horizons=horizons)
    got_a, t_ada = timed(lambda: ada.run())
    adaptive = {"horizons": list(horizons), "accepted_tok_per_s": round(w.B * (gen - 1) / t_ada, 1),
                "rounds": ada.rounds, "rounds_per_horizon": {str(k): v for k, v in ada.policy.chosen.items()},
                "mean_round_ms_per_horizon": {str(k): round(float(np.mean(v)) * 1e3, 2)
                                              for k, v in ada.policy.times.items() if v},
                "output_equals_greedy": bool(np.array_equal(got_a, ref))}
    del ada
    if remote:
        note("prefix staged from a file")
        remote = remote_prefix_rounds(w, sess, ref, slots, gen, timed)
    else:
        remote = None
    # the same batch with every layer's slot on the device (all staging under the drafts)
    note(f"{w.layers} device slots")
    loop4 = R.VeriCacheLoop(sess, slots=w.layers)
    got4, t_4 = timed(lambda: loop4.run())
    all_slots = {"device_kv_slots": w.layers, "accepted_tok_per_s": round(w.B * (gen - 1) / t_4, 1),
                 "rounds": loop4.rounds, "round_ms": round(t_4 / loop4.rounds * 1e3, 3),
                 "output_equals_greedy": bool(np.array_equal(got4, ref))}
    del loop4
    cost = cost_model_points(w, calib, slots, t_vc / loop.rounds, t_4 / all_slots["rounds"], adaptive, remote,
                             commits=(gen - 1) / loop.rounds)
    note("staggered batches")
    stag = staggered_rounds(w, shape, weights, sess, ref, slots, gen, chunk, timed)
    committed = w.B * (gen - 1)                                 # tokens produced after the prefill's first
    staged_bytes = loop.full.bytes_staged if hasattr(loop.full, "bytes_staged") else 0
    vc_tps = committed / t_vc
    res_tps = committed / t_res
    st_tps = w.B * n_staged / t_st
    return {"workload": w.name, "batch": w.B, "prompt_tokens": w.N, "generated_per_seq": gen,
            "draft_window": w.k, "layers": w.layers, "device_kv_slots": slots,
            "accepted_tok_per_s": round(vc_tps, 1),
            "mean_accept_len": round(float(np.mean(loop.accept_lens)), 3),
            "mean_commit_per_round": round(committed / w.B / loop.rounds, 3), "rounds": loop.rounds,
            "round_ms": round(t_vc / loop.rounds * 1e3, 3),
            "phase_ms_per_round": {k: round(v / loop.rounds, 3) for k, v in loop.phase_ms.items()},
            "staged_GB_per_round": round(staged_bytes / loop.rounds / 1e9, 3),
            "greedy_resident_tok_per_s": round(res_tps, 1),
            "greedy_staged_tok_per_s": round(st_tps, 1),
            "speedup_vs_greedy_staged": round(vc_tps / st_tps, 2),
            "speedup_vs_greedy_resident": round(vc_tps / res_tps, 3),
            "output_equals_greedy": ok, "prefill_s": round(prefill_s, 2),
            "adaptive_horizon": adaptive,
            "all_slots": all_slots,
            "cost_model": cost,
            "remote_prefix": remote,
            "staggered": stag,
            "note": "random-init weights and uniform-random prompts; acceptance is a property of this "
                    "synthetic model, not of a trained one"}


def cost_calibration(R, sess, w, timed, horizons=(4, 8, 16, 32), rounds=3):
    """Component times of a round, measured apart from the rounds the model predicts:
    loops over the resident full KV (no staging) at each horizon give the draft step,
    the verify pass per layer and what follows it (tokens, acceptance, cache update,
    sync); staging the full KV through the slot ring with nothing else running gives
    the link's time per layer."""
    import torch
    out = {"horizons": {}}
    for k in horizons:
        lp = R.VeriCacheLoop(sess, slots=None, horizons=[k])
        lp.round()                                              # warm
        lp.phase_ms = {n: 0.0 for n in lp.phase_ms}
        r0 = lp.rounds
        _, t = timed(lambda: [lp.round(timed=True) for _ in range(rounds)])
        n = lp.rounds - r0
        draft, verify = lp.phase_ms["draft"] / n / 1e3, lp.phase_ms["verify"] / n / 1e3
        out["horizons"][k] = {"t_step": draft / k, "t_layer": verify / w.layers, "t_tail": t / n - draft - verify}
        del lp
        torch.cuda.empty_cache()
    # the link: every layer staged through the slots of a staged loop, back to back
    lp = R.VeriCacheLoop(sess, slots=2, horizons=[horizons[0]])
    full, n_rows = lp.full, int(lp.Lb.max())
    t_best = None
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        b0 = full.bytes_staged
        full.begin(n_rows, n_rows, n_rows)
        for l in range(full.layers):
            full.acquire(l)
            full.release(l)
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
        t_best = t if t_best is None else min(t_best, t)
        nbytes = full.bytes_staged - b0
    out["layer_bytes"] = nbytes / full.layers
    out["link_Bps"] = nbytes / t_best
    del lp
    torch.cuda.empty_cache()
    return out


def cost_model_points(w, calib, slots, t_fixed, t_all_slots, adaptive, remote, commits):
    """Round times the cost model predicts from the calibration, beside the measured
    rounds: the fixed horizon over `slots` slots and over one slot per layer, each
    horizon of the adaptive loop, and the prefix staged from a file (its link rate
    from the file stager's measured rate).  Also the speedup over greedy with the full
    KV staged every token on a grid of acceptance lengths and link rates."""
    from lossy_kv_draft_amd import costmodel as CM
    hz = calib["horizons"]
    lb, link = calib["layer_bytes"], calib["link_Bps"]

    def costs(k, n_slots, rate=link):
        c = hz[k]
        return CM.RoundCosts(layers=w.layers, slots=n_slots, t_step=c["t_step"], t_layer=c["t_layer"],
                             t_stage=lb / rate, t_tail=c["t_tail"])

    pts = []

    def add(name, k, n_slots, measured_s, rate=link):
        pred = CM.round_time(k, costs(k, n_slots, rate))
        pts.append({"setting": name, "predicted_round_ms": round(pred * 1e3, 2),
                    "measured_round_ms": round(measured_s * 1e3, 2),
                    "rel_err": round(pred / measured_s - 1.0, 3)})

    add(f"fixed k={w.k}, {slots} slots", w.k, slots, t_fixed)
    add(f"fixed k={w.k}, {w.layers} slots", w.k, w.layers, t_all_slots)
    for k, ms in adaptive.get("mean_round_ms_per_horizon", {}).items():
        if int(k) in hz and adaptive["rounds_per_horizon"].get(k, 0) >= 3:
            add(f"adaptive, horizon {k}", int(k), slots, ms / 1e3)
    for r in remote or []:
        file_rate = r["file_stage_GBps"] * 1e9
        # per layer: the prompt rows from the file, the generated rows from pinned memory
        p_frac = w.N / (w.N + w.gen_tokens / 2)
        rate = 1.0 / (p_frac / file_rate + (1.0 - p_frac) / link)
        cap = r["link_cap_GBps"]
        add(f"prefix from a file, {'uncapped' if cap is None else f'{cap} GB/s cap'}", w.k, slots,
            r["round_ms"] / 1e3, rate)
    errs = [abs(p["rel_err"]) for p in pts]
    p_acc = CM.accept_p_from_commits(commits, w.k)
    surf = CM.speedup_surface(w.B, w.k, costs(w.k, slots), lb, hz[min(hz)]["t_layer"] * w.layers,
                              accepted_lens=(0.5, 4.0, 10.0, 25.0, 40.0),
                              link_rates=(8e9, 16e9, 32e9, link, 128e9))
    best = {str(a): CM.best_horizon(w.B, sorted(hz), CM.accept_p_from_commits(min(a + 1.0, w.k), w.k),
                                    lambda k: costs(k, slots))
            for a in (0.5, 4.0, 25.0)}
    return {"calibration": {"t_step_ms": {str(k): round(v["t_step"] * 1e3, 3) for k, v in hz.items()},
                            "t_layer_ms": {str(k): round(v["t_layer"] * 1e3, 3) for k, v in hz.items()},
                            "t_tail_ms": {str(k): round(v["t_tail"] * 1e3, 3) for k, v in hz.items()},
                            "layer_MB": round(lb / 1e6, 1), "link_GBps": round(link / 1e9, 2)},
            "points": pts, "max_abs_rel_err": round(max(errs), 3) if errs else None,
            "accept_p": round(p_acc, 3),
            "predicted_accepted_tok_per_s": round(CM.tokens_per_s(w.B, w.k, p_acc, costs(w.k, slots)), 1),
            "best_horizon_by_accepted_drafts": best,
            "speedup_vs_staged_greedy": [{"accepted": a, "link_GBps": round(r / 1e9, 1), "speedup": round(x, 2)}
                                         for a, r, _, x in surf]}


def remote_prefix_rounds(w, sess, ref, slots, gen, timed, rates=(0.0, 25e9)):
    """The remote-prefix-cache setting: the prompt's full KV staged every round from a
    file (page-cached; the store's stand-in) by the library's reader threads, uncapped
    and capped at 25 GB/s (a 200 Gb/s link); the generated rows from pinned host
    memory.  Also the stager's raw rate: the prompt rows of the first `slots` layers
    staged alone."""
    import torch
    from lossy_kv_draft_amd import round as R
    out = []
    for rate in rates:
        loop = R.VeriCacheLoop(sess, slots=slots, prefix_store=dict(max_bytes_per_s=rate))
        full = loop.full
        full.begin(w.N, w.N, w.N)                   # warm the file's pages and the stager
        for l in range(full.slots):
            full.acquire(l)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        b0 = full.bytes_from_file
        full.begin(w.N, w.N, w.N)
        for l in range(full.slots):
            full.acquire(l)
        torch.cuda.synchronize()
        t_stage = time.perf_counter() - t0
        stage_bytes = full.bytes_from_file - b0
        b0 = full.bytes_from_file
        got, t = timed(lambda: loop.run())
        out.append({"link_cap_GBps": rate / 1e9 if rate else None,
                    "file_stage_GBps": round(stage_bytes / t_stage / 1e9, 2),
                    "accepted_tok_per_s": round(w.B * (gen - 1) / t, 1), "rounds": loop.rounds,
                    "round_ms": round(t / loop.rounds * 1e3, 2),
                    "file_GB_per_round": round((full.bytes_from_file - b0) / loop.rounds / 1e9, 3),
                    "output_equals_greedy": bool(np.array_equal(got, ref))})
        full.close()
        del loop, full
        torch.cuda.empty_cache()
    return out


def staggered_rounds(w, shape, weights, sess0, ref0, slots, gen, chunk, timed):
    """Cross-resource staggering: the batch above plus a second batch of the same
    size (its own prompts, decoder buffers, caches and staging stream), decoded at
    once by two host threads on two compute streams, so that one batch's drafting
    overlaps the other's staging and verification.  Compared with one batch of twice
    the size decoded alone."""
    import torch
    from workloads import gen as G
    from lossy_kv_draft_amd import round as R
    prompt1 = G.tokens(w, 1, shape=(w.B, w.N), high=w.vocab)
    dec1 = R.DecoderGPU(shape, weights, max_rows=w.B * max(w.k, chunk))
    sess1 = R.Session(dec1, prompt1, w.k, gen, chunk=chunk, group=w.group, bits=(w.k_bits, w.v_bits))
    ref1 = R.Greedy(sess1).run()
    st = R.Staggered([R.VeriCacheLoop(sess0, slots=slots), R.VeriCacheLoop(sess1, slots=slots)])
    got, t_st = timed(lambda: st.run())
    ok = bool(np.array_equal(got[0], ref0) and np.array_equal(got[1], ref1))
    rounds = [lp.rounds for lp in st.loops]
    committed = 2 * w.B * (gen - 1)
    del st, sess1, dec1
    torch.cuda.empty_cache()
    # one batch of 2B sequences (both prompt sets), decoded alone
    dec2 = R.DecoderGPU(shape, weights, max_rows=2 * w.B * max(w.k, chunk))
    sess2 = R.Session(dec2, np.concatenate([G.tokens(w, 0, shape=(w.B, w.N), high=w.vocab), prompt1]), w.k, gen,
                      chunk=chunk, group=w.group, bits=(w.k_bits, w.v_bits))
    ref2 = R.Greedy(sess2).run()   # its own reference: its verify split is the one for 2B sequences
    big = R.VeriCacheLoop(sess2, slots=slots)
    got2, t_big = timed(lambda: big.run())
    ok = ok and bool(np.array_equal(got2, ref2))
    out = {"batches": 2, "batch": w.B, "accepted_tok_per_s": round(committed / t_st, 1),
           "rounds_per_batch": rounds, "wall_s": round(t_st, 3),
           "one_batch_of_2B_tok_per_s": round(committed / t_big, 1),
           "output_equals_greedy": ok}
    del big, sess2, dec2
    torch.cuda.empty_cache()
    return out


def verify_mfma_shape(steps=20, warmup=5):
    """Verification at the Qwen3-30B-A3B-shaped layer (B16, 32/4 heads, d 128, N 65536,
    window 40: AI 320 flop per byte, where the matrix cores and not HBM bound it):
    seeded N(0, 1) bf16 inputs made on the device, each call timed between HIP events."""
    import torch
    import lossy_kv_draft_amd as L
    w = workload("qwen30b")
    rows = w.N + w.k
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + w.index)
    kc = torch.randn(w.B, w.Hkv, rows, w.d, device="cuda", dtype=torch.bfloat16, generator=g)
    vc = torch.randn(w.B, w.Hkv, rows, w.d, device="cuda", dtype=torch.bfloat16, generator=g)
    q = torch.randn(w.B, w.Hq, w.k, w.d, device="cuda", dtype=torch.bfloat16, generator=g)
    out = torch.empty_like(q)
    ws = L.workspace(L.vc_verify_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.k, w.N))
    call = lambda: L.vc_verify_attn_full(q, kc, vc, w.N, out, ws=ws)
    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
    med = float(np.median(us))
    flops, nbytes = verify_flops(w, w.N), verify_bytes(w, w.N)
    tflops = flops / (med * 1e-6) / 1e12
    attain = min(BF16_PEAK_TFLOPS, flops / nbytes * HBM_PEAK_GBS / 1e3)
    del kc, vc, q, out, ws
    torch.cuda.empty_cache()
    return {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "seq_len": w.N, "window": w.k,
            "call_us": spread(us), "tflops": round(tflops, 1), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
            "ai_flop_per_byte": round(flops / nbytes, 1), "attainable_tflops": round(attain, 1),
            "frac_of_attainable": round(tflops / attain, 4), "hbm_gbs": round(nbytes / (med * 1e-6) / 1e9, 1)}


def gpu_state():
    """Clocks and power of the GPU from the amdgpu driver's files in sysfs (read-only;
    no child process is started, so nothing inherits a profiler's preloaded library):
    the current levels of pp_dpm_sclk / pp_dpm_mclk and the hwmon power reading."""
    import glob
    import re
    out = {"source": "sysfs (amdgpu)"}

    def read(path):
        try:
            with open(path) as fh:
                return fh.read()
        except OSError:
            return None

    for dev in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        if (read(dev + "/vendor") or "").strip() != "0x1002":
            continue
        for name, key in (("pp_dpm_sclk", "gfx_clk_mhz"), ("pp_dpm_mclk", "mem_clk_mhz")):
            txt = read(f"{dev}/{name}")
            if txt:
                levels = [int(m) for m in re.findall(r"(\d+)\s*[Mm][Hh]z", txt)]
                cur = re.search(r"(\d+)\s*[Mm][Hh]z\s*\*", txt)
                if cur:
                    out[key] = int(cur.group(1))
                if levels and key == "gfx_clk_mhz":
                    out["gfx_max_clk_mhz"] = max(levels)
        for hw in sorted(glob.glob(dev + "/hwmon/hwmon*")):
            for f in ("power1_average", "power1_input"):
                v = read(f"{hw}/{f}")
                if v and v.strip().isdigit():
                    out["socket_power_w"] = round(int(v) / 1e6, 1)
                    break
        if len(out) > 1:
            return out
    out["unavailable"] = "no amdgpu clock or power files visible"
    return out


def spread(v_us):
    """median, p10 and p90 of a list of durations in microseconds."""
    q = np.percentile(np.asarray(v_us, dtype=np.float64), [50, 10, 90])
    return {"median": round(float(q[0]), 3), "p10": round(float(q[1]), 3), "p90": round(float(q[2]), 3)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds):
    """The oracle (numpy; float64 attention, float32 quantization arithmetic) timed on
    the host, BLAS threads pinned to the visible cores, on bounded samples of the
    same workload.  The headline leg: whole (sequence, kv-head) slices -- dequantize
    the slice's compressed rows and decode one draft query of each of its q-heads --
    repeated until about `seconds` of work, scaled to GB/s of the same algorithmic
    bytes.  Beside it: compressing slices (quantize + pack), verifying one slice's
    window over its full context, acceptance of the batch's window, and one
    draft-and-verify round of the end-to-end decoder at a reduced prompt."""
    from workloads import gen as G, configs as Cfg
    from oracle import quant as OQ, attention as OA, drop as OD, accept as OC, model as OM
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=cores)
    except Exception:
        limit = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    grp = w.Hq // w.Hkv
    n_slices = w.B * w.Hkv
    per_slice = decode_bytes(w, w.N, 1) / n_slices
    done, t_total, b, h = 0, 0.0, 0, 0
    legs = {}
    # inputs and their compression are prepared outside the timed region
    comp_t, comp_n = 0.0, 0
    while t_total < seconds and done < n_slices:
        k, v = G.kv_slice(w, "k", b, h), G.kv_slice(w, "v", b, h)
        q = np.stack([G.window_q(w, b, h * grp + j)[0] for j in range(grp)])
        kw, vw = G.window_kv(w, "k", b, h)[:1], G.window_kv(w, "v", b, h)[:1]
        if w.method == "quant":
            t0 = time.perf_counter()
            c = OQ.compress_slice(k, v, w.k_bits, w.v_bits, w.group, w.scale_dtype)
            if comp_n < 2:                                   # the compress leg: two slices
                comp_t += time.perf_counter() - t0
                comp_n += 1
            t0 = time.perf_counter()
            kh, vh = OQ.dequantize_slice(c, w.d, w.k_bits, w.v_bits, w.group)
            OA.decode(q, kh[None], vh[None], w.d ** -0.5, kw[None], vw[None])
        else:
            t0 = time.perf_counter()
            nk = OD.n_keep(w.N, w.keep_ratio)   # same work as decoding the kept rows
            OA.decode(q, k[None, :nk], v[None, :nk], w.d ** -0.5, kw[None], vw[None])
        t_total += time.perf_counter() - t0
        done += 1
        h += 1
        if h == w.Hkv:
            h, b = 0, b + 1
    if comp_n:
        in_bytes = 2 * w.N * w.d * (4 if w.dtype == "f32" else 2)
        legs["compress"] = {"GBps": round(comp_n * in_bytes / comp_t / 1e9, 4),
                            "whole_workload_s": round(comp_t / comp_n * n_slices, 2),
                            "sample": f"quantize + pack {comp_n} of {n_slices} slices ({w.N} tokens each); "
                                      f"whole workload extrapolated"}
    # verify: the window of one (sequence, kv-head) over its full context, every q-head
    k, v = G.kv_slice(w, "k", 0, 0), G.kv_slice(w, "v", 0, 0)
    qw = np.stack([G.window_q(w, 0, j) for j in range(grp)])
    kw, vw = G.window_kv(w, "k", 0, 0), G.window_kv(w, "v", 0, 0)
    t0 = time.perf_counter()
    OA.verify_masked(qw, k[None], v[None], kw[None], vw[None], w.d ** -0.5)
    t_v = time.perf_counter() - t0
    slice_flops = verify_flops(w, w.N) / n_slices
    legs["verify"] = {"TFLOPs": round(slice_flops / t_v / 1e12, 5), "whole_workload_s": round(t_v * n_slices, 2),
                      "sample": f"1 of {n_slices} slices: {grp} q-heads x {w.k} window rows over {w.N} + {w.k} "
                                f"positions; whole workload extrapolated"}
    # accept: the batch's drafts against targets
    rng = np.random.default_rng(5)
    dr = rng.integers(0, 3, size=(w.B, w.k))
    tg = rng.integers(0, 3, size=(w.B, w.k))
    t0 = time.perf_counter()
    reps = 200
    for _ in range(reps):
        for bb in range(w.B):
            OC.accept_row(list(dr[bb]), list(tg[bb]))
    legs["accept"] = {"us_per_call": round((time.perf_counter() - t0) / reps * 1e6, 2),
                      "sample": f"{w.B} sequences x window {w.k}, {reps} calls"}
    # one draft-and-verify round of the end-to-end decoder (float64) at a reduced prompt
    e = Cfg.E2E
    P = 256
    cfg = OM.Config(layers=e.layers, d_model=e.d_model, Hq=e.Hq, Hkv=e.Hkv, hd=e.d, ffn=e.ffn, vocab=e.vocab)
    dec = OM.Decoder(cfg, OM.random_weights(cfg, np.random.default_rng(7)))
    prompt = G.tokens(e, 0, shape=(P,), high=e.vocab)
    run = lambda T, st=None: OM.vericache(dec, prompt, T, e.k, bits=(e.k_bits, e.v_bits), group=e.group,
                                          scale_dtype="f32", stats=st)
    run(1)                                                  # warm: the prefill and prompt compression only
    t0 = time.perf_counter()
    run(1)
    t_pre = time.perf_counter() - t0
    st = OM.RoundStats()
    t0 = time.perf_counter()
    run(2, st)                                              # the same, then one round
    t_round = time.perf_counter() - t0 - t_pre
    legs["round"] = {"round_s": round(t_round, 2), "rounds": st.rounds,
                     "sample": f"decoder {e.layers}L d_model {e.d_model}, 1 sequence, prompt {P} tokens "
                               f"(reduced from the end-to-end workload's), k {e.k}: {e.k} draft steps on the "
                               f"compressed cache, the verify pass, acceptance and the cache update (a run to "
                               f"two tokens minus a run to one)"}
    if limit is not None:
        limit.restore_original_limits()
    return {"value": round(done * per_slice / t_total / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(), "cores_visible": cores,
            "sample": f"{done} of {n_slices} (sequence, kv-head) slices: {'dequantize + ' if w.method == 'quant' else ''}"
                      f"decode of {grp} q-heads over {w.N} tokens, {t_total:.1f}s of CPU time; "
                      f"{'extrapolated to the whole workload' if done < n_slices else 'the whole workload'}",
            "legs": legs}


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the hot path is measured on a single MI355X "
              "(per-(sequence, kv-head) sharding needs no collectives; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch
    w = workload(a.workload)
    torch.cuda.set_device(0)
    if a.copy_calibration:
        n = a.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    st = setup(w, a.copies)
    graph = capture_draft(st)
    for _ in range(a.warmup):
        run_step(st, graph=graph)
    torch.cuda.synchronize()

    mk = lambda: torch.cuda.Event(enable_timing=True)
    evs = [[mk() for _ in range(4)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        run_step(st, evs[s], graph)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    state = gpu_state()  # right after the timed region
    # each decode call on its own, launched eagerly between HIP events (the spread of
    # single calls; the roofline takes the graph-replayed calls of the timed region)
    dec = [[(mk(), mk()) for _ in range(w.k)] for _ in range(a.steps)]
    for s in range(a.steps):
        draft_calls(st, dec[s])
    torch.cuda.synchronize()
    draft_ms = sum(e[0].elapsed_time(e[1]) for e in evs)
    verify_ms = sum(e[1].elapsed_time(e[2]) for e in evs)
    tok_ms = sum(e[2].elapsed_time(e[3]) for e in evs)
    step_ms = sum(e[0].elapsed_time(e[3]) for e in evs) / a.steps
    dec_launch_ms = [p[0].elapsed_time(p[1]) for d in dec for p in d]
    # average duration of one decode call in the timed region: the draft phase (HIP
    # events on the stream the graph is replayed on) over its k calls
    dec_avg_ms = draft_ms / a.steps / w.k

    # algorithmic work: draft step i reads the compressed context plus i + 1 tail rows
    n_ctx = st["ckvs"][0].n_main
    dbytes = sum(decode_bytes(w, n_ctx, i + 1) for i in range(w.k))
    decode_gbs = dbytes * a.steps / (draft_ms * 1e-3) / 1e9
    per_launch = dbytes / w.k
    achieved = per_launch / (dec_avg_ms * 1e-3) / 1e9
    vflops = verify_flops(w, w.N)
    verify_tflops = vflops * a.steps / (verify_ms * 1e-3) / 1e12
    verify_gbs = verify_bytes(w, w.N) * a.steps / (verify_ms * 1e-3) / 1e9
    accepted = int(st["nc"].sum().item())
    acc_len = st["acc"].float().mean().item()

    line = {
        "metric": METRIC, "value": round(decode_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "global_batch": w.B, "seq_len": w.N, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.d, "draft_window": w.k, "compressor": (
                       f"KIVI-style K{w.k_bits}/V{w.v_bits} group {w.group}" if w.method == "quant"
                       else f"top-{w.keep_ratio:g} accumulated attention, {w.n_probes} probes"),
                   "parallelism": "none (1 GPU)", "cache_copies_rotated": a.copies},
        "verify_attn_tflops": round(verify_tflops, 2),
        "verify_attn_hbm_gbs": round(verify_gbs, 1),
        "verify_mfma_frac": round(verify_tflops / BF16_PEAK_TFLOPS, 4),
        # roofline of the verify pass: arithmetic intensity (algorithmic flops per byte of
        # the full cache), the attainable rate min(MFMA peak, AI x HBM peak), and the
        # fraction of it reached
        "verify_roofline": {"ai_flop_per_byte": round(vflops / verify_bytes(w, w.N), 1),
                            "attainable_tflops": round(min(BF16_PEAK_TFLOPS, vflops / verify_bytes(w, w.N) *
                                                           HBM_PEAK_GBS / 1e3), 1),
                            "frac_of_attainable": round(verify_tflops / min(BF16_PEAK_TFLOPS, vflops / verify_bytes(
                                w, w.N) * HBM_PEAK_GBS / 1e3), 4)},
        "decode_call_us": {"graph_replay_mean": round(dec_avg_ms * 1e3, 3),
                           "eager": spread([x * 1e3 for x in dec_launch_ms])},
        "verify_call_us": spread([e[1].elapsed_time(e[2]) * 1e3 for e in evs]),
        "gpu_state": state,
        "kernel_round_accepted_tok_per_s": round(accepted / (step_ms * 1e-3), 1),
        "mean_accept_len": round(acc_len, 3),
        "draft_replay": f"HIP graph of the {w.k} decode calls",
        "phase_ms": {"draft": round(draft_ms / a.steps, 4), "verify": round(verify_ms / a.steps, 4),
                     "tokens_accept": round(tok_ms / a.steps, 4)},
        "wall_ms_per_step": round(wall / a.steps * 1e3, 4),
        "compress_ms": round(st["comp_ms"], 4),
        "roofline": {"bound": "hbm", "kernel": "decode_mfma_kernel + decode_merge_kernel (quant)" if w.method == "quant"
                     else "decode_dense_kernel + decode_merge_kernel (kept rows)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name),
                     "bytes_per_launch": int(per_launch), "avg_launch_us": round(dec_avg_ms * 1e3, 3)},
    }
    line["verify_mfma_shape"] = verify_mfma_shape() if w.name != workload("qwen30b").name else None
    line["rotation_prepass"] = measure_rotation(st)
    line["split_stream"] = measure_split_stream(st)
    if not a.no_stage:
        line["stage_full_kv"] = measure_stage(st)
    if not a.no_e2e:
        del st
        torch.cuda.empty_cache()
        line["e2e"] = e2e_rounds(a.e2e_ctx, a.e2e_gen, a.e2e_slots, remote=not a.no_remote_prefix)
        line["accepted_tok_per_s"] = line["e2e"]["accepted_tok_per_s"]
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
