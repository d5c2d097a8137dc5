"""Benchmark: wave-index decode attention on one MI355X.

Workload: the Llama3.1-8B-shaped layer at 128K context (32 query / 8 KV heads,
head_dim 128, bf16, batch 1, 16 segments x 8K tokens, 512 clusters per
segment, retrieval 1.8 %, estimation 23 %, steady 4 + 64), seeded synthetic
clustered keys (see sparse_long_context_segmented_amd/synth.py).

A timed step is one wi_decode_attention call (score, select, gather + exact
attention, estimation, merge) for every sequence of the batch; value =
decode queries per second per layer (batch / step time). Inputs (the index
built by wi_build_index from the seeded K/V, and the queries) are resident in
HBM before timing; steps rotate over R copies of the index at distinct
addresses so the 256 MB last-level cache cannot serve repeated steps. The
index build is timed in the same run and reported beside it ("build").

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_llama8b_128k_b1_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_long_context_segmented_amd", "csrc", f)
                  for f in ("decode_fused.hip", "decode_score.hip", "wi_internal.h")]
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b-128k-b1")
    ap.add_argument("--instances", type=int, default=32,
                    help="index copies the steps rotate over")
    ap.add_argument("--build-reps", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="bound on the oracle's timed decode loop")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-wb", action="store_true", help="skip the wave-buffer leg")
    ap.add_argument("--policy", default="uniform", choices=["uniform", "dense-first2", "banded"],
                    help="per-layer zone policy of a multi-layer model (wi_layer_plan)")
    ap.add_argument("--wg", type=int, default=0,
                    help="fused-kernel workgroups per (sequence, KV head); 0 = automatic")
    ap.add_argument("--profile", action="store_true",
                    help="short run for rocprofv3 (no CPU leg, few steps)")
    return ap.parse_args()


def measured_traffic(workload):
    """HBM bytes per launch of the select/attend kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by a copy kernel), or
    None when that summary is for another workload or for other kernel
    sources than the ones built here."""
    if workload != "llama8b-128k-b1" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    import hashlib
    line = [x for x in open(TRAFFIC_PROFILE) if x.startswith("traffic: ")]
    if not line:
        return None
    rec = json.loads(line[0][len("traffic: "):])
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    if h.hexdigest()[:16] != rec.get("sources_sha256"):
        return None
    return int(rec["bytes"])


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {a.gpus} is not supported "
              "(the path shards by KV head / sequence with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_long_context_segmented_amd import synth, wi

    w = next(x for x in synth.WORKLOADS if x.name == a.workload)
    if w.layers > 1:
        return model_bench(a, w)
    if a.profile:
        a.steps, a.warmup, a.no_cpu, a.build_reps = min(a.steps, 20), 5, True, 1
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    # ---- inputs: seeded synthetic K, V, q (host), then resident in HBM ----
    t0 = time.time()
    K, V, q = synth.gen_batch(w)
    gen_s = time.time() - t0
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    kt = torch.from_numpy(K).to(dev, dt)
    vt = torch.from_numpy(V).to(dev, dt)
    qt = torch.from_numpy(q).to(dev, dt)
    desc = wi.make_desc(w.dtype, w.batch, w.n_kv_heads, w.n_ctx, seg_len=w.seg_len,
                        clusters_per_seg=w.clusters_per_seg, n_iters=w.n_iters)
    ns, C, cap, wsb = wi.index_sizes(desc)
    U = w.batch * w.n_kv_heads
    e = 2 if w.dtype == "bf16" else 4

    # ---- build leg ----
    ws_build = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ix = wi.alloc_index(desc, dev)
    wi.build_index(desc, kt, vt, index=ix, ws=ws_build)  # warm
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    build_ms = []
    for _ in range(a.build_reps):
        ev0.record(stream)
        wi.build_index(desc, kt, vt, index=ix, ws=ws_build)
        ev1.record(stream)
        torch.cuda.synchronize()
        build_ms.append(ev0.elapsed_time(ev1))
    wi.timing_start()
    wi.build_index(desc, kt, vt, index=ix, ws=ws_build)
    brec = wi.timing_stop()
    bk = {}
    for name, ms in brec:
        bk.setdefault(name, []).append(ms)
    n_assign = len(bk.get("assign", []))
    assign_ms = float(np.mean(bk["assign"])) if n_assign else float("nan")
    # assignment FLOPs per launch: 2 * n_s * C_s * 128 summed over segments
    seg_n = [min(w.seg_len, (w.n_ctx - 68) - s * w.seg_len) for s in range(ns)]
    flops = sum(2.0 * n * min(w.clusters_per_seg, n) * 128 for n in seg_n) * U
    peak_mfma = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    assign_tflops = flops / (assign_ms * 1e-3) / 1e12
    # the whole assignment step: the MFMA kernel plus its exact fallback
    fix_ms = float(np.mean(bk["assign_fix"])) if bk.get("assign_fix") else 0.0
    step_tflops = flops / ((assign_ms + fix_ms) * 1e-3) / 1e12
    build = {
        "ms": round(float(np.median(build_ms)), 3),
        "phase_ms": {k: round(float(np.sum(v)), 3) for k, v in bk.items()},
        "assign": {"bound": "mfma", "achieved": round(assign_tflops, 2),
                   "peak": peak_mfma, "unit": "TFLOP/s",
                   "frac": round(assign_tflops / peak_mfma, 4),
                   "ms_per_launch": round(assign_ms, 4), "launches": n_assign,
                   "fix_ms_per_launch": round(fix_ms, 4),
                   "step_achieved": round(step_tflops, 2),
                   "step_frac": round(step_tflops / peak_mfma, 4)},
    }
    # ---- a dense layer of the same shape (the per-layer policy's full-
    # attention layers): every token read once per query ----
    ddn = wi.DecodeDesc(w.n_q_heads, 0, 0, 0.0)
    wsdn = torch.empty(max(wi.dense_sizes(desc, ddn), 16), dtype=torch.uint8, device=dev)
    outd = torch.empty(w.batch, w.n_q_heads, 128, dtype=torch.float32, device=dev)
    for _ in range(3):
        wi.dense_attention(desc, ddn, kt, vt, qt, out=outd, ws=wsdn)
    dense_reps = 20
    ev0.record(stream)
    for _ in range(dense_reps):
        wi.dense_attention(desc, ddn, kt, vt, qt, out=outd, ws=wsdn)
    ev1.record(stream)
    torch.cuda.synchronize()
    dense_ms = ev0.elapsed_time(ev1) / dense_reps
    wi.timing_start()
    for _ in range(dense_reps):
        wi.dense_attention(desc, ddn, kt, vt, qt, out=outd, ws=wsdn)
    drec = wi.timing_stop()
    dk = {}
    for name, ms in drec:
        dk.setdefault(name, []).append(ms)
    dense_kernel_ms = float(np.mean(dk["dense"]))
    dense_bytes = U * w.n_ctx * 128 * e * 2 + w.batch * w.n_q_heads * 128 * (e + 4)
    dense_gbs = dense_bytes / (dense_kernel_ms * 1e-3) / 1e9
    policy = {"dense_layer": {
        "ms_per_call": round(dense_ms, 4), "queries_per_s": round(w.batch / (dense_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "dense", "achieved": round(dense_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dense_gbs / PEAK_HBM_GBS, 4),
                     "kernel_ms": {k: round(float(np.mean(v)), 5) for k, v in dk.items()},
                     "algorithmic_bytes": int(dense_bytes)}}}
    del kt, vt, ws_build, wsdn

    # ---- decode: R index copies at distinct addresses ----
    k_r, k_e = w.budgets()
    dd = wi.DecodeDesc(w.n_q_heads, k_r, k_e, 0.0, a.wg)
    nexe = torch.empty(U, dtype=torch.int32, device=dev)
    sel = torch.empty(U, k_r + min(k_e, C - k_r), dtype=torch.int32, device=dev)
    wi.decode_attention(ix, dd, qt, n_exec=nexe, sel_ids=sel)
    torch.cuda.synchronize()
    retrieved = int((nexe.cpu().numpy() - 68).sum())  # sum over units of sum_R n_c
    # index-quality diagnostic: recall@100 of each query head's retrieval zone
    k_rec = min(100, w.n_ctx - 68)
    rec = wi.recall_at_k(ix, dd, qt, sel, k_r, k_rec).cpu().numpy()
    policy["recall_at_100"] = {"k": k_rec, "min": round(float(rec.min()), 4),
                               "mean": round(float(rec.mean()), 4),
                               "query_heads": int(rec.size)}
    del sel
    copies = [ix]
    for _ in range(a.instances - 1):
        copies.append(wi.Index(desc, *[getattr(ix, f).clone() for f in (
            "centroids", "cluster_size", "value_sum", "block_off", "k_blocks", "v_blocks",
            "slot_token", "steady_k", "steady_v", "assign")]))
    wsd = torch.empty(wi.decode_sizes(desc, dd), dtype=torch.uint8, device=dev)
    outs = [torch.empty(w.batch, w.n_q_heads, 128, dtype=torch.float32, device=dev)
            for _ in range(len(copies))]
    # warm-up on copies 0 .. warmup-1; the timed steps continue from copy
    # `warmup`, so a warm-up copy is read again only after R - warmup other
    # copies (R x the step's bytes far exceeds the 256 MB last-level cache)
    for i in range(a.warmup):
        wi.decode_attention(copies[i % len(copies)], dd, qt, out=outs[i % len(copies)], ws=wsd)
    torch.cuda.synchronize()
    ev0.record(stream)
    t_start = time.perf_counter()
    for i in range(a.steps):
        j = (a.warmup + i) % len(copies)
        wi.decode_attention(copies[j], dd, qt, out=outs[j], ws=wsd)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = ev0.elapsed_time(ev1) / a.steps

    # per-step distribution: HIP events around each of the steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    for i in range(a.steps):
        j = i % len(copies)
        evs[i][0].record(stream)
        wi.decode_attention(copies[j], dd, qt, out=outs[j], ws=wsd)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    step_pct = {"p10": round(float(np.percentile(per_step, 10)), 5),
                "p50": round(float(np.percentile(per_step, 50)), 5),
                "p90": round(float(np.percentile(per_step, 90)), 5)}

    # the same steps replayed from a HIP graph (one decode call per index copy,
    # captured once): launch overhead between the two kernels of a step
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(len(copies)):
            wi.decode_attention(copies[j], dd, qt, out=outs[j], ws=wsd)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, a.steps // len(copies))
    ev0.record(stream)
    for _ in range(reps):
        graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    graph_step_ms = ev0.elapsed_time(ev1) / (reps * len(copies))
    del graph

    # per-kernel durations over the same number of steps (timing hook)
    wi.timing_start()
    for i in range(a.steps):
        j = i % len(copies)
        wi.decode_attention(copies[j], dd, qt, out=outs[j], ws=wsd)
    recs = wi.timing_stop()
    kt_ms = {}
    for name, ms in recs:
        kt_ms.setdefault(name, []).append(ms)
    avg = {k: float(np.mean(v)) for k, v in kt_ms.items()}

    # algorithmic bytes per step (each unit): centroids, E value sums, metadata,
    # retrieved K/V (measured sum of R cluster sizes), steady K/V, q, out
    G = w.group
    k_e_eff = min(k_e, C - k_r)
    b_score = U * (C * 128 * e + G * 128 * e)
    b_attend = (U * (k_e_eff * 128 * 4 + (k_r + k_e_eff) * 4 + k_r * 8 + 68 * 128 * e * 2)
                + retrieved * 128 * e * 2)
    b_out = U * G * 128 * 4
    step_bytes = b_score + b_attend + b_out
    # score streams the centroids; select_attend gathers the retrieval zone,
    # reads the estimation clusters' value sums and writes the output
    per_kernel = {"score": b_score, "select_attend": b_attend + b_out}
    # the dominant kernel among those that move the method's HBM bytes
    dom = max((k for k in avg if per_kernel.get(k, 0) > 0), key=lambda k: avg[k])
    dom_bytes = per_kernel.get(dom, 0)
    achieved = dom_bytes / (avg[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(w.name),
                "kernel_ms": {k: round(v, 5) for k, v in avg.items()},
                "algorithmic_bytes": {k: int(v) for k, v in per_kernel.items()}}

    # ---- wave buffer: the same index with its K/V blocks in pinned host
    # memory behind a GPU block cache, on a drifting query stream ----
    wave = wave_buffer_leg(w, desc, ix, dd, qt, q, a.steps, a.warmup) if not a.no_wb else None

    qps = w.batch * a.steps / (step_ms * a.steps * 1e-3)
    res = {
        "metric": "decode attention queries/s per layer at 128K ctx; achieved HBM GB/s vs peak",
        "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.n_ctx,
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": 128,
                   "seg_len": w.seg_len, "clusters_per_seg": w.clusters_per_seg,
                   "k_retrieve": k_r, "k_estimate": k_e_eff, "index_copies": len(copies)},
        "step_hbm_GBps": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
        "ms_per_step_bracketed": step_pct,
        "graph_replay": {"ms_per_step": round(graph_step_ms, 5),
                         "queries_per_s": round(w.batch / (graph_step_ms * 1e-3), 1)},
        "step_bytes": int(step_bytes),
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "build": build,
        "policy": policy,
        "wave_buffer": wave,
        "gen_s": round(gen_s, 1),
    }

    if not a.no_cpu:
        # every unit of the layer when the oracle builds them in about half a
        # minute on the host (the 128K batch-1 layer); otherwise the units of
        # the first sequence, scaled to the whole batch
        U1 = w.n_kv_heads if w.batch > 1 else U
        res["cpu_baseline"] = cpu_baseline(w, K, V, q, k_r, k_e, a.cpu_seconds,
                                           units=list(range(U1)))
    print(json.dumps(res), flush=True)


def model_bench(a, w):
    """A whole multi-layer model (the 32-layer 1M-token Llama3-8B-1048K shape):
    every layer's index is built and stays resident in HBM (about 213 GB for
    32 layers x 8 KV heads), then a decode step is one wi_decode_attention
    call per layer. The raw K/V of each layer (4.3 GB) is drawn on the GPU
    (synth.gen_layer_device), built into its index, and freed. value =
    layer-queries/s (batch x layers / step time), the per-layer decode rate."""
    import torch
    from sparse_long_context_segmented_amd import synth, wi

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    L, U, e = w.layers, w.batch * w.n_kv_heads, (2 if w.dtype == "bf16" else 4)
    steps = min(a.steps, 20) if a.steps == 200 else a.steps
    warmup = min(a.warmup, 3)
    descs = [wi.make_desc(w.dtype, w.batch, w.n_kv_heads, w.n_ctx, seg_len=w.seg_len,
                          clusters_per_seg=w.clusters_per_seg, n_iters=w.n_iters, layer_id=l)
             for l in range(L)]
    # the per-layer plan: dense layers keep their raw K/V and build no index
    pol = {"uniform": wi.WI_POLICY_UNIFORM, "dense-first2": wi.WI_POLICY_DENSE_FIRST2,
           "banded": wi.WI_POLICY_BANDED}[a.policy]
    plans = [wi.layer_plan(pol, l, L, w.n_ctx, w.seg_len, w.clusters_per_seg) for l in range(L)]
    dense = [p[0] == wi.WI_LAYER_DENSE for p in plans]
    raw = {}
    ns, C, cap, wsb = wi.index_sizes(descs[0])
    ws_build = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    indexes, qs, build_ms, gen_ms = [], [], [], []
    bk = {}
    for l in range(L):
        g0 = time.perf_counter()
        K, V, q = synth.gen_layer_device(w, l, dev)
        torch.cuda.synchronize()
        gen_ms.append((time.perf_counter() - g0) * 1e3)
        if dense[l]:
            raw[l] = (K, V)
            indexes.append(None)
            qs.append(q)
            print(f"layer {l}: dense (raw K/V kept)", file=sys.stderr, flush=True)
            continue
        ix = wi.alloc_index(descs[l], dev)
        if l == L - 1:
            wi.timing_start()
        ev0.record(stream)
        wi.build_index(descs[l], K, V, index=ix, ws=ws_build)
        ev1.record(stream)
        torch.cuda.synchronize()
        if l == L - 1:
            for name, ms in wi.timing_stop():
                bk.setdefault(name, []).append(ms)
        build_ms.append(ev0.elapsed_time(ev1))
        if l == L - 1 and not a.no_cpu:
            # unit (b=0, h=0) of the last layer, for the oracle's baseline
            host0 = (K[:1, :1].float().cpu().numpy(), V[:1, :1].float().cpu().numpy(),
                     q[:1, :w.group].float().cpu().numpy())
        del K, V
        indexes.append(ix)
        qs.append(q)
        print(f"layer {l}: built in {build_ms[-1]:.1f} ms", file=sys.stderr, flush=True)
    del ws_build

    k_r, k_e = w.budgets()
    dd = wi.DecodeDesc(w.n_q_heads, k_r, k_e, 0.0, a.wg)
    dds = [wi.DecodeDesc(w.n_q_heads, p[1], p[2], 0.0, a.wg) for p in plans]
    ddn = wi.DecodeDesc(w.n_q_heads, 0, 0, 0.0)
    wsd = torch.empty(max([wi.decode_sizes(descs[0], x) for x, d_ in zip(dds, dense) if not d_]
                          + [16]), dtype=torch.uint8, device=dev)
    wsdn = torch.empty(max(wi.dense_sizes(descs[0], ddn), 16), dtype=torch.uint8, device=dev)
    outs = [torch.empty(w.batch, w.n_q_heads, 128, dtype=torch.float32, device=dev)
            for _ in range(L)]
    nexe = torch.zeros(L, U, dtype=torch.int32, device=dev) + 68
    for l in range(L):
        if dense[l]:
            wi.dense_attention(descs[l], ddn, *raw[l], qs[l], out=outs[l], ws=wsdn)
        else:
            wi.decode_attention(indexes[l], dds[l], qs[l], out=outs[l], n_exec=nexe[l], ws=wsd)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(o).all()) for o in outs), "non-finite decode output"
    retrieved = int((nexe.cpu().numpy() - 68).sum())  # over hybrid layers and units

    def step():
        for l in range(L):
            if dense[l]:
                wi.dense_attention(descs[l], ddn, *raw[l], qs[l], out=outs[l], ws=wsdn)
            else:
                wi.decode_attention(indexes[l], dds[l], qs[l], out=outs[l], ws=wsd)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    step_ms = ev0.elapsed_time(ev1) / steps
    wi.timing_start()
    for _ in range(2):
        step()
    recs = wi.timing_stop()
    kt_ms = {}
    for name, ms in recs:
        kt_ms.setdefault(name, []).append(ms)
    avg = {k: float(np.mean(v)) for k, v in kt_ms.items()}

    G = w.group
    k_e_eff = min(k_e, C - k_r)
    # algorithmic bytes per launch (one layer), averaged over the hybrid
    # layers; a dense layer reads every token's K and V
    Lh = sum(1 for d_ in dense if not d_)
    ke_l = [min(p[2], C - p[1]) for p, d_ in zip(plans, dense) if not d_]
    kr_l = [p[1] for p, d_ in zip(plans, dense) if not d_]
    b_score = U * (C * 128 * e + G * 128 * e)
    b_attend = (sum(U * (ke * 128 * 4 + (kr + ke) * 4 + kr * 8 + 68 * 128 * e * 2 + G * 128 * 4)
                    for kr, ke in zip(kr_l, ke_l)) + retrieved * 128 * e * 2) / max(Lh, 1)
    b_dense = U * w.n_ctx * 128 * e * 2 + w.batch * w.n_q_heads * 128 * (e + 4)
    per_kernel = {"score": b_score, "select_attend": b_attend, "dense": b_dense}
    dom = max((k for k in avg if per_kernel.get(k, 0) > 0), key=lambda k: avg[k] * (
        (L - Lh) if k == "dense" else Lh))
    achieved = per_kernel[dom] / (avg[dom] * 1e-3) / 1e9
    step_bytes = Lh * (b_score + b_attend) + (L - Lh) * b_dense
    seg_n = [min(w.seg_len, (w.n_ctx - 68) - s_ * w.seg_len) for s_ in range(ns)]
    flops = sum(2.0 * n * min(w.clusters_per_seg, n) * 128 for n in seg_n) * U
    assign_ms = float(np.mean(bk["assign"]))
    res = {
        "metric": "decode attention queries/s per layer at 128K ctx; achieved HBM GB/s vs peak",
        "value": round(w.batch * L / (step_ms * 1e-3), 1), "unit": "layer-queries/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (drawn on the GPU)",
        "config": {"workload": w.name, "batch": w.batch, "layers": L, "seq_len": w.n_ctx,
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": 128,
                   "seg_len": w.seg_len, "clusters_per_seg": w.clusters_per_seg,
                   "k_retrieve": k_r, "k_estimate": k_e_eff, "policy": a.policy,
                   "dense_layers": [l for l in range(L) if dense[l]],
                   "estimate_clusters_per_layer": [p[2] for p in plans]},
        "step_hbm_GBps": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
        "step_bytes": int(step_bytes),
        "resident_GB": round(torch.cuda.memory_allocated(dev) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel_ms": {k: round(v, 5) for k, v in avg.items()},
                     "algorithmic_bytes": {k: int(v) for k, v in per_kernel.items()}},
        "build": {"ms_total": round(float(np.sum(build_ms)), 1),
                  "ms_per_layer": round(float(np.mean(build_ms)), 2),
                  "layers_built": len(build_ms),
                  "phase_ms_last_layer": {k: round(float(np.sum(v)), 3) for k, v in bk.items()},
                  "assign": {"bound": "mfma",
                             "achieved": round(flops / (assign_ms * 1e-3) / 1e12, 2),
                             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(flops / (assign_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                             "ms_per_launch": round(assign_ms, 4)}},
        "gen_ms_per_layer": round(float(np.mean(gen_ms)), 1),
    }
    if not a.no_cpu:
        # one unit, (b=0, h=0) of the last layer: with a single KV head its
        # random stream is that unit's, so the oracle builds exactly it
        import dataclasses
        w1 = dataclasses.replace(w, n_kv_heads=1, n_q_heads=w.group, layers=1)
        res["cpu_baseline"] = cpu_baseline(w1, *host0, k_r, k_e, a.cpu_seconds, units=[0],
                                           layer=L - 1, units_per_step=L * U,
                                           queries_per_step=w.batch * L)
        del host0
    print(json.dumps(res), flush=True)


def wave_buffer_leg(w, desc, ix, dd, qt, q, steps, warmup, fracs=(0.05, 0.10, 0.20)):
    """Decode through the wave buffer (K/V blocks in pinned host memory, a GPU
    cache of a fraction of the used blocks per unit) on a seeded drifting
    query stream: hit rate, misses per step and the step time, beside the
    HBM-resident decode of the same queries."""
    import torch
    from sparse_long_context_segmented_amd import synth, wi
    dev = qt.device
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(1234)
    cur, qs = q.copy(), []
    for _ in range(warmup + steps):
        cur = cur + 0.35 * rng.standard_normal(q.shape).astype(np.float32)
        qs.append(torch.from_numpy(synth._round_to_dtype(0.8 * cur + 0.2 * q, w.dtype))
                  .to(dev, qt.dtype))
    hix = wi.host_tier(ix)
    U = w.batch * w.n_kv_heads
    used = int(ix.block_off[:, -1].max())
    e = 2 if w.dtype == "bf16" else 4
    T = 2048 // (128 * e)
    out = torch.empty(w.batch, w.n_q_heads, 128, dtype=torch.float32, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the HBM-resident decode of the same stream
    wsd = torch.empty(wi.decode_sizes(desc, dd), dtype=torch.uint8, device=dev)
    for i in range(warmup):
        wi.decode_attention(ix, dd, qs[i], out=out, ws=wsd)
    ev0.record(stream)
    for i in range(warmup, warmup + steps):
        wi.decode_attention(ix, dd, qs[i], out=out, ws=wsd)
    ev1.record(stream)
    torch.cuda.synchronize()
    res = {"queries": "seeded random walk of the workload's queries (step 0.35, pulled 20 % "
                      "back to the start)",
           "hbm_ms_per_step": round(ev0.elapsed_time(ev1) / steps, 5), "caches": []}
    for frac in fracs:
        S = max(1, min(8192, int(frac * used)))
        wb = wi.alloc_wave_buffer(desc, S, dev)
        ws = torch.empty(wi.decode_wb_sizes(desc, dd, S), dtype=torch.uint8, device=dev)
        # rows padded to an even unit count: each step's [U, 2] slice starts 16-byte aligned
        stats = torch.zeros(warmup + steps, U + U % 2, 2, dtype=torch.int32, device=dev)
        for i in range(warmup):
            wi.decode_attention_wb(hix, dd, wb, i + 1, qs[i], out=out, stats=stats[i], ws=ws)
        ev0.record(stream)
        for i in range(warmup, warmup + steps):
            wi.decode_attention_wb(hix, dd, wb, i + 1, qs[i], out=out, stats=stats[i], ws=ws)
        ev1.record(stream)
        torch.cuda.synchronize()
        st = stats[warmup:, :U].cpu().numpy().astype(np.int64)
        hits, misses = int(st[:, :, 0].sum()), int(st[:, :, 1].sum())
        # kernel durations of the same steps replayed on a second cache (the
        # timing hook's events would perturb the timed loop above)
        wb2 = wi.alloc_wave_buffer(desc, S, dev)
        for i in range(warmup):
            wi.decode_attention_wb(hix, dd, wb2, i + 1, qs[i], out=out, ws=ws)
        wi.timing_start()
        for i in range(warmup, warmup + steps):
            wi.decode_attention_wb(hix, dd, wb2, i + 1, qs[i], out=out, ws=ws)
        kk = {}
        for name, ms in wi.timing_stop():
            kk.setdefault(name, []).append(ms)
        del wb2
        res["caches"].append({
            "slots_per_unit": S, "fraction_of_blocks": round(S / used, 4),
            "cache_MB": round(2 * U * S * T * 128 * e / 1e6, 1),
            "hit_rate": round(hits / max(1, hits + misses), 4),
            "misses_per_step": round(misses / steps, 1),
            "host_read_MB_per_step": round(misses / steps * 2 * 2 * T * 128 * e / 1e6, 3),
            "ms_per_step": round(ev0.elapsed_time(ev1) / steps, 5),
            "kernel_ms": {k: round(float(np.mean(v)), 5) for k, v in kk.items()}})
        del wb, ws
    del hix
    return res


def cpu_baseline(w, K, V, q, k_r, k_e, seconds, units, layer=0, units_per_step=None,
                 queries_per_step=None):
    """The oracle, untuned, on the host cores, on a bounded sample of the same
    workload: the sampled units (b, h) of one layer are built in one oracle
    call (OpenMP over the (unit, segment) jobs) and then decoded in one call
    (OpenMP over the units), repeatedly for about `seconds`. K, V: host arrays
    [B, H, N, 128] holding at least the sampled units' sequences. A decode
    step covers units_per_step units (default: every unit of the layer); when
    the sample holds fewer, the time is scaled by units_per_step / sample and
    marked extrapolated (units are independent). value = queries_per_step
    (default: the batch) / step time."""
    import oracle
    oracle.compile_oracle()
    threads = oracle.num_threads()
    H, G = w.n_kv_heads, w.group
    U = units_per_step or w.batch * H
    bmax = max(units) // H + 1
    od = oracle.make_desc(w.dtype, bmax, H, w.n_ctx, seg_len=w.seg_len,
                          clusters_per_seg=w.clusters_per_seg, n_iters=w.n_iters,
                          layer_id=layer)
    ns = oracle.sizes(od)[0]
    t0 = time.perf_counter()
    idx = oracle.build(od, K[:bmax], V[:bmax], units=units)
    build_s = time.perf_counter() - t0
    sub = {k: np.ascontiguousarray(v[list(units)]) for k, v in idx.items()}
    del idx
    # the sampled units' query heads, as one sequence of len(units) KV heads
    qs = np.concatenate([q[u // H, (u % H) * G:(u % H + 1) * G] for u in units])[None]
    od1 = oracle.make_desc(w.dtype, 1, len(units), w.n_ctx, seg_len=w.seg_len,
                           clusters_per_seg=w.clusters_per_seg, n_iters=w.n_iters)
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode(od1, G * len(units), k_r, k_e, sub, qs)
        n += 1
        if time.perf_counter() - t0 > seconds:
            break
    sample_step = (time.perf_counter() - t0) / n
    factor = U / len(units)
    step = sample_step * factor
    qps = queries_per_step or w.batch
    return {"value": round(qps / step, 3),
            "unit": "queries/s" if queries_per_step is None else "layer-queries/s",
            "cores": min(threads, len(units)), "kind": "oracle",
            "sample": (f"{len(units)} of {U} units per step (b, h) = "
                       f"{[divmod(u, H) for u in units][:8]}{'...' if len(units) > 8 else ''}: "
                       f"oracle build of those units in one call ({build_s:.1f} s, "
                       f"{min(threads, len(units) * ns)} threads), then {n} decode calls over "
                       f"them ({min(threads, len(units))} threads, one per unit)"
                       + (f"; step time scaled x{factor:g} (extrapolated)" if factor != 1 else "")),
            "extrapolated": factor != 1,
            "decode_ms_per_step": round(step * 1e3, 3),
            "decode_ms_sample": round(sample_step * 1e3, 3),
            "build_s_sample": round(build_s, 2),
            "build_s_per_step_units": round(build_s * factor, 1),
            "threads_available": threads}


if __name__ == "__main__":
    main()
