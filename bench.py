#!/usr/bin/env python3
"""Batch-1 greedy decode throughput on one MI355X, with the roofline of the
dominant kernel and the fp64 CPU oracle timed beside it.

Default workload: the K2-Horizon-3.7B-shaped dense decoder (hidden 2560,
36 layers, 32 q / 8 kv heads, head_dim 128, SwiGLU 10240, vocab 250624,
untied lm_head) with seeded random bf16 weights 0.02*N(0,1), a bf16 KV cache
of context 4096 and a 512-token uniform-random prompt.  One step is one
decode position: embedding, 36 layers (norm + QKV, RoPE + KV append + GQA
attention, O + residual, norm + gate/up + SwiGLU, down + residual), final
norm, lm_head and argmax, with the argmax fed back on the device.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

With --config k3-latent-moe-layer it times the K3-shaped latent-MoE layer
(896 MXFP4 routed experts, top-16, 2 shared bf16 experts) at 1, 8 and 32
token rows instead.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0

# HBM bytes per launch from two profiler counter runs (FETCH_SIZE, then
# WRITE_SIZE; KiB per dispatch, averaged over every dispatch of the kernel in
# a short decode run), scaled by what the same counters read for the copy
# probe (--copy-probe 1024: 1 GiB read reads as 524301.8 KiB fetched, 1 GiB
# written as 1048576 KiB).  A reading holds only for the kernel sources it was
# taken on: if their digest differs, the traffic is reported as null.
FETCH_SCALE = 1073741824 / (524301.8 * 1024)
WRITE_SCALE = 1073741824 / (1048576.0 * 1024)
GEMV_BF16_SOURCES = ("k2_dev.h", "gemv_impl.h", "gemv.hip", "gemv_bf16.hip")
PMC_TRAFFIC = {
    "k2h-3.7b-bf16-kvbf16-ctx4096": {
        "sources": GEMV_BF16_SOURCES, "digest": "1afad823727be8ef",
        "kib": {"qkv_norm_gemv": (15493.5, 24.0), "o_gemv_residual": (10375.7, 20.0),
                "gate_up_norm_gemv_swiglu": (51345.0, 40.0),
                "down_gemv_residual": (25848.0, 20.0),
                "lm_head_norm_gemv_argmax": (626715.9, 1237.6)}},
}


def source_digest(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        with open(os.path.join(ROOT, "quantized_gemv_gqa_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(workload: str, kernel: str):
    """Counter-measured HBM bytes per launch of `kernel`, or None when no
    reading was taken for it or its sources changed since."""
    e = PMC_TRAFFIC.get(workload)
    if e is None or kernel not in e["kib"] or source_digest(e["sources"]) != e["digest"]:
        return None
    f, w = e["kib"][kernel]
    return int(round(f * 1024 * FETCH_SCALE + w * 1024 * WRITE_SCALE))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_bytes(cfg, L: int, weight_bytes: int) -> int:
    """Algorithmic HBM bytes of one decode position at prefix length L:
    every projection and the lm_head once, the KV prefix of every layer once,
    the new K/V row, the embedding row, the norm gains and the logits."""
    kv_elem = {"f32": 4, "bf16": 2, "i8": 1}[cfg.kvdt]
    kv_row = 2 * cfg.n_kv * cfg.head_dim * kv_elem + (2 * cfg.n_kv * 4 if cfg.kvdt == "i8" else 0)
    emb = cfg.hidden * (4 if cfg.embed_dt == "f32" else 2)
    gains = (2 * cfg.n_layers + 1) * cfg.hidden * 4
    return (weight_bytes + cfg.n_layers * kv_row * L + emb + gains + cfg.vocab * 4)


def time_kernel(fn, n_launch: int, stream) -> float:
    """Average duration (ms) of `n_launch` back-to-back launches issued by fn(i).

    The launches are captured once into a HIP graph so that host issue cost
    does not enter the measurement; each of 5 replays is bracketed by HIP
    events on the stream it runs on, and the median replay is reported."""
    import torch
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.graph(g, stream=cap):
        for i in range(n_launch):
            fn(i)
    stream.wait_stream(cap)
    times = []
    with torch.cuda.stream(stream):
        g.replay()                                   # warm
        torch.cuda.synchronize()
        for _ in range(5):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            g.replay()
            e.record(stream)
            e.synchronize()
            times.append(s.elapsed_time(e) / n_launch)
    return sorted(times)[len(times) // 2]


def kernel_table(gm, stream, reps: int):
    """Per-kernel average duration and algorithmic bytes for the projection
    kernels of the step, launched exactly as k2_decode_step launches them,
    rotating over the layers so no launch finds its weights in a cache."""
    import torch
    from quantized_gemv_gqa_decode_amd import k2
    cfg = gm.cfg
    dev = gm.device
    H, I = cfg.hidden, cfg.inter
    qd = cfg.n_qh * cfg.head_dim
    wdt = k2.DTYPES[cfg.wdt]
    h = torch.randn(H, device=dev) * 0.5
    hb = torch.empty_like(h)
    x_o = torch.randn(qd, device=dev)
    x_d = torch.randn(I, device=dev)
    qkv = torch.empty(cfg.qkv_rows, device=dev)
    act = torch.empty(I, device=dev)
    logits = torch.empty(cfg.vocab, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    am_b = k2.k2_argmax_workspace_bytes(cfg.vocab)
    am_ws = torch.zeros(am_b, dtype=torch.uint8, device=dev)
    Ls = gm.layers
    nl = len(Ls)

    def mats(i, name):
        m = Ls[i % nl]["mats"][name]
        return m.w, m.s, m.nbytes

    def gemv_plain(m, x, y, N, K):
        w, s, _ = m
        if cfg.wdt == "bf16":
            return k2.k2_gemv_qbf16(w, x, y, y, N, K, 1)
        if cfg.wdt == "f32":
            return k2.k2_gemv_f32(w, x, y, y, N, K, 1)
        if cfg.wdt == "fp8":
            return k2.k2_gemv_qfp8(w, s, x, y, y, N, K, 1)
        if cfg.wdt == "q4s":
            return k2.k2_gemv_qq4s(w, s, x, y, y, N, K, 1)
        return k2.k2_gemv_qmxfp4(w, s, x, y, y, N, K, 1)

    n = reps * nl
    out = {}
    ms = time_kernel(lambda i: k2.k2_norm_gemv(wdt, mats(i, "wqkv")[0], mats(i, "wqkv")[1], h,
                                               Ls[i % nl]["g_in"], cfg.groups, cfg.eps, qkv,
                                               cfg.qkv_rows, H), n, stream)
    out["qkv_norm_gemv"] = (ms, mats(0, "wqkv")[2] + 2 * H * 4 + cfg.qkv_rows * 4)
    ms = time_kernel(lambda i: gemv_plain(mats(i, "wo"), x_o, hb, H, qd), n, stream)
    out["o_gemv_residual"] = (ms, mats(0, "wo")[2] + qd * 4 + 2 * H * 4)
    ms = time_kernel(lambda i: k2.k2_norm_gemv_swiglu(wdt, mats(i, "wgu")[0], mats(i, "wgu")[1], h,
                                                      Ls[i % nl]["g_post"], cfg.groups, cfg.eps,
                                                      act, I, H), n, stream)
    out["gate_up_norm_gemv_swiglu"] = (ms, mats(0, "wgu")[2] + 2 * H * 4 + I * 4)
    ms = time_kernel(lambda i: gemv_plain(mats(i, "wd"), x_d, hb, H, I), n, stream)
    out["down_gemv_residual"] = (ms, mats(0, "wd")[2] + I * 4 + 2 * H * 4)
    # fused RoPE + KV append + attention at the next free position (the slot it
    # writes is the one the next decode step would write anyway)
    pos = gm.bench_next_pos
    L = pos + 1
    qkvb = torch.randn(cfg.qkv_rows, device=dev)
    ob = torch.empty(qd, device=dev)
    awb = k2.k2_attn_workspace_bytes(cfg.n_qh, cfg.n_kv, cfg.head_dim, cfg.cap)
    aws = torch.zeros(awb, dtype=torch.uint8, device=dev)
    kvdt = k2.DTYPES[cfg.kvdt]
    ms = time_kernel(lambda i: k2.k2_rope_append_attn(
        kvdt, qkvb, gm.rope, Ls[i % nl]["kc"], Ls[i % nl]["vc"], Ls[i % nl]["ks"], Ls[i % nl]["vs"],
        ob, cfg.n_qh, cfg.n_kv, cfg.head_dim, cfg.cap, pos, aws, awb), n, stream)
    elem = {"f32": 4, "bf16": 2, "i8": 1}[cfg.kvdt]
    kv_bytes = 2 * cfg.n_kv * cfg.head_dim * elem * L + (2 * cfg.n_kv * 4 * L if cfg.kvdt == "i8" else 0)
    out["attention_rope_append"] = (ms, kv_bytes + cfg.qkv_rows * 4 + qd * 4)
    # what the step runs: attention and then the O projection + residual,
    # one launch where the shape allows it (else the two kernels above)
    hb2 = torch.randn(H, device=dev)
    ms = time_kernel(lambda i: k2.k2_rope_append_attn_o(
        kvdt, qkvb, gm.rope, Ls[i % nl]["kc"], Ls[i % nl]["vc"], Ls[i % nl]["ks"], Ls[i % nl]["vs"],
        ob, cfg.n_qh, cfg.n_kv, cfg.head_dim, cfg.cap, pos, wdt, mats(i, "wo")[0], mats(i, "wo")[1],
        hb2, H, aws, awb), n, stream)
    out["attention_o_rope_append"] = (ms, kv_bytes + cfg.qkv_rows * 4 + mats(0, "wo")[2] + 2 * H * 4)
    nlm = max(4, reps)
    ms = time_kernel(lambda i: k2.k2_norm_gemv_argmax(wdt, gm.lm.w, gm.lm.s, h, gm.g_final,
                                                      cfg.groups, cfg.eps, logits, cfg.vocab, H,
                                                      nxt, am_ws, am_b), nlm, stream)
    out["lm_head_norm_gemv_argmax"] = (ms, gm.lm.nbytes + 2 * H * 4 + cfg.vocab * 4)
    torch.cuda.synchronize()
    return out


def cpu_baseline(cfg, budget_s: float, prefix: int = 0):
    """The oracle as it stands (fp64, OpenMP over rows) on this host's cores,
    on a bounded sample of the same workload: n full decode positions of the
    whole model (after the same synthetic int8 history when one is used), n
    chosen so the sample takes about budget_s seconds."""
    import numpy as np
    import oracle
    import synth
    log("cpu baseline: drawing oracle weights")
    dec = oracle.Decoder.from_synth(cfg, progress=log if cfg.n_layers > 4 else None)
    if prefix:
        dec.load_int8_prefix(prefix)
    pr = synth.prompt(cfg)
    dec.step(int(pr[0]), prefix, want_logits=True)
    # positions 1..m, in passes: a later pass decodes the same positions
    # again (the same work per step), so a small model's sample still
    # lasts about budget_s; a large model's stops at 16 steps
    m = min(16, len(pr) - 1, cfg.cap - prefix - 1)
    n_max = 16 if cfg.n_layers > 4 else 1 << 20
    n = 0
    t0 = time.perf_counter()
    while n < n_max and (n == 0 or time.perf_counter() - t0 < budget_s):
        p = 1 + n % m
        dec.step(int(pr[p]), prefix + p, want_logits=True)
        n += 1
    dt = time.perf_counter() - t0
    where = f"positions {prefix + 1}..{prefix + min(n, m)}" + (
        f" in {-(-n // m)} passes" if n > m else "") + (
        f" after a synthetic int8 history of {prefix}" if prefix else "")
    return {"value": n / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} full decode steps ({where}) of the whole model incl. lm_head, "
                      f"fp64 oracle, after one untimed step; {dt:.1f} s",
            "cpu": platform.processor() or platform.machine()}


def graph_time(calls, stream) -> float:
    """Average ms of one call of `calls` (a list of closures launched back to
    back), captured once into a HIP graph and replayed twice (the first replay
    warms), bracketed by HIP events on the replay stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.graph(g, stream=cap):
        for c in calls:
            c()
    stream.wait_stream(cap)
    with torch.cuda.stream(stream):
        g.replay()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record(stream)
        g.replay()
        e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / len(calls)


def moe_cpu_baseline(cfg, budget_s: float):
    """The oracle's latent-MoE layer (router, latent norm, 16 MXFP4 experts
    quantized from their bf16 windows, up-projection, 2 shared experts) on a
    bounded sample of token rows."""
    import numpy as np
    import oracle
    import synth
    log("cpu baseline: oracle MoE weights")
    wr = oracle.Mat.from_draw("bf16", synth.moe_dense_weight(cfg, "router"))
    bias = synth.moe_router_bias(cfg)
    wdn = oracle.Mat.from_draw("bf16", synth.moe_dense_weight(cfg, "down"))
    wup = oracle.Mat.from_draw("bf16", synth.moe_dense_weight(cfg, "up"))
    s13 = synth.moe_dense_weight(cfg, "shared_w13")
    s2 = synth.moe_dense_weight(cfg, "shared_w2")
    I, H = cfg.inter, cfg.hidden
    sh13 = [oracle.Mat.from_draw("bf16", s13[s * 2 * I:(s + 1) * 2 * I]) for s in range(cfg.n_shared)]
    sh2 = [oracle.Mat.from_draw("bf16", s2[s * H:(s + 1) * H]) for s in range(cfg.n_shared)]
    pool = synth.moe_expert_pool(cfg)
    x = synth.moe_activations(cfg, 32, rep=99)

    def token(t):
        sel, gate = oracle.moe_route(wr, bias, x[t], cfg.top_k, cfg.routed_scale)
        e13, e2 = {}, {}
        for e in sel:
            a, b = synth.moe_expert_draw(cfg, int(e), pool)
            e13[int(e)] = oracle.Mat.from_draw("mxfp4", a)
            e2[int(e)] = oracle.Mat.from_draw("mxfp4", b)
        return oracle.moe_apply(wdn, wup, e13, e2, sh13, sh2, x[t], cfg.latent, cfg.inter,
                                cfg.eps, sel, gate)

    t0 = time.perf_counter()
    token(0)
    t1 = time.perf_counter() - t0
    n = int(max(1, min(31, budget_s / max(t1, 1e-6))))
    t0 = time.perf_counter()
    for t in range(1, n + 1):
        token(t)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} token rows through the whole layer (routing, expert quantization "
                      f"from the bf16 windows, 16 experts, 2 shared), fp64 oracle, after one "
                      f"untimed row; {dt:.1f} s",
            "cpu": platform.processor() or platform.machine()}


def bench_moe(cfg, args, dev):
    """The K3-shaped latent-MoE layer at T = 1, 8, 32 token rows.  Each timed
    call uses the next of 8 seeded activation sets, so consecutive calls route
    to different experts and no call finds its expert weights in a cache."""
    import numpy as np
    import torch
    import synth
    from quantized_gemv_gqa_decode_amd import k2
    from quantized_gemv_gqa_decode_amd.moe import MoeLayer

    tokens = [int(t) for t in args.tokens.split(",")] if args.tokens else list(cfg.tokens)
    log(f"building {cfg.name}: {cfg.n_experts} MXFP4 experts")
    t0 = time.perf_counter()
    lay = MoeLayer(cfg, dev, max_tokens=max(tokens))
    torch.cuda.synchronize()
    eb, db = lay.expert_bytes(), lay.dense_bytes()
    log(f"layer ready in {time.perf_counter() - t0:.1f} s: experts "
        f"{eb * cfg.n_experts / 1e9:.2f} GB ({eb} B each), dense {db / 1e9:.3f} GB")
    stream = torch.cuda.current_stream()
    R = 8
    per_T = {}
    for T in tokens:
        xs = [torch.from_numpy(synth.moe_activations(cfg, T, rep=r)).to(dev) for r in range(R)]
        y = torch.empty((T, cfg.hidden), device=dev)
        idx = [torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev) for _ in range(R)]
        gw = [torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev) for _ in range(R)]
        for r in range(R):
            lay.forward(xs[r], y, idx[r], gw[r])
        torch.cuda.synchronize()
        if int(lay.err.item()) != 0:
            sys.exit(f"device error flag {int(lay.err.item())}")
        distinct = [len(np.unique(idx[r].cpu().numpy())) for r in range(R)]
        n = max(R, (args.steps // R) * R)
        ms = graph_time([lambda r=r: lay.forward(xs[r % R], y, idx[r % R], gw[r % R])
                         for r in range(n)], stream)
        u_mean = float(np.mean(distinct))
        act_bytes = T * cfg.hidden * 4 * 2
        call_bytes = db + u_mean * eb + act_bytes
        # the routed-expert call alone (bucket, W13 + SwiGLU, W2, combine)
        z = [torch.randn((T, cfg.latent), device=dev) for _ in range(R)]
        r_out = torch.empty((T, cfg.latent), device=dev)
        wsb = k2.k2_moe_workspace_bytes(T, cfg.top_k, cfg.latent, cfg.inter)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)

        def routed(r):
            return k2.k2_moe_expert_gemv(z[r], T, cfg.latent, cfg.inter, idx[r], gw[r],
                                         cfg.top_k, cfg.n_experts, lay.w13q, lay.w13s, lay.w2q,
                                         lay.w2s, r_out, lay.err, ws, wsb)

        ms_r = graph_time([lambda r=r: routed(r % R) for r in range(n)], stream)
        routed_bytes = u_mean * eb + T * cfg.latent * 4 * 2
        per_T[T] = {"us_per_call": round(ms * 1000, 2), "tokens_per_s": round(T / (ms * 1e-3), 1),
                    "distinct_experts_mean": u_mean, "bytes_per_call": int(call_bytes),
                    "GBps": round(call_bytes / (ms * 1e-3) / 1e9, 1),
                    "routed_us": round(ms_r * 1000, 2), "routed_bytes": int(routed_bytes),
                    "routed_GBps": round(routed_bytes / (ms_r * 1e-3) / 1e9, 1)}
        log(f"T={T}: {per_T[T]}")
    Th = max(tokens)
    h = per_T[Th]
    cpu = None if args.no_cpu_baseline else moe_cpu_baseline(cfg, args.cpu_budget)
    out = {
        "metric": "latent-MoE layer tokens/s (K3 shape, MXFP4 routed experts) + achieved HBM GB/s",
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": R,
        "ms_per_step": round(h["us_per_call"] / 1000, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": Th, "hidden": cfg.hidden, "latent": cfg.latent,
                   "inter": cfg.inter, "n_experts": cfg.n_experts, "top_k": cfg.top_k,
                   "n_shared": cfg.n_shared, "experts": "mxfp4", "dense": "bf16"},
        "roofline": {"bound": "hbm", "kernel": "moe_expert_gemv (bucket, W13+SwiGLU, W2, combine)",
                     "achieved": h["routed_GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(h["routed_GBps"] / PEAK_HBM_GBPS, 4),
                     "bytes_per_launch": h["routed_bytes"], "us_per_launch": h["routed_us"],
                     "traffic": None},
        "per_tokens": per_T,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_prefill(cfg, gm, P, args, stream):
    """Prompt prefill throughput: the P-position prompt through k2_prefill in
    chunks (weights streamed once per chunk, projections on the matrix cores,
    attention per position), timed with HIP events after one untimed pass;
    the next token is checked against position-by-position decode."""
    import torch
    import synth
    prompt = synth.prompt(cfg, P)
    T = args.prefill_chunk
    gm.prefill(prompt, 0, chunk=T)                   # warm (also the caches' first write)
    torch.cuda.synchronize()
    first = int(gm.next.item())
    reps = 3
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        gm.prefill(prompt, 0, chunk=T)
    e.record(stream)
    e.synchronize()
    ms = s.elapsed_time(e) / reps
    for p, t in enumerate(prompt):                   # position by position, same caches
        gm.step(int(t), p, want_logits=(p == P - 1))
    torch.cuda.synchronize()
    serial = int(gm.next.item())
    chunks = (P + T - 1) // T
    out = {
        "metric": "prompt prefill tokens/s (chunked, matrix-core projections)",
        "value": round(P / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": reps,
        "warmup": 1, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 activations (bf16 hi+lo on the matrix cores)",
        "data": "synthetic",
        "config": {"workload": cfg.name, "prompt_len": P, "chunk": T, "chunks": chunks,
                   "weights": cfg.wdt, "kv_cache": cfg.kvdt},
        "weight_GBps": round(chunks * gm.weight_bytes() / (ms * 1e-3) / 1e9, 1),
        "next_token": first, "next_token_serial_decode": serial,
    }
    print(json.dumps(out), flush=True)


def bench_verify(cfg, gm, P, args, stream):
    """One draft-and-verify round: k2_verify of T positions right after the
    prompt (the weights and lm_head read once for all T), timed with HIP
    events over repeated rounds at the same positions.  T positions per round
    is what the round yields when every draft is accepted (an upper bound;
    with synthetic random weights there is no drafter to measure)."""
    import torch
    import synth
    prompt = synth.prompt(cfg, P)
    T = args.verify_chunk
    gm.prefill(prompt, 0)
    torch.cuda.synchronize()
    feed = [int(gm.next.item())] + [int(t) for t in synth.prompt(cfg, T - 1)]
    gm.verify(feed, P)                               # warm
    torch.cuda.synchronize()
    reps = 16
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        gm.verify(feed, P)
    e.record(stream)
    e.synchronize()
    ms = s.elapsed_time(e) / reps
    wb = gm.weight_bytes()
    out = {
        "metric": "batched greedy verification: positions verified per second (all drafts accepted)",
        "value": round(T / (ms * 1e-3), 1), "unit": "positions/s", "n_gpus": 1, "steps": reps,
        "warmup": 1, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 activations (bf16 hi+lo on the matrix cores)",
        "data": "synthetic",
        "config": {"workload": cfg.name, "prompt_len": P, "positions_per_round": T,
                   "weights": cfg.wdt, "kv_cache": cfg.kvdt},
        "weight_GBps": round(wb / (ms * 1e-3) / 1e9, 1),
    }
    print(json.dumps(out), flush=True)


def bench_spec(cfg, gm, P, args, stream):
    """Speculative greedy decode with the n-gram drafter (draft.py): the
    512-token prompt, then N greedy tokens as draft-and-verify rounds
    (k2_verify of [last token, drafts]; a round without a draft is one
    k2_decode_step), wall-clock timed with the host loop it needs.  The same
    N tokens by plain greedy decode are timed first and must be equal."""
    import numpy as np
    import torch
    import synth
    prompt = synth.prompt(cfg, P)
    N = args.steps
    gm.prefill(prompt, 0)
    hist = torch.zeros(N + 1, dtype=torch.int32, device=gm.device)
    hist[0:1].copy_(gm.next)
    gm.set_pos(P)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(N - 1):
        gm.step_dev(hist[j:j + 1], hist[j + 1:j + 2])
    torch.cuda.synchronize()
    plain_s = time.perf_counter() - t0
    plain = hist[:N].cpu().numpy().tolist()
    gm.generate_speculative(prompt, 8, None, args.spec)           # warm (also the verify workspace)
    gm.prefill(prompt, 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    toks, rounds = gm.generate_speculative(prompt, N, None, args.spec, prefilled=True)
    torch.cuda.synchronize()
    spec_s = time.perf_counter() - t0
    st = gm.spec_stats
    out = {
        "metric": "speculative greedy decode tokens/s (n-gram drafter, batched verification)",
        "value": round(N / spec_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": N, "warmup": 1,
        "ms_per_step": round(spec_s / N * 1000, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "prompt_len": P, "max_drafts": args.spec,
                   "weights": cfg.wdt, "kv_cache": cfg.kvdt},
        "plain_greedy_tokens_per_s": round(N / plain_s, 1),
        "rounds": rounds, "drafted": st["drafted"], "accepted": st["accepted"],
        "acceptance": round(st["accepted"] / st["drafted"], 4) if st["drafted"] else None,
        "tokens_equal_plain_greedy": toks == plain,
        "note": "wall clock of the host loops after the prompt's prefill, both ways",
    }
    print(json.dumps(out), flush=True)


def synth_config(name):
    import synth
    return synth.CONFIGS[name]


def cpu_baseline_sample(lg, prev, params, seed, budget_s: float = 5.0):
    """The sampling oracle as it stands (fp64 numpy, one core) on the same
    logits: consecutive counters until about budget_s seconds have passed."""
    import numpy as np
    from oracle import sampling as S
    l64 = lg.astype(np.float64)
    S.sample(l64, *params, prev.tolist(), seed, 0)       # untimed
    n, t0 = 0, time.time()
    while time.time() - t0 < budget_s:
        S.sample(l64, *params, prev.tolist(), seed, n)
        n += 1
    dt = time.time() - t0
    return {"value": n / dt, "unit": "calls/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} calls of the sampling oracle on the same logits and parameters, "
                      f"consecutive counters, after one untimed call; {dt:.1f} s"}


def bench_sample(cfg, cpu: bool = True, top_k: int = 40, n_prev: int = 32):
    """k2_sample on seeded N(0, 1.5) logits of the config's vocabulary: one
    call per decode position, 200 calls with consecutive counters timed with
    HIP events (parity with the sampling oracle is the tests' job).  top_k 0
    (off) or above 64, or more than 64 previous ids, time the
    whole-vocabulary path."""
    import numpy as np
    import torch
    from quantized_gemv_gqa_decode_amd import k2
    dev = torch.device("cuda:0")
    k2.load(build_if_missing=False)
    V = cfg.vocab
    rng = np.random.default_rng(3)
    lg = (rng.standard_normal(V) * 1.5).astype(np.float32)
    prev = rng.integers(0, V, n_prev).astype(np.int32)
    params = (0.8, top_k, 0.9, 0.05, 1.2)                # temperature, top-k, top-p, min-p, penalty
    X = torch.from_numpy(lg).to(dev)
    P = torch.from_numpy(prev).to(dev)
    sp = k2.k2_sampling(temperature=params[0], top_k=params[1], top_p=params[2], min_p=params[3],
                        repetition_penalty=params[4])
    wsb = k2.k2_sample_workspace_bytes(V)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    n = 200
    out = torch.zeros(n, dtype=torch.int32, device=dev)
    for c in range(8):
        k2.check(k2.k2_sample(X, V, sp, P, n_prev, 5, c, out[c:c + 1], ws, wsb))
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for c in range(n):
        k2.check(k2.k2_sample(X, V, sp, P, n_prev, 5, c, out[c:c + 1], ws, wsb))
    e.record()
    e.synchronize()
    us = s.elapsed_time(e) / n * 1000
    line = {"metric": "k2_sample calls per second", "value": round(1e6 / us, 1),
            "unit": "calls/s", "n_gpus": 1, "steps": n, "warmup": 8,
            "ms_per_step": round(us / 1000, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "config": {"workload": cfg.name, "vocab": V,
                                            "top_k": top_k, "n_prev": n_prev,
                                            "path": "one-wave sort" if 1 <= top_k <= 64 and n_prev <= 64
                                            else "whole vocabulary"},
            "us_per_call": round(us, 1), "tokens_head": out[:8].cpu().tolist()}
    if cpu:
        line["cpu_baseline"] = cpu_baseline_sample(lg, prev, params, 5)
    print(json.dumps(line))


def read_ceiling(dev, gib: int = 2, reps: int = 10):
    """Measured read ceiling ("achievable"): k2_read_probe streams a buffer of
    `gib` GiB (far beyond the 256 MB memory-side cache) with the GEMVs' load
    policy, `reps` back-to-back launches per grid size timed with HIP events;
    the best grid size's bytes / time."""
    import torch
    from quantized_gemv_gqa_decode_amd import k2
    nbytes = gib << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    buf.fill_(0x3C3C3C3C)
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    best, table = 0.0, {}
    for blocks in (256, 512, 1024, 2048, 4096, 8192):
        read = (nbytes // 16 // blocks) * 16 * blocks
        k2.check(k2.k2_read_probe(buf, nbytes, blocks, sink))
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            k2.check(k2.k2_read_probe(buf, nbytes, blocks, sink))
        e.record(stream)
        e.synchronize()
        gbps = read * reps / (s.elapsed_time(e) * 1e-3) / 1e9
        table[blocks] = round(gbps, 1)
        best = max(best, gbps)
    del buf
    torch.cuda.empty_cache()
    log(f"read ceiling: {table}")
    return {"GBps": round(best, 1), "frac_of_peak": round(best / PEAK_HBM_GBPS, 4),
            "kernel": "k2_read_probe (non-temporal 128-bit loads, one slab per block)",
            "bytes": nbytes, "by_blocks": table}


def gemv_launches(fmts):
    """Ten launches each of the 3.7B shape's gate/up (norm + SwiGLU,
    20480 x 2560) and lm_head (norm + argmax, 250624 x 2560) GEMVs per weight
    format, on random weights quantized by the library: a fixed workload for
    profiler counter runs (rocprofv3 --pmc ... -- python3 bench.py
    --gemv-launches bf16,fp8,mxfp4,q4s)."""
    import torch
    from quantized_gemv_gqa_decode_amd import k2
    k2.load(build_if_missing=False)
    dev = torch.device("cuda:0")
    H, I, V = 2560, 10240, 250624

    def mat(wdt, N, K):
        src = (torch.randn(N, K, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
        if wdt == "bf16":
            return src, None
        if wdt == "fp8":
            w = torch.empty(N, K, dtype=torch.uint8, device=dev)
            s = torch.empty(N, device=dev)
            k2.check(k2.k2_quantize_fp8_rows(src, w, s, N, K))
        elif wdt == "mxfp4":
            w = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
            s = torch.empty(N, K // 32, dtype=torch.uint8, device=dev)
            k2.check(k2.k2_quantize_mxfp4(src, w, s, N, K))
        else:
            w = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
            s = torch.empty(N, K // 64, device=dev)
            k2.check(k2.k2_quantize_q4s(src, w, s, N, K))
        torch.cuda.synchronize()
        return w, s

    h = torch.randn(H, device=dev)
    g = torch.ones(H, device=dev)
    act = torch.empty(I, device=dev)
    lg = torch.empty(V, device=dev)
    nx = torch.zeros(1, dtype=torch.int32, device=dev)
    amb = k2.k2_argmax_workspace_bytes(V)
    amws = torch.zeros(amb, dtype=torch.uint8, device=dev)
    for f in fmts:
        dt = k2.DTYPES[f]
        gu, gus = mat(f, 2 * I, H)
        lm, lms = mat(f, V, H)
        for _ in range(10):
            k2.check(k2.k2_norm_gemv_swiglu(dt, gu, gus, h, g, 2, 1e-6, act, I, H))
        for _ in range(10):
            k2.check(k2.k2_norm_gemv_argmax(dt, lm, lms, h, g, 2, 1e-6, lg, V, H, nx, amws, amb))
        torch.cuda.synchronize()
        del gu, gus, lm, lms
        torch.cuda.empty_cache()
    print(json.dumps({"gemv_launches": fmts, "per_kernel": 10}))


def copy_probe(mib: int):
    """Five launches of an elementwise fp32 copy (y = x * 1) over mib MiB:
    each reads and writes exactly mib MiB.  Profiler counters of these
    launches calibrate the byte counters read for the decode kernels."""
    import torch
    n = mib * (1 << 20) // 4
    dev = torch.device("cuda:0")
    x = torch.rand(n, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    assert torch.equal(x, y)
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "launches": 5}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="k2h-3.7b-bf16-kvbf16-ctx4096")
    ap.add_argument("--prompt-len", type=int, default=None)
    ap.add_argument("--prefix", type=int, default=0,
                    help="int8 KV only: start from a seeded synthetic history of this many "
                         "positions in every layer instead of a prompt prefill")
    ap.add_argument("--kernel-reps", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--tokens", default=None,
                    help="latent-MoE workload only: comma-separated token counts")
    ap.add_argument("--prefill-chunk", type=int, default=0, metavar="T",
                    help="instead of the decode bench: time the prompt's prefill through "
                         "k2_prefill in chunks of T positions (2..256; bf16, fp8, MXFP4 or Q4S "
                         "weights)")
    ap.add_argument("--verify-chunk", type=int, default=0, metavar="T",
                    help="instead of the decode bench: time k2_verify of T positions (2..32; "
                         "bf16, fp8, MXFP4 or Q4S weights) after the prompt, i.e. one "
                         "draft-and-verify round")
    ap.add_argument("--spec", type=int, default=0, metavar="K",
                    help="instead of the decode bench: greedy decode of --steps tokens as "
                         "draft-and-verify rounds with the n-gram drafter (up to K drafts), "
                         "against plain greedy decode of the same tokens")
    ap.add_argument("--sample", action="store_true",
                    help="instead of the decode bench: time k2_sample over the config's vocabulary "
                         "(temperature 0.8, top-k 40, top-p 0.9, min-p 0.05, penalty 1.2 on 32 ids)")
    ap.add_argument("--sample-top-k", type=int, default=40, help="--sample: top-k (0 = off)")
    ap.add_argument("--sample-prev", type=int, default=32, help="--sample: previous ids")
    ap.add_argument("--prefill-steps", action="store_true",
                    help="consume the prompt one decode step per position instead of k2_prefill")
    ap.add_argument("--gemv-launches", default=None, metavar="FMTS",
                    help="instead of the decode bench: 10 launches each of the gate/up and "
                         "lm_head GEMVs per weight format (comma list of bf16, fp8, mxfp4, q4s), "
                         "a fixed workload for profiler counter runs")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the decode bench: launch a plain fp32 copy kernel over "
                         "MIB MiB five times (the known-size reference that scales the HBM "
                         "byte counters of a profiler run)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs the decode path on one GPU only; "
                                   "--gpus must be 1 (multi-GPU sharding is a design note)"}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.gemv_launches:
        return gemv_launches(args.gemv_launches.split(","))
    if args.sample:
        return bench_sample(synth_config(args.config), cpu=not args.no_cpu_baseline,
                            top_k=args.sample_top_k, n_prev=args.sample_prev)

    import synth
    from quantized_gemv_gqa_decode_amd import k2
    from quantized_gemv_gqa_decode_amd.model import DecodeModel

    cfg = synth.CONFIGS[args.config]
    if isinstance(cfg, synth.MoeConfig):
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        k2.load(build_if_missing=False)
        return bench_moe(cfg, args, dev)
    P = cfg.prompt_len if args.prompt_len is None else args.prompt_len
    W, K = args.warmup, args.steps
    if args.prefix:
        P = args.prefix + 1
    if P + W + K > cfg.cap:
        sys.exit(f"prompt {P} + warmup {W} + steps {K} exceeds the context {cfg.cap}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    k2.load(build_if_missing=False)

    log(f"building {cfg.name} on {torch.cuda.get_device_name(dev)}")
    t0 = time.perf_counter()
    gm = DecodeModel(cfg, dev)
    torch.cuda.synchronize()
    log(f"model ready in {time.perf_counter() - t0:.1f} s, weights {gm.weight_bytes() / 1e9:.3f} GB")
    stream = torch.cuda.current_stream()

    if args.prefill_chunk:
        return bench_prefill(cfg, gm, P, args, stream)
    if args.verify_chunk:
        return bench_verify(cfg, gm, P, args, stream)
    if args.spec:
        return bench_spec(cfg, gm, P, args, stream)

    if args.prefix:
        if cfg.kvdt != "i8":
            sys.exit("--prefix needs an int8 KV cache")
        t0 = time.perf_counter()
        gm.load_int8_prefix(args.prefix)
        gm.step(int(synth.prompt(cfg, 1)[0]), args.prefix, want_logits=True)
        torch.cuda.synchronize()
        P = args.prefix + 1
        log(f"synthetic int8 history of {args.prefix} positions loaded in "
            f"{time.perf_counter() - t0:.1f} s")
    else:
        prompt = synth.prompt(cfg, P)
        t0 = time.perf_counter()
        if cfg.wdt != "f32" and P >= 2 and not args.prefill_steps:
            gm.prefill(prompt, 0)                    # k2_prefill, 256 positions per call
            how = "k2_prefill, chunks of 256"
        else:
            for p, t in enumerate(prompt):
                gm.step(int(t), p, want_logits=(p == P - 1))
            how = "as decode steps"
        torch.cuda.synchronize()
        log(f"prefill of {P} positions ({how}) in {time.perf_counter() - t0:.2f} s")

    hist = torch.zeros(W + K + 1, dtype=torch.int32, device=dev)
    hist[0:1].copy_(gm.next)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    gm.set_pos(P)                                    # k2_decode_step_dev advances it
    for j in range(W):
        gm.step_dev(hist[j:j + 1], hist[j + 1:j + 2], err)
    torch.cuda.synchronize()

    ev_s = torch.cuda.Event(enable_timing=True)
    ev_e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev_s.record(stream)
    for j in range(W, W + K):
        gm.step_dev(hist[j:j + 1], hist[j + 1:j + 2], err)
    ev_e.record(stream)
    ev_e.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev_s.elapsed_time(ev_e)
    ms_step = ms_total / K
    if int(err.item()) != 0:
        sys.exit(f"device error flag {int(err.item())}")
    toks = hist.cpu().numpy().tolist()
    log(f"{K} steps: {ms_step * 1000:.1f} us/step (events), wall {wall / K * 1e6:.1f} us/step")

    # the same K positions again with a HIP event between consecutive steps:
    # the per-step latency series (median, p90)
    hist2 = hist.clone()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    gm.set_pos(P + W)
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i, j in enumerate(range(W, W + K)):
        gm.step_dev(hist2[j:j + 1], hist2[j + 1:j + 2], err)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(K)])
    same = hist2.cpu().numpy().tolist() == toks
    log(f"per-step series: median {np.median(per_step) * 1000:.1f} us, "
        f"p90 {np.percentile(per_step, 90) * 1000:.1f} us (tokens equal: {same})")

    # the K-step greedy loop captured once as a HIP graph and replayed: the
    # position advances on the device, so the replay walks the same positions
    graph = None
    try:
        hist3 = hist.clone()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        gm.set_pos(P + W)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            for j in range(W, W + K):
                gm.step_dev(hist3[j:j + 1], hist3[j + 1:j + 2], err)
        stream.wait_stream(cap)
        reps = []
        for r in range(3):                           # replay 0 warms; eager work in between
            gm.set_pos(P + W)
            hist3[W + 1:].zero_()
            torch.cuda.synchronize()
            gs = torch.cuda.Event(enable_timing=True)
            ge = torch.cuda.Event(enable_timing=True)
            gs.record(stream)
            g.replay()
            ge.record(stream)
            ge.synchronize()
            reps.append((gs.elapsed_time(ge), hist3.cpu().numpy().tolist() == toks))
        if int(err.item()) != 0:
            sys.exit(f"device error flag {int(err.item())} after the graph replays")
        gms = min(r[0] for r in reps[1:]) / K
        graph = {"ms_per_step": round(gms, 4), "tokens_per_s": round(1000.0 / gms, 2),
                 "steps_per_replay": K,
                 "tokens_equal_eager": all(r[1] for r in reps)}
        log(f"graph replay: {gms * 1000:.1f} us/step, tokens equal: {graph['tokens_equal_eager']}")
        del g
    except Exception as e:  # pragma: no cover - reported, not fatal
        graph = {"error": repr(e)}
        log(f"graph replay failed: {e!r}")

    Lavg = P + W + (K + 1) / 2.0
    wb = gm.weight_bytes()
    sb = step_bytes(cfg, int(round(Lavg)), wb)
    step_gbps = sb / (ms_step * 1e-3) / 1e9

    gm.bench_next_pos = P + W + K
    log("per-kernel timing")
    kt = kernel_table(gm, stream, args.kernel_reps)
    # launches per step; the stand-alone attention and O GEMV are listed for
    # reference only (the step runs them as attention_o_rope_append)
    per_step_share = {
        "attention_rope_append": 0, "o_gemv_residual": 0,
        "attention_o_rope_append": cfg.n_layers, "qkv_norm_gemv": cfg.n_layers,
        "gate_up_norm_gemv_swiglu": cfg.n_layers, "down_gemv_residual": cfg.n_layers,
        "lm_head_norm_gemv_argmax": 1}
    kernels = {}
    for name, (ms, nbytes) in kt.items():
        share = per_step_share[name]
        kernels[name] = {"us": round(ms * 1000, 2), "bytes": nbytes,
                         "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "us_per_step": round(ms * 1000 * share, 1) if share else None,
                         "traffic": pmc_traffic(cfg.name, name)}
    dom = max((k for k in kernels if kernels[k]["us_per_step"]), key=lambda k: kernels[k]["us_per_step"])
    d = kernels[dom]
    achieved = d["GBps"]

    cpu = None
    if not args.no_cpu_baseline:
        try:
            cpu = cpu_baseline(cfg, args.cpu_budget, args.prefix)
        except MemoryError as e:  # pragma: no cover
            cpu = {"error": str(e)}

    ach = read_ceiling(dev)
    out = {
        "metric": "decode tokens/s at batch 1 (3.7B-shaped) + achieved HBM GB/s vs peak",
        "value": round(1000.0 / ms_step, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(float(np.median(per_step)), 4),
        "ms_per_step_p90": round(float(np.percentile(per_step, 90)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "graph_replay": graph,
        "achievable": ach,
        "config": {"workload": cfg.name, "weights": cfg.wdt, "kv_cache": cfg.kvdt,
                   "prompt_len": 0 if args.prefix else P, "synthetic_int8_history": args.prefix,
                   "context": cfg.cap, "layers": cfg.n_layers,
                   "hidden": cfg.hidden, "vocab": cfg.vocab, "batch": 1,
                   "prefix_len_mean": Lavg},
        "step_bytes": sb,
        "step_GBps": round(step_gbps, 1),
        "step_frac_of_peak": round(step_gbps / PEAK_HBM_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "achievable": ach.get("GBps") if ach else None,
                     "bytes_per_launch": d["bytes"], "us_per_launch": d["us"],
                     "traffic": d["traffic"]},
        "kernels": kernels,
        "cpu_baseline": cpu,
        "tokens_head": toks[:8],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
