#!/usr/bin/env python3
"""Benchmark of the KVA projector forward pass on one MI355X.

One step = one call of kva_project_ubatch on one 1024-token ubatch of the r2
projector (d 2560, 3 blocks, 20 heads, SwiGLU 7040, 24 DeltaNet + 8
attention heads: 264,448 outputs per token), inputs already resident in HBM.
Prints ONE JSON line.  `value` is projected tokens/s; the r3 projector
(d 3072, + 4 drafter heads) is timed the same way and reported under "r3".

The roofline entry is for the dominant kernel, the grouped head GEMM
(about 72% of the algorithmic FLOPs): its device time is taken with HIP
event pairs that the library records around it on the launch stream during
the timed steps (kva_profile_enable); its work is 2 * n * N_heads * d FLOP.
The CPU baseline is the float64 NumPy oracle on one r2 ubatch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "projector tokens/s per 1024-token ubatch (r2,r3 bf16) + % bf16 MFMA peak"
PEAK_TFLOPS = 2516.6        # MI355X dense bf16/fp16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
HBM_GBS = 8000.0
STAGE_HEADS = 7
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "heads_gemm_r2_traffic.json")


def flops(cfg: dict, n: int) -> dict:
    """Algorithmic FLOPs of one call on n tokens: 2*M*N*K per GEMM plus the
    causal half of attention (4 * head_dim * H * B(B+1)/2 per block)."""
    d, F, n_in = cfg["d_model"], cfg["d_ffn"], cfg["n_in"]
    H, hd = cfg["n_heads"], cfg["head_dim"]
    nb = cfg["n_blocks"]
    B = cfg["attn_block"]
    blocks = [min(B, n - s) for s in range(0, n, B)]
    f = {
        "gemm_in": 2.0 * n * d * n_in,
        "gemm_qkv": nb * 2.0 * n * 3 * H * hd * d,
        "attn": nb * sum(4.0 * hd * H * b * (b + 1) / 2 for b in blocks),
        "gemm_o": nb * 2.0 * n * d * H * hd,
        "gemm_gateup": nb * 2.0 * n * 2 * F * d,
        "gemm_down": nb * 2.0 * n * d * F,
        "gemm_heads": 2.0 * n * sum(h["out_dim"] for h in cfg["heads"]) * d,
    }
    f["total"] = sum(f.values())
    return f


def src_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "learned_kv_approximation_amd", "csrc", "kva_gemm.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes():
    """Measured HBM bytes per head-GEMM launch (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    scaled by a copy-kernel calibration), if taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kva_gemm_src_sha256_16") != src_hash():
        return None
    return t.get("bytes_per_launch")


def time_config(name: str, steps: int, warmup: int, n_tokens: int = 1024, prompt: int = 0,
                stages: bool = True):
    """Times kva_project_ubatch on `n_tokens`-token calls of projector `name`.
    With prompt > 0, one step is a whole prompt of `prompt` tokens processed
    in consecutive n_tokens-token calls (output buffers reused per call)."""
    import torch

    import learned_kv_approximation_amd as kva

    cfg = synth.config(name)
    t0 = time.time()
    w = synth.make_weights(cfg)
    total = prompt or n_tokens
    x = synth.make_input(cfg, n_tokens=total)
    print(f"[bench] {name}: inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    proj = kva.Projector(cfg, w, max_tokens=n_tokens)
    del w
    xd = torch.from_numpy(x).cuda()
    del x
    outs = proj.alloc_outputs(n_tokens)

    def step():
        for c0 in range(0, total, n_tokens):
            proj.project(xd[c0:c0 + n_tokens], outs)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    kva.kva_profile_enable(proj.ctx, 1 << STAGE_HEADS)
    kva.kva_profile_read(proj.ctx)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record()
    for k in range(steps):
        step()
        evs[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [evs[k].elapsed_time(evs[k + 1]) for k in range(steps)]
    total_ms = evs[0].elapsed_time(evs[-1])
    heads = kva.kva_profile_read(proj.ctx)["gemm_heads"]

    stage_ms = {}
    if stages:
        # per-stage breakdown, a separate set of steps with every stage bracketed
        kva.kva_profile_enable(proj.ctx, (1 << len(kva.STAGES)) - 1)
        n_prof = max(3, steps // 4)
        for _ in range(n_prof):
            step()
        torch.cuda.synchronize()
        stage_ms = {k: v[1] / n_prof for k, v in kva.kva_profile_read(proj.ctx).items()}
    kva.kva_profile_enable(proj.ctx, 0)
    proj.close()
    del outs, xd
    torch.cuda.empty_cache()
    f = flops(cfg, n_tokens)
    calls = total // n_tokens
    ms = total_ms / steps
    sec = ms / 1e3
    res = {
        "tokens_per_s": total / sec,
        "ms_per_step": ms,
        "ms_median": float(np.median(per)),
        "ms_p10": float(np.percentile(per, 10)),
        "ms_p90": float(np.percentile(per, 90)),
        "wall_s": wall,
        "tflop_per_step": calls * f["total"] / 1e12,
        "pct_mfma_peak": 100.0 * calls * f["total"] / sec / (PEAK_TFLOPS * 1e12),
        "heads_gemm_ms": heads[1] / max(heads[0], 1),
        "heads_gemm_tflop": f["gemm_heads"] / 1e12,
        "stages_ms_per_step": stage_ms,
        "stage_tflops": {k: (calls * f[k] / 1e12) / (v / 1e3) if v > 0 and k in f else None
                         for k, v in stage_ms.items()},
    }
    return res


def time_kv_write(n_tokens: int = 65536, layers: int = 8, chunk: int = 8192, steps: int = 5, q8: bool = False):
    """kva_attn_kv_write for every attention layer over an n_tokens prompt
    (chunk tokens per call, as after each projection call).  Per token and
    layer it reads 2048 fp32 (8 KiB) and writes 2 x 1024 bf16 (4 KiB), or with
    q8 the Hadamard-rotated q8_0 rows (2 x 4 x 272 bytes)."""
    import torch

    import learned_kv_approximation_amd as kva

    gains, ptab, n_pages = synth.make_kv_write_inputs(n_tokens, n_layers=layers)
    # one input buffer per layer (8 x 64 MiB at 8192 tokens per call), so that
    # the reads are not served from the last-level cache
    kv0 = torch.from_numpy(synth.make_kv_rows(chunk, scale=3.0)).cuda()
    kvs = [kv0.clone() for _ in range(layers)]
    g = torch.from_numpy(gains).cuda()
    pt = torch.from_numpy(ptab).cuda()
    row_bytes = 272 if q8 else 512
    pools = [(torch.empty((n_pages, 256, 4, row_bytes), dtype=torch.uint8, device="cuda"),
              torch.empty((n_pages, 256, 4, row_bytes), dtype=torch.uint8, device="cuda")) for _ in range(layers)]
    kv_type = kva.KVA_KV_Q8_0_HADAMARD if q8 else kva.KVA_KV_BF16
    caches = [kva.kva_paged_kv(kp.data_ptr(), vp.data_ptr(), pt.data_ptr(), 256, n_pages, len(ptab),
                               4, 256, 64, 1.0e7, 1e-6, kv_type) for kp, vp in pools]
    st = kva.current_stream()

    def step():
        for c0 in range(0, n_tokens, chunk):
            for li in range(layers):
                kva.kva_attn_kv_write(kvs[li].data_ptr(), 2048, chunk, c0, g[li].data_ptr(), caches[li], st)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = n_tokens * layers * (2048 * 4 + 2 * 4 * row_bytes)
    del pools, kvs
    torch.cuda.empty_cache()
    return {"tokens": n_tokens, "layers": layers, "cache": "q8_0 + Hadamard" if q8 else "bf16",
            "ms": round(ms, 4), "bytes": nbytes,
            "gb_s": round(nbytes / (ms / 1e3) / 1e9, 1), "frac_hbm": round(nbytes / (ms / 1e3) / 1e9 / HBM_GBS, 4),
            "launches": (n_tokens // chunk) * layers}


def time_prompt_kv(prompt: int = 65536, chunk: int = 8192, steps: int = 3, warmup: int = 1):
    """The r3 bf16 projector over a `prompt`-token prompt in `chunk`-token
    calls, with the attention-layer state update (k_norm + RoPE + paged bf16
    KV write for the 8 attention heads): chained (kva_project_ubatch, then
    kva_attn_kv_write per attention head) and fused into the head GEMM
    (kva_project_ubatch_kv).  Both fill the same pools with the same bits."""
    import torch

    import learned_kv_approximation_amd as kva

    cfg = synth.config("r3_kv")
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=prompt)
    proj = kva.Projector(cfg, w, max_tokens=chunk)
    del w
    xd = torch.from_numpy(x).cuda()
    del x
    attn = [i for i, h in enumerate(cfg["heads"]) if h["kind"] == "attn"]
    gains, ptab, n_pages = synth.make_kv_write_inputs(prompt, n_layers=len(attn), seed=cfg["seed"])
    g = torch.from_numpy(gains).cuda()
    pt = torch.from_numpy(ptab).cuda()
    pools = [(torch.empty((n_pages, 256, 4, 256), dtype=torch.int16, device="cuda"),
              torch.empty((n_pages, 256, 4, 256), dtype=torch.int16, device="cuda")) for _ in attn]
    caches = [kva.kva_paged_kv(kp.data_ptr(), vp.data_ptr(), pt.data_ptr(), 256, n_pages, len(ptab),
                               4, 256, 64, 1.0e7, 1e-6) for kp, vp in pools]
    dests = [kva.kva_attn_dest(g[li].data_ptr(), caches[li]) for li in range(len(attn))]
    outs = proj.alloc_outputs(chunk)
    st = kva.current_stream()
    ptrs = [0 if i in attn else o.data_ptr() for i, o in enumerate(outs)]

    def chained():
        for c0 in range(0, prompt, chunk):
            proj.project(xd[c0:c0 + chunk], outs)
            for li, hi in enumerate(attn):
                kva.kva_attn_kv_write(outs[hi].data_ptr(), 2048, chunk, c0, g[li].data_ptr(), caches[li], st)

    def fused():
        for c0 in range(0, prompt, chunk):
            kva.kva_project_ubatch_kv(proj.ctx, xd[c0:].data_ptr(), chunk, ptrs, c0, dests, st)

    res = {"tokens": prompt, "tokens_per_call": chunk, "attention_layers": len(attn)}
    for name, fn in (("chained", chained), ("fused", fused)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"ms_per_prompt": round(ms, 3), "tokens_per_s": round(prompt / (ms / 1e3), 1)}
    res["fused_speedup"] = round(res["chained"]["ms_per_prompt"] / res["fused"]["ms_per_prompt"], 4)
    proj.close()
    del pools, outs, xd
    torch.cuda.empty_cache()
    return res


def time_deltanet(n_tokens: int = 1024, layers: int = 24, steps: int = 10):
    """kva_deltanet_update for the 24 DeltaNet layers of one 1024-token
    ubatch (rows of qkv | a | b like the projector's DeltaNet heads, ~N(0,1)).
    Algorithmic bytes per layer: the k, v, a, b columns of every row read once
    (8288 fp32), the 128x128 fp32 states of the 48 value heads read and
    written, the conv weights of k and v, and the new conv state (3 rows of
    all 10240 channels read from the rows and written)."""
    import torch

    import learned_kv_approximation_amd as kva

    conv_w, a_log, dt_bias = synth.make_deltanet_params(layers)
    conv, S = synth.make_deltanet_state(layers)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    rows = [torch.randn((n_tokens, 10336), generator=g, device="cuda") for _ in range(layers)]
    dev = [(torch.from_numpy(conv_w[l]).cuda(), torch.from_numpy(a_log[l]).cuda(), torch.from_numpy(dt_bias[l]).cuda(),
            torch.from_numpy(conv[l]).cuda(), torch.from_numpy(S[l]).cuda()) for l in range(layers)]
    ls = [kva.kva_deltanet_layer(rows[l].data_ptr(), 10336, *[t.data_ptr() for t in dev[l]]) for l in range(layers)]
    st = kva.current_stream()
    kva.kva_deltanet_update(ls, n_tokens, stream=st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        kva.kva_deltanet_update(ls, n_tokens, stream=st)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    per_layer = (n_tokens * 8288 * 4 + 2 * 48 * 128 * 128 * 4 + 8192 * 16 + 2 * 3 * 10240 * 4)
    nbytes = layers * per_layer
    del rows, dev
    torch.cuda.empty_cache()
    return {"tokens": n_tokens, "layers": layers, "ms": round(ms, 4), "bytes": nbytes,
            "gb_s": round(nbytes / (ms / 1e3) / 1e9, 1), "frac_hbm": round(nbytes / (ms / 1e3) / 1e9 / HBM_GBS, 4),
            "tokens_per_s": round(n_tokens / (ms / 1e3), 1)}


def time_map(start_layer: int = 12, n_layers: int = 64, n_in: int = 5120, n_tokens: int = 1024,
             steps: int = 10, warmup: int = 3):
    """The single-map projector: one bf16 map per later layer (start_layer+1 ..
    n_layers-1) on the raw residual, 1024-token calls; one grouped GEMM of
    2 * n_tokens * n_in * n_in * n_maps FLOP per call."""
    import torch

    import learned_kv_approximation_amd as kva

    n_maps = synth.map_layers(start_layer, n_layers)
    t0 = time.time()
    maps, biases = synth.make_map_weights(n_in, n_maps, "bf16")
    x = torch.from_numpy(synth.make_map_input(n_tokens, n_in)).cuda()
    mp = kva.MapProjector(maps, biases, dtype="bf16", n_in=n_in, max_tokens=n_tokens)
    del maps, biases
    print(f"[bench] single-map projector: {n_maps} maps built in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    outs = mp.project(x)
    for _ in range(warmup):
        mp.project(x, outs)
    torch.cuda.synchronize()
    kva.kva_profile_enable(mp.ctx, 1 << STAGE_HEADS)
    kva.kva_profile_read(mp.ctx)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        mp.project(x, outs)
    e1.record()
    torch.cuda.synchronize()
    heads = kva.kva_profile_read(mp.ctx)["gemm_heads"]
    kva.kva_profile_enable(mp.ctx, 0)
    ms = e0.elapsed_time(e1) / steps
    flop = 2.0 * n_tokens * n_in * n_in * n_maps
    mp.close()
    del outs, x
    torch.cuda.empty_cache()
    return {"start_layer": start_layer, "n_layers": n_layers, "maps": n_maps, "n_in": n_in, "tokens": n_tokens,
            "ms": round(ms, 4), "tokens_per_s": round(n_tokens / (ms / 1e3), 1),
            "tflop_per_call": round(flop / 1e12, 5), "pct_mfma_peak": round(100 * flop / (ms / 1e3) / (PEAK_TFLOPS * 1e12), 2),
            "gemm_ms": round(heads[1] / max(heads[0], 1), 4)}


def mfma_loop(n_iter: int = 4000, workgroups_per_cu: int = 4, reps: int = 10):
    """The MFMA rate the device sustains with no memory traffic (the library's
    kva_debug_mfma_loop): the achievable ceiling at the clock it runs at."""
    import torch

    import learned_kv_approximation_amd as kva

    n_wg = torch.cuda.get_device_properties(0).multi_processor_count * workgroups_per_cu
    sink = torch.empty(256 * n_wg, dtype=torch.float32, device="cuda")
    st = kva.current_stream()
    for _ in range(3):
        kva.kva_debug_mfma_loop(n_iter, n_wg, sink.data_ptr(), st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        kva.kva_debug_mfma_loop(n_iter, n_wg, sink.data_ptr(), st)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flop = n_wg * 4 * n_iter * 8 * 32768
    tf = flop / (ms / 1e3) / 1e12
    return {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS, 4), "ms": round(ms, 4),
            "waves": n_wg * 4, "mfma_per_wave": n_iter * 8, "instr": "v_mfma_f32_32x32x16_bf16"}


def linear_weight_params(cfg: dict) -> int:
    """Weights of every Linear of the projector (what q8_0 stores in blocks)."""
    d, F, hd = cfg["d_model"], cfg["d_ffn"], cfg["n_heads"] * cfg["head_dim"]
    trunk = cfg["n_in"] * d + cfg["n_blocks"] * (3 * hd * d + d * hd + 2 * F * d + d * F)
    return trunk + sum(h["out_dim"] for h in cfg["heads"]) * d


def q8_m_sweep(ms=(16, 32, 64, 128, 256, 512, 1024), steps: int = 10, warmup: int = 3):
    """The r3 q8_0 projector at M tokens per call, each M in a context sized for
    it: each call reads every weight once, so below M of a few hundred the
    path is bound by weight bandwidth (reported as GB/s of the weight bytes a
    call reads, for the whole call and for the head GEMM alone: q8_0's 34 per
    32 weights, or 2 per weight where a context of more than 256 tokens per
    call holds the weights expanded to fp16)."""
    import torch

    import learned_kv_approximation_amd as kva

    cfg = synth.config("r3_q8_0")
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=max(ms))
    xd = torch.from_numpy(x).cuda()
    n_w = linear_weight_params(cfg)
    n_head = sum(h["out_dim"] for h in cfg["heads"]) * cfg["d_model"]
    res = {}
    for m in ms:
        expanded = m > 256
        wbytes = n_w * 2 if expanded else n_w * 34 // 32
        head_bytes = n_head * 2 if expanded else n_head * 34 // 32
        # a context sized for the call (max_tokens = M), as a caller that runs
        # calls of this size would create
        proj = kva.Projector(cfg, w, max_tokens=m)
        outs = proj.alloc_outputs(m)
        xm = xd[:m].contiguous()
        for _ in range(warmup):
            proj.project(xm, outs)
        torch.cuda.synchronize()
        kva.kva_profile_enable(proj.ctx, 1 << STAGE_HEADS)
        kva.kva_profile_read(proj.ctx)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            proj.project(xm, outs)
        e1.record()
        torch.cuda.synchronize()
        hs = kva.kva_profile_read(proj.ctx)["gemm_heads"]
        proj.close()
        t = e0.elapsed_time(e1) / steps
        th = hs[1] / max(hs[0], 1)
        f = flops(cfg, m)["total"]
        res[str(m)] = {"weights": "fp16" if expanded else "q8_0",
                       "ms": round(t, 4), "tokens_per_s": round(m / (t / 1e3), 1),
                       "pct_mfma_peak": round(100.0 * f / (t / 1e3) / (PEAK_TFLOPS * 1e12), 2),
                       "weight_gb_s": round(wbytes / (t / 1e3) / 1e9, 1),
                       "frac_hbm": round(wbytes / (t / 1e3) / 1e9 / HBM_GBS, 4),
                       "heads_gemm_ms": round(th, 4),
                       "heads_weight_gb_s": round(head_bytes / (th / 1e3) / 1e9, 1),
                       "heads_frac_hbm": round(head_bytes / (th / 1e3) / 1e9 / HBM_GBS, 4)}
    del w
    del outs, xd
    torch.cuda.empty_cache()
    return {"weight_bytes_q8_0": n_w * 34 // 32, "head_weight_bytes_q8_0": n_head * 34 // 32,
            "by_tokens_per_call": res}


def traffic_probe():
    """Kernels whose HBM counters calibrate the head GEMM's traffic: two r2
    projections, then two copies of exactly COPY_BYTES (read COPY_BYTES,
    write COPY_BYTES) with torch's device copy."""
    import torch

    import learned_kv_approximation_amd as kva
    cfg = synth.config("r2")
    proj = kva.Projector(cfg, synth.make_weights(cfg), max_tokens=1024)
    xd = torch.from_numpy(synth.make_input(cfg)).cuda()
    outs = proj.alloc_outputs(1024)
    for _ in range(2):
        proj.project(xd, outs)
    torch.cuda.synchronize()
    proj.close()
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()


COPY_BYTES = 1 << 30


def cpu_baseline(min_seconds: float = 10.0, max_reps: int = 8):
    """The oracle, as it stands, on whole r2 ubatches (1024 tokens, all 32 heads),
    repeated until about `min_seconds` of CPU work; tokens/s over all reps.
    Beside it (key "fp32"), the same steps in float32 NumPy (sgemm): the
    oracle's algorithm without rounding points, timed the same way."""
    import oracle
    from oracle import emu
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:
        threads = os.cpu_count() or 1
    cfg = synth.config("r2")
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=1024)
    prep = oracle.prepare(cfg, w)          # weight decode to float64, outside the timed region
    reps, t0 = 0, time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.project(cfg, prep, x)
        reps += 1
    dt = time.perf_counter() - t0
    del prep
    # float32: weight decode happens inside the call (it is part of emu.project),
    # so time it separately and subtract it from the total
    t1 = time.perf_counter()
    emu.project(cfg, w, x[:1], points=(), arith=np.float32)
    decode = time.perf_counter() - t1
    r32, t2 = 0, time.perf_counter()
    while r32 < max_reps and (r32 == 0 or time.perf_counter() - t2 < min_seconds / 2):
        emu.project(cfg, w, x, points=(), arith=np.float32)
        r32 += 1
    dt32 = max(time.perf_counter() - t2 - r32 * decode, 1e-9)
    return {"value": 1024 * reps / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"r2, {reps} x one 1024-token ubatch (all 32 heads), float64 NumPy with "
                      f"{threads} BLAS threads, {dt:.1f} s",
            "cpu_model": _cpu_model(), "blas": blas,
            "affinity_cores": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "fp32": {"value": 1024 * r32 / dt32, "unit": "tokens/s", "cores": int(threads),
                     "sample": f"r2, {r32} x one 1024-token ubatch, the oracle's steps in float32 NumPy "
                               f"(sgemm), {dt32:.1f} s after subtracting the weight decode "
                               f"({decode:.1f} s per call)"}}


def power_loop(seconds: float, interval: float = 0.5):
    """Loops r2 projections (one 1024-token ubatch per call) for `seconds`
    while a second thread samples `amd-smi metric -p -c --json` every
    `interval` s; returns the socket power and clock samples."""
    import subprocess
    import threading

    import torch

    import learned_kv_approximation_amd as kva

    cfg = synth.config("r2")
    w = synth.make_weights(cfg)
    proj = kva.Projector(cfg, w, max_tokens=1024)
    del w
    xd = torch.from_numpy(synth.make_input(cfg)).cuda()
    outs = proj.alloc_outputs(1024)
    for _ in range(5):
        proj.project(xd, outs)
    torch.cuda.synchronize()
    kva.kva_profile_enable(proj.ctx, 1 << STAGE_HEADS)
    kva.kva_profile_read(proj.ctx)
    for _ in range(20):
        proj.project(xd, outs)
    heads = kva.kva_profile_read(proj.ctx)["gemm_heads"]
    kva.kva_profile_enable(proj.ctx, 0)
    samples, stop = [], [False]

    def find(obj, key):
        if isinstance(obj, dict):
            for k, v in obj.items():
                if k == key:
                    yield v
                yield from find(v, key)
        elif isinstance(obj, list):
            for v in obj:
                yield from find(v, key)

    def sampler():
        while not stop[0]:
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                   timeout=10)
                d = json.loads(r.stdout)
                pw = next((v.get("value") for v in find(d, "socket_power") if isinstance(v, dict)), None)
                gfx = [v["clk"]["value"] for v in find(d, "gfx_0") if isinstance(v, dict) and isinstance(v.get("clk"), dict)]
                mem = [v["clk"]["value"] for v in find(d, "mem_0") if isinstance(v, dict) and isinstance(v.get("clk"), dict)]
                samples.append({"t": round(time.perf_counter() - t0, 2), "socket_power_w": pw,
                                "gfx_mhz": gfx[0] if gfx else None, "mem_mhz": mem[0] if mem else None})
            except Exception as ex:   # the tool is optional: report, do not fail the run
                samples.append({"error": str(ex)[:200]})
            time.sleep(interval)

    t0 = time.perf_counter()
    th = threading.Thread(target=sampler)
    th.start()
    calls = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            proj.project(xd, outs)
        torch.cuda.synchronize()
        calls += 50
    stop[0] = True
    th.join()
    proj.close()
    return {"calls": calls, "seconds": round(time.perf_counter() - t0, 2),
            "heads_gemm_ms": round(heads[1] / max(heads[0], 1), 4), "samples": samples}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-r3", action="store_true")
    ap.add_argument("--quick", action="store_true", help="r2 and r3 one-ubatch lines only")
    ap.add_argument("--line", choices=["deltanet", "map", "kv_write", "kv_write_q8", "prompt_kv"],
                    help="run one extra line alone and print its JSON (for profiling runs)")
    ap.add_argument("--power-loop", type=float, default=0.0, metavar="SECONDS",
                    help="loop r2 projections for SECONDS while sampling socket power and clocks (amd-smi)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run 2 r2 projections and 2 plain 1 GiB device copies, print nothing (for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(multi-GPU runs are not part of this benchmark).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import learned_kv_approximation_amd as kva
    kva.lib()   # fails loudly if libkva.so is missing
    if args.traffic_probe:
        traffic_probe()
        return
    if args.power_loop > 0:
        print(json.dumps({"line": "power_loop", **power_loop(args.power_loop)}), flush=True)
        return
    if args.line:
        fn = {"deltanet": time_deltanet, "map": time_map, "kv_write": time_kv_write,
              "kv_write_q8": lambda: time_kv_write(q8=True), "prompt_kv": time_prompt_kv}[args.line]
        print(json.dumps({"line": args.line, **fn()}), flush=True)
        return

    r2 = time_config("r2", args.steps, args.warmup)
    print(f"[bench] r2: {r2['tokens_per_s']:.0f} tok/s, {r2['pct_mfma_peak']:.1f}% peak", file=sys.stderr, flush=True)
    r3 = r3b = q8 = q8p = q4 = kvw = kvw8 = kvp = dnu = p2 = sweep = mloop = None
    if not args.no_r3:
        r3 = time_config("r3", args.steps, args.warmup)
        print(f"[bench] r3: {r3['tokens_per_s']:.0f} tok/s, {r3['pct_mfma_peak']:.1f}% peak", file=sys.stderr,
              flush=True)
        if not args.quick:
            r3b = time_config("r3", max(5, args.steps // 3), 2, n_tokens=8192, stages=False)
            print(f"[bench] r3 8192: {r3b['tokens_per_s']:.0f} tok/s", file=sys.stderr, flush=True)
            q8 = time_config("r3_q8_0", args.steps, args.warmup, stages=True)
            print(f"[bench] r3 q8_0: {q8['tokens_per_s']:.0f} tok/s", file=sys.stderr, flush=True)
            q8p = time_config("r3_q8_0", 3, 1, n_tokens=8192, prompt=65536, stages=False)
            print(f"[bench] r3 q8_0 65536: {q8p['tokens_per_s']:.0f} tok/s", file=sys.stderr, flush=True)
            q4 = time_config("r3_q4_0", args.steps, args.warmup, stages=True)
            print(f"[bench] r3 q4_0: {q4['tokens_per_s']:.0f} tok/s", file=sys.stderr, flush=True)
            kvw = time_kv_write()
            print(f"[bench] kv write: {kvw['gb_s']} GB/s", file=sys.stderr, flush=True)
            kvw8 = time_kv_write(q8=True)
            print(f"[bench] kv write q8_0: {kvw8['gb_s']} GB/s", file=sys.stderr, flush=True)
            dnu = time_deltanet()
            print(f"[bench] deltanet update 24 layers x 1024: {dnu['ms']} ms, {dnu['gb_s']} GB/s",
                  file=sys.stderr, flush=True)
            p2 = time_map()
            print(f"[bench] single-map projector (start 12, 51 maps): {p2['tokens_per_s']:.0f} tok/s, "
                  f"{p2['pct_mfma_peak']}% peak", file=sys.stderr, flush=True)
            kvp = time_prompt_kv()
            print(f"[bench] r3 65536 + KV: chained {kvp['chained']['tokens_per_s']:.0f} tok/s, "
                  f"fused {kvp['fused']['tokens_per_s']:.0f} tok/s", file=sys.stderr, flush=True)
            sweep = q8_m_sweep()
            print("[bench] q8_0 M sweep: " + ", ".join(f"{m}: {v['weight_gb_s']} GB/s (heads {v['heads_weight_gb_s']})"
                                                        for m, v in sweep["by_tokens_per_call"].items()),
                  file=sys.stderr, flush=True)
    if not args.quick:
        mloop = mfma_loop()
        print(f"[bench] pure MFMA loop: {mloop['tflops']} TFLOP/s", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()
        print(f"[bench] cpu oracle: {cpu['value']:.1f} tok/s", file=sys.stderr, flush=True)

    achieved = r2["heads_gemm_tflop"] / (r2["heads_gemm_ms"] / 1e3)
    out = {
        "metric": METRIC,
        "value": round(r2["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r2["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 heads + fp16 trunk MFMA, fp32 accumulate",
        "data": "synthetic (seeded N(0,1/fan_in) bf16 weights, N(0,1) residuals at RMS 4)",
        "config": {"workload": "r2 KVA projector forward, one 1024-token ubatch: 5120 -> d 2560, 3 blocks "
                               "(20 heads x 128, SwiGLU 7040), 24 DeltaNet heads (10240+48+48) + 8 attention "
                               "heads (1024+1024)",
                   "tokens_per_step": 1024, "tflop_per_step": round(r2["tflop_per_step"], 5)},
        "pct_mfma_peak": round(r2["pct_mfma_peak"], 2),
        "ms_median": round(r2["ms_median"], 4), "ms_p10": round(r2["ms_p10"], 4), "ms_p90": round(r2["ms_p90"], 4),
        "roofline": {"bound": "mfma", "kernel": "gemm_t32_heads<bf16>",
                     "achieved": round(achieved, 1), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic_bytes(),
                     "launch_ms": round(r2["heads_gemm_ms"], 4),
                     "flop_per_launch": r2["heads_gemm_tflop"] * 1e12},
        "stages_ms_per_step": {k: round(v, 4) for k, v in r2["stages_ms_per_step"].items()},
        "stage_tflops": {k: (round(v, 1) if v else None) for k, v in r2["stage_tflops"].items()},
        "cpu_baseline": cpu,
    }
    def brief(r):
        return {"tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 4),
                "pct_mfma_peak": round(r["pct_mfma_peak"], 2), "tflop_per_step": round(r["tflop_per_step"], 5),
                "heads_gemm_ms": round(r["heads_gemm_ms"], 4),
                "stages_ms_per_step": {k: round(v, 4) for k, v in r["stages_ms_per_step"].items()}}
    if r3 is not None:
        out["r3"] = brief(r3)
    if r3b is not None:
        out["r3_8192_tokens_one_call"] = brief(r3b)
    if q8 is not None:
        out["r3_q8_0"] = brief(q8)
    if q8p is not None:
        out["r3_q8_0_prompt_65536"] = brief(q8p)
    if q4 is not None:
        out["r3_q4_0"] = brief(q4)
    if kvw is not None:
        out["kv_write_65536x8"] = kvw
    if kvw8 is not None:
        out["kv_write_q8_0_65536x8"] = kvw8
    if kvp is not None:
        out["r3_prompt_65536_with_kv"] = kvp
    if dnu is not None:
        out["deltanet_update_24x1024"] = dnu
    if p2 is not None:
        out["single_map_projector_start12"] = p2
    if sweep is not None:
        out["r3_q8_0_m_sweep"] = sweep
    if mloop is not None:
        out["mfma_loop"] = mloop
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
