"""Benchmark of the H3 DiT block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one h3_block_forward over the full-width block at the pages'
packed length: 58,758 valid tokens in a 58,816-token buffer, hidden 5376,
42 heads x 128, SwiGLU width 21504, BF16 with FP32 modulation. Inputs are
synthetic (seeded normal weights ~N(0, 0.02), activations ~N(0, 1), AdaLN
table ~N(0, 0.1)) generated on the GPU and resident in HBM before timing.

Prints ONE JSON line: ms per block (HIP events on the library's stream,
bracketed by synchronize), algorithmic TFLOP/s, a per-kernel breakdown timed
the same way with the block's own launch configurations, the roofline of the
dominant kernel (attention) and the FP64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import statistics
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 (and MXFP8) MFMA, published
SEED = 20260903


def block_flops(V: int, H: int, F: int, heads_dim_total: int | None = None):
    """Algorithmic work over valid rows: GEMMs 2 V H (4H + 3F); attention
    4 V^2 H (QK^T and PV, no causal halving)."""
    gemm = 2.0 * V * H * (4 * H + 3 * F)
    attn = 4.0 * V * V * H
    return gemm, attn


def elementwise_bytes(V: int, H: int, F: int):
    """Algorithmic HBM bytes of the memory-bound steps (BF16 = 2 B):
    modnorm x->h 4VH; qk-norm+RoPE in place on q,k 8VH; modnorm x1->h2 4VH."""
    return {"modnorm": 4.0 * V * H, "qk_norm_rope": 8.0 * V * H, "modnorm2": 4.0 * V * H}


def counter_traffic(kernel: str, sources):
    """HBM-side bytes per dispatch of `kernel` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (profiles/counters.json, already scaled by
    the copy calibration), or None when any of the kernel's sources has
    changed since the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
            c = json.load(f)
        for source in sources:
            with open(os.path.join(ROOT, "video_diffusion_transformer_dit_amd", "csrc", source), "rb") as f:
                sha = hashlib.sha256(f.read()).hexdigest()[:16]
            if c["source_sha256_16"].get(source) != sha:
                return None
        k = c["kernels"][kernel]
        return int(k["read_bytes"] + k["write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def time_calls(torch, fn, iters: int, warmup: int, per_call: bool = False):
    """Average ms per call with HIP events on the current stream (all `iters`
    calls between one pair of events). With per_call, an event is also
    recorded between consecutive calls and the per-call times are returned too."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1 if per_call else 2)]
    ev[0].record()
    for i in range(iters):
        fn()
        if per_call:
            ev[i + 1].record()
    ev[-1].record()
    torch.cuda.synchronize()
    mean = ev[0].elapsed_time(ev[-1]) / iters
    if not per_call:
        return mean
    return mean, [ev[i].elapsed_time(ev[i + 1]) for i in range(iters)]


def cpu_baseline(seconds_target: float = 20.0, configs: bool = True):
    """FP64 oracle on a bounded sample: the full-width block at L tokens, scaled
    to ms per block at the 58,758-token workload by algorithmic flops. A
    1,024-token probe sizes the sample: L grows (in steps of 64 rows, at most
    8,192) until the sample takes about `seconds_target` on this host."""
    from oracle import h3_oracle as O
    from video_diffusion_transformer_dit_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def run(L):
        s = I.scaled(I.FULL_4096, L, name=f"full-{L}")
        wb = I.block_weights(s, "cpu0")
        w = {k: O.bf16_to_f64(v) for k, v in wb.items()}
        x = O.bf16_to_f64(I.activations(s, tag="cpu0.x"))
        mod = I.mod_table(s, 1, tag="cpu0.mod").astype(np.float64)
        t0 = time.perf_counter()
        O.block_forward(x, w, mod, heads=s.heads, head_dim=128, ffn=s.ffn, valid_len=L, rot_dim=s.rot_dim)
        return time.perf_counter() - t0

    L, dt = 1024, run(1024)
    if dt < seconds_target / 3:
        L = int(min(8192, max(1024, 1024 * seconds_target / dt)) // 64 * 64)
        if L > 1024:
            dt = run(L)
    g_s, a_s = block_flops(L, 5376, 21504)
    g_f, a_f = block_flops(58758, 5376, 21504)
    ms_full = dt * 1e3 * (g_f + a_f) / (g_s + a_s)
    out = {"value": round(ms_full, 1), "unit": "ms/block", "cores": int(threads), "cpu": cpu_model(),
           "kind": "oracle", "extrapolated": True,
           "sample": f"FP64 numpy oracle, one full-width block (H 5376, 42x128, F 21504) at {L} tokens: "
                     f"{dt:.2f} s for {(g_s + a_s) / 1e12:.3f} TFLOP, scaled by algorithmic flops to the "
                     f"58,758-token block ({(g_f + a_f) / 1e12:.1f} TFLOP)",
           "sample_tokens": L, "sample_seconds": round(dt, 3), "sample_gflops_per_s": round((g_s + a_s) / dt / 1e9, 1)}
    if configs:
        out["configs"] = cpu_oracle_configs(threads)
        # the same extrapolation from the 4,096-token block: a second sample size
        c2 = out["configs"]["full_4096"]
        g4, a4 = block_flops(4096, 5376, 21504)
        out["extrapolation_from_4096_tokens_ms"] = round(c2["s"] * 1e3 * (g_f + a_f) / (g4 + a4), 1)
    return out


def cpu_model():
    """Host CPU: /proc/cpuinfo's model name with its family / model / stepping
    numbers (the name alone can be generic), logical CPUs and usable ones."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" in ln:
                    k, v = (t.strip() for t in ln.split(":", 1))
                    info.setdefault(k, v)
                if not ln.strip() and info:
                    break
    except OSError:  # pragma: no cover
        pass
    name = info.get("model name") or platform.processor() or "unknown"
    fms = "/".join(info.get(k, "?") for k in ("cpu family", "model", "stepping"))
    return (f"{name} (family/model/stepping {fms}; {os.cpu_count()} logical CPUs, "
            f"{len(os.sched_getaffinity(0))} usable)")


def cpu_oracle_configs(threads: int):
    """The FP64 oracle timed once per workload that fits a bounded CPU run
    (wall clock of the oracle call alone, inputs generated before): the tiny
    block, the full-width block at 4,096 tokens, one forward of the streaming
    chunk (its 4 denoise forwards and the refresh forward are the same work;
    the chunk is 5 of them) and the stacked loop's check of 2 layers at 2,048
    tokens. The 58,758-token block is not run; cpu_baseline extrapolates it."""
    from oracle import h3_oracle as O
    from video_diffusion_transformer_dit_amd import inputs as I

    def timed(s, groups=None, pos=None, tag="cpu"):
        wb = I.block_weights(s, tag)
        w = {k: O.bf16_to_f64(v) for k, v in wb.items()}
        x = O.bf16_to_f64(I.activations(s, tag=f"{tag}.x"))
        mod = I.mod_table(s, 1, tag=f"{tag}.mod").astype(np.float64)
        t0 = time.perf_counter()
        O.block_forward(x, w, mod, heads=s.heads, head_dim=128, ffn=s.ffn, valid_len=s.valid_len,
                        rot_dim=s.rot_dim, groups=groups, pos=pos)
        return time.perf_counter() - t0

    out = {"cores": int(threads), "kind": "oracle", "unit": "s"}
    t = timed(I.TINY, tag="cpu.tiny")
    out["tiny_block"] = {"workload": "tiny block, 512 rows (500 valid), H 256, 2x128, F 1024", "s": round(t, 3)}
    progress(f"CPU oracle: tiny block {t:.2f} s")
    t = timed(I.FULL_4096, tag="cpu.c2")
    g, a = block_flops(4096, 5376, 21504)
    out["full_4096"] = {"workload": "full-width block at 4,096 valid tokens", "s": round(t, 3),
                        "gflops_per_s": round((g + a) / t / 1e9, 1)}
    progress(f"CPU oracle: 4,096-token block {t:.2f} s")
    s = I.streaming_shape()
    hk, hv = I.history_kv(I.STREAM_HISTORY, s.hidden, tag="cpu.hist")
    c, au, L = I.STREAM_COND, I.STREAM_AUDIO, s.L_buf
    cur = ("self", 0, L)
    groups = [(0, c, [cur]), (c, c + au, [cur]), (c + au, L, [(O.bf16_to_f64(hk), O.bf16_to_f64(hv)), cur])]
    pos = np.arange(L, dtype=np.int64) + I.STREAM_HISTORY
    t = timed(s, groups=groups, pos=pos, tag="cpu.c4")
    out["streaming_forward"] = {"workload": "one streaming forward: [cond 256 | audio 128 | video 5,040] over "
                                            "15,120 history rows, full width", "s": round(t, 3),
                                "chunk_s_5_forwards": round(5 * t, 3)}
    progress(f"CPU oracle: streaming forward {t:.2f} s")
    s = I.scaled(I.FULL_4096, 2048, name="full-2048")
    t = sum(timed(s, tag=f"cpu.c5.{i}") for i in range(2))
    out["stacked_two_layers_2048"] = {"workload": "2 full-width blocks at 2,048 tokens (the stacked loop's "
                                                  "per-layer check)", "s": round(t, 3)}
    progress(f"CPU oracle: 2 layers at 2,048 tokens {t:.2f} s")
    return out


def lora_consumers(torch, h3, dev, gen, L, V, H, heads, F, iters):
    """Precision-preserving LoRA consumer fusion at the block's full sizes: each
    consumer fused (it forms bf16(base + delta) itself) against the unfused
    sequence (a separate BF16 add that stores the sum, then the plain consumer).
    saved_gb is the sum's HBM write + read that the fusion removes."""
    def rnd(shape, std=1.0):
        t = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        t.mul_(std)
        return t.to(torch.bfloat16)

    res = {}
    # QKV consumer: QK-norm + RoPE on q, k and packing of v
    qkv, dq, tmp = rnd((L, 3 * H), 3.0), rnd((L, 3 * H), 0.3), torch.empty((L, 3 * H), dtype=torch.bfloat16,
                                                                            device=dev)
    gq = torch.ones(128, dtype=torch.bfloat16, device=dev)
    f_ms = time_calls(torch, lambda: h3.qk_norm_rope_lora(qkv[:, :H], qkv[:, H:2 * H], dq[:, :H], dq[:, H:2 * H],
                                                         gq, gq, V, heads, v=qkv[:, 2 * H:], dv=dq[:, 2 * H:]),
                      iters, 1)

    def unfused_qkv():
        torch.add(qkv, dq, out=tmp)
        h3.qk_norm_rope(tmp[:, :H], tmp[:, H:2 * H], gq, gq, V, heads)
    u_ms = time_calls(torch, unfused_qkv, iters, 1)
    res["qk_norm_rope"] = {"fused_ms": round(f_ms, 4), "unfused_ms": round(u_ms, 4),
                           "saved_gb": round(2 * V * 3 * H * 2 / 1e9, 3)}
    del qkv, dq, tmp
    # residual-modulation consumer (out projection -> x1 and the FFN norm)
    x, br, d = rnd((L, H)), rnd((L, H)), rnd((L, H), 0.05)
    mod = torch.randn((1, 6, H), generator=gen, device=dev) * 0.1
    x1, hh, tmp = (torch.empty((L, H), dtype=torch.bfloat16, device=dev) for _ in range(3))
    f_ms = time_calls(torch, lambda: h3.fused_modulate_norm_lora(x, br, d, mod[:, 2], x1, V, shift=mod[:, 0],
                                                                scale=mod[:, 1], h_out=hh, ld_mod_group=6 * H),
                      iters, 1)

    def unfused_mn():
        torch.add(br, d, out=tmp)
        h3.fused_modulate_norm(x, mod[:, 0], mod[:, 1], hh, V, branch=tmp, gate=mod[:, 2], x1_out=x1,
                               ld_mod_group=6 * H)
    u_ms = time_calls(torch, unfused_mn, iters, 1)
    res["modulate_norm"] = {"fused_ms": round(f_ms, 4), "unfused_ms": round(u_ms, 4),
                            "saved_gb": round(2 * V * H * 2 / 1e9, 3)}
    del x, br, d, x1, hh, tmp
    # SwiGLU consumer
    u, du, tmp = rnd((L, 2 * F), 2.0), rnd((L, 2 * F), 0.05), torch.empty((L, 2 * F), dtype=torch.bfloat16,
                                                                            device=dev)
    g = torch.empty((L, F), dtype=torch.bfloat16, device=dev)
    f_ms = time_calls(torch, lambda: h3.swiglu_lora(u, du, g, V, F), iters, 1)

    def unfused_sw():
        torch.add(u, du, out=tmp)
        h3.swiglu(tmp, g, V, F)
    u_ms = time_calls(torch, unfused_sw, iters, 1)
    res["swiglu"] = {"fused_ms": round(f_ms, 4), "unfused_ms": round(u_ms, 4),
                     "saved_gb": round(2 * V * 2 * F * 2 / 1e9, 3)}
    del u, du, tmp, g
    return res


def reference_kv_cache(torch, h3, dev, dims, weights, mod, gen, L, V, H, n_ref=14344):
    """Reference K/V caching at the benchmarked sequence plus one image's
    reference tokens (14,344): the first denoising step runs the full sequence
    [text 512 | reference | audio and video] and exports the reference rows'
    K/V; later steps run only the generation rows at their original positions
    and attend over [cached reference K/V ; own rows]."""
    n_text = 512
    Lf, Vf = L + n_ref, V + n_ref
    xf = torch.randn((Lf, H), generator=gen, device=dev).to(torch.bfloat16)
    yf = torch.empty_like(xf)
    ek = torch.empty((n_ref, H), dtype=torch.bfloat16, device=dev)
    ev = torch.empty_like(ek)
    exp = (ek, ev, n_text, n_ref)
    wsf = torch.empty(h3.workspace_bytes(dims, Lf), dtype=torch.uint8, device=dev)
    full_ms = time_calls(torch, lambda: h3.block_forward(dims, weights, xf, yf, mod, 1, Vf, wsf, kv_export=exp), 2, 1)
    del wsf
    keep = torch.cat([torch.arange(0, n_text), torch.arange(n_text + n_ref, Lf)]).to(dev)
    xc = xf[keep].contiguous()
    yc = torch.empty_like(xc)
    pos = keep.to(torch.int32)
    groups = [(0, V, [(ek, ev, 0, n_ref), ("self", 0, V)])]
    wsc = torch.empty(h3.workspace_bytes(dims, L, groups), dtype=torch.uint8, device=dev)
    cached_ms = time_calls(torch, lambda: h3.block_forward(dims, weights, xc, yc, mod, 1, V, wsc, groups=groups,
                                                           pos=pos), 2, 1)
    del wsc, xf, yf, xc, yc
    return {"reference_tokens": n_ref, "generation_tokens": V, "full_step_ms": round(full_ms, 3),
            "cached_step_ms": round(cached_ms, 3), "speedup": round(full_ms / cached_ms, 3)}


def block_sparse(torch, h3, dev, q, k, v, o, V, heads, dense_ms, iters, block, prefix=1536):
    """Sol-Attn block-sparse attention on the block's own q~, k~, v (after
    QK-norm and RoPE) at the pages' refinement tau schedule. The prefix is
    the workload's 512 text + 1,024 audio rows. Reports the selection and
    attention times, the fraction of target KV blocks selected, and the
    attention's rate on the work it does (4 * 128 flops per query-key pair
    actually attended)."""
    nq, nk = h3.sparse_geometry(V, prefix)
    T = V - prefix
    blocks = torch.empty((heads, nq, nk), dtype=torch.int16, device=dev)
    counts = torch.empty((heads, nq), dtype=torch.int32, device=dev)
    sws = torch.empty(h3.sparse_select_workspace_bytes(V, prefix, heads), dtype=torch.uint8, device=dev)
    aws = torch.empty(h3.sparse_attention_workspace_bytes(V, prefix, heads), dtype=torch.uint8, device=dev)
    rows_b = torch.full((nq,), 256.0, dtype=torch.float64)
    rows_b[-1] = T - 256 * (nq - 1)
    last_len = T - 64 * (nk - 1)
    out = {"prefix_rows": prefix, "target_rows": T, "query_block": h3.H3_SPARSE_Q_BLOCK,
           "kv_block": h3.H3_SPARSE_K_BLOCK, "dense_attention_ms": round(dense_ms, 3), "tau": {}}
    for tau in (1.0, 1.25, 1.5):
        sel_ms = time_calls(torch, lambda: h3.sparse_select(q, k, V, prefix, heads, tau, blocks, counts, sws), iters, 1)
        att_ms = time_calls(torch, lambda: h3.sparse_attention(q, k, v, o, V, prefix, heads, blocks, counts,
                                                               workspace=aws), iters, 1)
        c = counts.cpu().to(torch.float64)
        # lists are ascending: the short last KV block is selected when it ends the list
        tail = blocks.cpu().to(torch.int64).gather(2, (c.long() - 1).clamp(min=0).unsqueeze(-1)).squeeze(-1)
        has_last = ((c > 0) & (tail == nk - 1)).to(torch.float64)
        keys = prefix + 64.0 * c - (64 - last_len) * has_last
        pairs = float((keys * rows_b).sum()) + heads * prefix * V
        tf = 4.0 * 128 * pairs / (att_ms * 1e-3) / 1e12
        out["tau"][str(tau)] = {"select_ms": round(sel_ms, 3), "attention_ms": round(att_ms, 3),
                                "kv_block_density": round(float(c.sum()) / (heads * nq * nk), 4),
                                "attended_fraction": round(pairs / (heads * V * V), 4),
                                "attention_tflops_on_attended": round(tf, 1),
                                "speedup_vs_dense": round(dense_ms / (sel_ms + att_ms), 2)}
    # the whole block with Sol-Attn attention (tau = 1.0), against the dense block
    dims, weights, x, y, mod, dense_block_ms = block
    L = x.shape[0]
    wsb = torch.empty(h3.block_sparse_workspace_bytes(dims, L, V, prefix), dtype=torch.uint8, device=dev)
    blk_ms = time_calls(torch, lambda: h3.block_forward_sparse(dims, weights, x, y, mod, 1, V, prefix, 1.0, wsb),
                        iters, 1)
    del wsb
    out["block_tau_1.0"] = {"block_ms": round(blk_ms, 3), "dense_block_ms": round(dense_block_ms, 3),
                            "speedup": round(dense_block_ms / blk_ms, 3)}
    return out


def mxfp8_gemms(torch, h3, dev, w, bufs, mod, L, V, H, F, bf16_ms, iters, dims, block_ms, fp8_ceiling=None):
    """The block's four projections as MXFP8 GEMMs (E4M3 with one E8M0 scale
    per 32 along K) at the benchmark's shapes, on the block's own
    activations. Weights are quantized once, outside the timing (they are
    constants of the model); activations by h3_mxfp8_quantize, timed
    separately."""
    hbuf, o, x, x1, h2, g, y = bufs

    def quant(t, rows_valid):
        rows, K = t.shape
        q = torch.empty((rows, K), dtype=torch.uint8, device=dev)
        sc = torch.empty(h3.mx_scales_shape(rows, K), dtype=torch.uint8, device=dev)
        h3.mxfp8_quantize(t, rows_valid, q, sc)
        return q, sc

    wq = {k: quant(w[k], w[k].shape[0]) for k in ("w_qkv", "w_o", "w_up", "w_down")}
    aq = {"h": quant(hbuf, V), "o": quant(o, V), "h2": quant(h2, V), "g": quant(g, V)}
    qkv = torch.empty((L, 3 * H), dtype=torch.bfloat16, device=dev)
    gout = torch.empty((L, F), dtype=torch.bfloat16, device=dev)
    x1o = torch.empty((L, H), dtype=torch.bfloat16, device=dev)
    yo = torch.empty((L, H), dtype=torch.bfloat16, device=dev)
    calls = {
        "gemm_qkv": (lambda: h3.linear_mxfp8(*aq["h"], *wq["w_qkv"], qkv, V), 2.0 * V * H * 3 * H),
        "gemm_out_residual": (lambda: h3.linear_mxfp8(*aq["o"], *wq["w_o"], x1o, V, h3.H3_EPI_RESIDUAL, resid=x,
                                                      gate=mod[:, 2], ld_gate_group=6 * H), 2.0 * V * H * H),
        "gemm_up_swiglu": (lambda: h3.linear_mxfp8(*aq["h2"], *wq["w_up"], gout, V, h3.H3_EPI_SWIGLU),
                           2.0 * V * H * 2 * F),
        "gemm_down_residual": (lambda: h3.linear_mxfp8(*aq["g"], *wq["w_down"], yo, V, h3.H3_EPI_RESIDUAL, resid=x1,
                                                       gate=mod[:, 5], ld_gate_group=6 * H), 2.0 * V * F * H),
    }
    out = {"peak_fp8_tflops": PEAK_FP8_TFLOPS, "measured_fp8_ceiling_tflops": fp8_ceiling, "gemms": {}}
    tot_mx, tot_bf = 0.0, 0.0
    for k, (fn, fl) in calls.items():
        t = time_calls(torch, fn, iters, 1)
        tf = fl / (t * 1e-3) / 1e12
        out["gemms"][k] = {"ms": round(t, 4), "tflops": round(tf, 1), "frac_fp8_mfma": round(tf / PEAK_FP8_TFLOPS, 4),
                           "bf16_ms": round(bf16_ms[k], 4), "speedup_vs_bf16": round(bf16_ms[k] / t, 3)}
        if fp8_ceiling:
            out["gemms"][k]["frac_fp8_ceiling"] = round(tf / fp8_ceiling, 4)
        tot_mx += t
        tot_bf += bf16_ms[k]
    qt = {}
    for name, t in (("h", hbuf), ("g", g)):
        q, sc = aq[name]
        qt[name] = round(time_calls(torch, lambda: h3.mxfp8_quantize(t, V, q, sc), iters, 1), 4)
    out["quantize_ms"] = qt
    out["gemm_total_ms"] = round(tot_mx, 3)
    out["bf16_gemm_total_ms"] = round(tot_bf, 3)
    # the whole MXFP8 block (fused producers, same attention)
    wmx = dict(wq)
    wmx.update({k: w[k] for k in ("q_gain", "k_gain")})
    weights_mx = h3.make_weights_mx(wmx)
    wsm = torch.empty(h3.block_mxfp8_workspace_bytes(dims, L, V, 1536), dtype=torch.uint8, device=dev)
    blk = time_calls(torch, lambda: h3.block_forward_mxfp8(dims, weights_mx, x, y, mod, 1, V, wsm), iters, 1)
    # the pages' refinement block: MXFP8 projections and Sol-Attn attention
    # (prefix 512 text + 1,024 audio rows, tau 1.0)
    blk_sp = time_calls(torch, lambda: h3.block_forward_mxfp8(dims, weights_mx, x, y, mod, 1, V, wsm, prefix_len=1536,
                                                              tau=1.0), iters, 1)
    del wsm
    out["block_ms"] = round(blk, 3)
    out["dense_bf16_block_ms"] = round(block_ms, 3)
    out["block_speedup"] = round(block_ms / blk, 3)
    out["block_sparse_tau_1.0_ms"] = round(blk_sp, 3)
    out["block_sparse_tau_1.0_speedup"] = round(block_ms / blk_sp, 3)
    return out


def qkv_fill_sweep(torch, h3, dev, gen, H: int) -> int:
    """The QKV projection's time against the fill of its last round of 256
    workgroup slots (63 tiles per 256-row tile row): rounds of 63 to 252
    tiles alone, then whole rounds followed by a partial one."""
    rows = [256, 512, 768, 1024, 4096, 4352, 4608, 5120, 5376, 5424]
    Lm = max(rows)
    h = torch.randn((Lm, H), generator=gen, device=dev).to(torch.bfloat16)
    wq = (0.02 * torch.randn((3 * H, H), generator=gen, device=dev)).to(torch.bfloat16)
    qkv = torch.empty((Lm, 3 * H), dtype=torch.bfloat16, device=dev)
    out = []
    for m in rows:
        ms = time_calls(torch, lambda: h3.linear(h[:m], wq, qkv[:m], m), 10, 2)  # no padding rows to zero
        tiles = (m + 255) // 256 * 63
        out.append({"rows": m, "tiles": tiles, "rounds": round(tiles / 256, 3), "ms": round(ms, 4)})
        progress(f"qkv fill sweep: {m} rows, {tiles} tiles, {ms:.4f} ms")
    print(json.dumps({"qkv_fill_sweep": out}), flush=True)
    return 0


def progress(msg: str) -> None:
    """One line on stderr per finished section (stdout carries only the JSON)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def streaming_chunk(torch, h3, dev, gen, dims, weights, H, heads, F, iters):
    """The chunked streaming variant at full width: a current chunk of
    [cond 256 | audio 128 | video 5 x 1,008] rows whose video queries also
    attend to 15,120 history rows of K/V; cond and audio attend over the
    current chunk only. One chunk is 4 denoise forwards plus 1 refresh forward
    that exports the video rows' k~ and v. Also times the grouped attention
    alone (2.27 TFLOP per forward)."""
    cond, audio, video, hist = 256, 128, 5040, 15120
    L = cond + audio + video
    x = torch.randn((L, H), generator=gen, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    hk = torch.randn((hist, H), generator=gen, device=dev).to(torch.bfloat16)
    hv = torch.randn((hist, H), generator=gen, device=dev).to(torch.bfloat16)
    mod = (0.1 * torch.randn((1, 6, H), generator=gen, device=dev)).float()
    ek = torch.empty((video, H), dtype=torch.bfloat16, device=dev)
    ev = torch.empty_like(ek)
    cur = ("self", 0, L)
    groups = [(0, cond, [cur]), (cond, cond + audio, [cur]), (cond + audio, L, [(hk, hv, 0, hist), cur])]
    pos = (torch.arange(L, device=dev) + hist).to(torch.int32)
    ws = torch.empty(h3.workspace_bytes(dims, L, groups), dtype=torch.uint8, device=dev)
    # SolarWM stage 3: the history is staged once per chunk (V^T and key norms)
    # and read in place by the chunk's five forwards
    vt = torch.empty(h3.kv_stage_bytes(hist, heads) // 2, dtype=torch.bfloat16, device=dev)
    km = torch.empty(heads, dtype=torch.float32, device=dev)
    groups_st = [(0, cond, [cur]), (cond, cond + audio, [cur]),
                 (cond + audio, L, [(hk, hv, 0, hist, (vt, km)), cur])]

    def chunk():
        h3.kv_stage(hk, hv, heads, vt=vt, kmax2=km)
        for _ in range(4):
            h3.block_forward(dims, weights, x, y, mod, 1, L, ws, groups=groups_st, pos=pos)
        h3.block_forward(dims, weights, x, y, mod, 1, L, ws, groups=groups_st, pos=pos,
                         kv_export=(ek, ev, cond + audio, video))

    def chunk_restaged():
        for _ in range(4):
            h3.block_forward(dims, weights, x, y, mod, 1, L, ws, groups=groups, pos=pos)
        h3.block_forward(dims, weights, x, y, mod, 1, L, ws, groups=groups, pos=pos,
                         kv_export=(ek, ev, cond + audio, video))

    chunk_ms = time_calls(torch, chunk, iters, 1)
    restaged_ms = time_calls(torch, chunk_restaged, iters, 1)
    off, lds = h3.workspace_layout(dims, L, groups)
    qkv = ws[off[h3.H3_WS_QKV]:off[h3.H3_WS_QKV] + L * 3 * H * 2].view(torch.bfloat16).view(L, 3 * H)
    o = ws[off[h3.H3_WS_O]:off[h3.H3_WS_O] + L * H * 2].view(torch.bfloat16).view(L, H)
    aws = torch.empty(h3.attention_workspace_bytes(L, heads, groups_st), dtype=torch.uint8, device=dev)
    attn_ms = time_calls(torch, lambda: h3.attention(qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], o, L, heads,
                                                     groups=groups_st, workspace=aws), iters, 1)
    attn_f = 4.0 * H * (video * (hist + L) + (cond + audio) * L)
    gemm_f = 2.0 * L * H * (4 * H + 3 * F)
    fwd_ms = chunk_ms / 5
    del ws, aws, x, y, hk, hv, vt, km
    return {"workload": "streaming chunk [cond 256 | audio 128 | video 5 x 1,008] over 15,120 history rows, "
                        "4 denoise + 1 refresh forward (one block)",
            "chunk_ms": round(chunk_ms, 3), "forward_ms": round(fwd_ms, 3),
            "history": "staged once per chunk (h3_kv_stage), read in place by the 5 forwards",
            "chunk_ms_history_staged_per_forward": round(restaged_ms, 3),
            "forward_tflops": round((gemm_f + attn_f) / (fwd_ms * 1e-3) / 1e12, 1),
            "grouped_attention": {"ms": round(attn_ms, 4), "tflop": round(attn_f / 1e12, 3),
                                  "tflops": round(attn_f / (attn_ms * 1e-3) / 1e12, 1),
                                  "frac_mfma": round(attn_f / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}}


def full_4096(torch, h3, dev, gen, dims, weights, w, H, heads, F, iters, n_rot=4):
    """The full-width block at 4,096 valid tokens (no padding). Its
    activations (44 MB) would stay in the 256 MB last-level cache between
    calls, so the block is timed over n_rot input/output sets in turn. Also
    the four projections and attention alone, on the block's own buffers."""
    L = V = 4096
    xs = [torch.randn((L, H), generator=gen, device=dev).to(torch.bfloat16) for _ in range(n_rot)]
    ys = [torch.empty_like(xs[0]) for _ in range(n_rot)]
    mod = (0.1 * torch.randn((1, 6, H), generator=gen, device=dev)).float()
    ws = torch.empty(h3.workspace_bytes(dims, L), dtype=torch.uint8, device=dev)
    turn = [0]

    def block():
        i = turn[0] % n_rot
        turn[0] += 1
        h3.block_forward(dims, weights, xs[i], ys[i], mod, 1, V, ws)

    blk = time_calls(torch, block, 4 * iters, n_rot)
    off, lds = h3.workspace_layout(dims, L)

    def wsv(i, cols):
        return ws[off[i]:off[i] + L * cols * 2].view(torch.bfloat16).view(L, cols)

    hbuf, qkv, o, x1, h2, g = (wsv(h3.H3_WS_H, H), wsv(h3.H3_WS_QKV, 3 * H), wsv(h3.H3_WS_O, H),
                               wsv(h3.H3_WS_X1, H), wsv(h3.H3_WS_H2, H), wsv(h3.H3_WS_G, F))
    vt_ws = ws[off[h3.H3_WS_VT]:off[h3.H3_WS_VT] + lds[h3.H3_WS_VT]]
    x, y = xs[0], ys[0]
    lws = torch.empty(128 << 20, dtype=torch.uint8, device=dev)  # stream-K partial sums
    calls = {
        "gemm_qkv": (lambda: h3.linear(hbuf, w["w_qkv"], qkv, V, workspace=lws), 2.0 * V * H * 3 * H),
        "attention": (lambda: h3.attention(qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], o, V, heads,
                                           workspace=vt_ws), 4.0 * V * V * H),
        "gemm_out_residual": (lambda: h3.linear(o, w["w_o"], x1, V, h3.H3_EPI_RESIDUAL, resid=x, gate=mod[:, 2],
                                                ld_gate_group=6 * H, workspace=lws), 2.0 * V * H * H),
        "gemm_up_swiglu": (lambda: h3.linear(h2, w["w_up"], g, V, h3.H3_EPI_SWIGLU, workspace=lws),
                           2.0 * V * H * 2 * F),
        "gemm_down_residual": (lambda: h3.linear(g, w["w_down"], y, V, h3.H3_EPI_RESIDUAL, resid=x1,
                                                 gate=mod[:, 5], ld_gate_group=6 * H, workspace=lws),
                               2.0 * V * F * H),
    }
    kern = {}
    for k, (fn, fl) in calls.items():
        t = time_calls(torch, fn, iters, 1)
        tf = fl / (t * 1e-3) / 1e12
        kern[k] = {"ms": round(t, 4), "tflops": round(tf, 1), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)}
    gemm_f, attn_f = block_flops(V, H, F)
    tf = (gemm_f + attn_f) / (blk * 1e-3) / 1e12
    del xs, ys, ws
    return {"workload": "one full-width H3 DiT block forward at 4,096 valid tokens (no padding)",
            "block_ms": round(blk, 4), "tflop": round((gemm_f + attn_f) / 1e12, 3), "tflops": round(tf, 1),
            "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4), "input_sets_rotated": n_rot, "kernels": kern}


def stacked_denoise(torch, h3, dev, dims, x, L, V, H, F, n_blocks=50, n_steps=4):
    """The stacked denoise loop: n_blocks random-init blocks (46 GB of BF16
    weights at 50) resident at once, n_steps denoising steps at the
    benchmarked sequence, each step one h3_stack_forward over all blocks with
    that step's slice of an FP32 AdaLN table [blocks][steps][6][H]. Reports
    DiT forwards per second (one forward = all blocks once) over the whole
    loop, timed once after a one-block warmup."""
    g = torch.Generator(device=dev)
    g.manual_seed(SEED + 1)

    def draw(shape, std, mean=0.0):
        t = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).mul_(std)
        if mean:
            t.add_(mean)
        return t.to(torch.bfloat16)

    blocks = [{"w_qkv": draw((3 * H, H), 0.02), "w_o": draw((H, H), 0.02), "w_up": draw((2 * F, H), 0.02),
               "w_down": draw((H, F), 0.02), "q_gain": draw((128,), 0.02, 1.0), "k_gain": draw((128,), 0.02, 1.0)}
              for _ in range(n_blocks)]
    wbytes = sum(t.numel() * 2 for b in blocks for t in b.values())
    arr = h3.make_weight_stack([h3.make_weights(b) for b in blocks])
    mod = (0.1 * torch.randn((n_blocks, n_steps, 6, H), generator=g, device=dev)).float()
    ws = torch.empty(h3.workspace_bytes(dims, L), dtype=torch.uint8, device=dev)
    xs = x.clone()
    ld_blk = n_steps * 6 * H
    h3.stack_forward(dims, h3.make_weight_stack([h3.make_weights(blocks[0])]), xs, mod[0, 0], 0, 1, V, ws)
    xs.copy_(x)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(n_steps):
        h3.stack_forward(dims, arr, xs, mod[0, s], ld_blk, 1, V, ws)
    t1.record()
    torch.cuda.synchronize()
    loop_ms = t0.elapsed_time(t1)
    gemm_f, attn_f = block_flops(V, H, F)
    per_block = loop_ms / (n_blocks * n_steps)
    out = {"workload": f"{n_blocks} resident blocks, {n_steps} denoising steps, 58,758 valid tokens in 58,816",
           "resident_weight_gb": round(wbytes / 1e9, 2), "loop_s": round(loop_ms / 1e3, 3),
           "dit_forwards_per_s": round(n_steps / (loop_ms * 1e-3), 4), "ms_per_block": round(per_block, 3),
           "tflops": round((gemm_f + attn_f) / (per_block * 1e-3) / 1e12, 1),
           "finite": bool(torch.isfinite(xs[:V].float()).all().item())}
    del blocks, ws, xs, mod
    torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-iters", type=int, default=5)
    ap.add_argument("--no-next", action="store_true",
                    help="skip the measurements of the rows beyond the block (LoRA consumer fusion)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (streaming chunk, 50-block stacked denoise loop)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (the known-size reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--qkv-fill-sweep", action="store_true",
                    help="instead of the bench: time the QKV projection (K 5,376, N 16,128, no workspace) at row "
                         "counts whose last round of 256 tiles is filled to different degrees, one JSON line")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        return 2

    import torch
    from video_diffusion_transformer_dit_amd import h3

    H, heads, F = 5376, 42, 21504
    L, V = 58816, 58758
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(SEED)
    if a.qkv_fill_sweep:
        return qkv_fill_sweep(torch, h3, dev, gen, H)

    def normal(shape, std=1.0, mean=0.0, dtype=torch.bfloat16):
        t = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        if mean != 0.0:
            t.add_(mean)
        return t.to(dtype)

    w = {"w_qkv": normal((3 * H, H), 0.02), "w_o": normal((H, H), 0.02), "w_up": normal((2 * F, H), 0.02),
         "w_down": normal((H, F), 0.02), "q_gain": normal((128,), 0.02, 1.0), "k_gain": normal((128,), 0.02, 1.0)}
    x = normal((L, H))
    mod = normal((1, 6, H), 0.1, dtype=torch.float32)
    y = torch.empty_like(x)
    dims = h3.make_dims(H, heads, F)
    weights = h3.make_weights(w)
    ws = torch.empty(h3.workspace_bytes(dims, L), dtype=torch.uint8, device=dev)
    off, lds = h3.workspace_layout(dims, L)

    def wsv(i, cols):
        return ws[off[i]:off[i] + L * cols * 2].view(torch.bfloat16).view(L, cols)

    def step():
        h3.block_forward(dims, weights, x, y, mod, 1, V, ws)

    ms, step_ms = time_calls(torch, step, a.steps, a.warmup, per_call=True)
    progress(f"block timed: {ms:.3f} ms over {a.steps} steps")

    # Per-kernel breakdown: the block's launches, one at a time, same buffers.
    hbuf, qkv, o, x1, h2, g = (wsv(h3.H3_WS_H, H), wsv(h3.H3_WS_QKV, 3 * H), wsv(h3.H3_WS_O, H),
                               wsv(h3.H3_WS_X1, H), wsv(h3.H3_WS_H2, H), wsv(h3.H3_WS_G, F))
    kit = a.kernel_iters
    k_ms = {}
    k_ms["modnorm"] = time_calls(torch, lambda: h3.fused_modulate_norm(
        x, mod[:, 0], mod[:, 1], hbuf, V, ld_mod_group=6 * H), kit, 1)
    lws = torch.empty(128 << 20, dtype=torch.uint8, device=dev)  # stream-K partial sums (at most 128 MiB)
    k_ms["gemm_qkv"] = time_calls(torch, lambda: h3.linear(hbuf, w["w_qkv"], qkv, V, workspace=lws), kit, 1)
    k_ms["qk_norm_rope"] = time_calls(torch, lambda: h3.qk_norm_rope(
        qkv[:, :H], qkv[:, H:2 * H], w["q_gain"], w["k_gain"], V, heads), kit, 1)
    vt_ws = ws[off[h3.H3_WS_VT]:off[h3.H3_WS_VT] + lds[h3.H3_WS_VT]]
    k_ms["attention"] = time_calls(torch, lambda: h3.attention(
        qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], o, V, heads, workspace=vt_ws), kit, 1)
    # The attention kernel's own launches: the same call over K/V staged
    # beforehand (V^T planes and key-norm maxima from h3_kv_stage), so it runs
    # no pre-pass, only the fixed-reference launch, the online launch (every
    # workgroup leaves at once here) and three tiny fills.
    st_vt, st_km = h3.kv_stage(qkv[:V, H:2 * H], qkv[:V, 2 * H:], heads)
    st_groups = [(0, V, [(qkv[:, H:2 * H], qkv[:, 2 * H:], 0, V, (st_vt, st_km))])]
    st_ws = torch.empty(h3.attention_workspace_bytes(V, heads, st_groups), dtype=torch.uint8, device=dev)
    k_ms["attention_kernel"] = time_calls(torch, lambda: h3.attention(
        qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], o, V, heads, groups=st_groups, workspace=st_ws), kit, 1)
    del st_vt, st_km, st_ws
    k_ms["gemm_out_residual"] = time_calls(torch, lambda: h3.linear(
        o, w["w_o"], x1, V, h3.H3_EPI_RESIDUAL, resid=x, gate=mod[:, 2], ld_gate_group=6 * H, workspace=lws), kit, 1)
    k_ms["modnorm2"] = time_calls(torch, lambda: h3.fused_modulate_norm(
        x1, mod[:, 3], mod[:, 4], h2, V, ld_mod_group=6 * H), kit, 1)
    k_ms["gemm_up_swiglu"] = time_calls(torch, lambda: h3.linear(h2, w["w_up"], g, V, h3.H3_EPI_SWIGLU,
                                                                 workspace=lws), kit, 1)
    k_ms["gemm_down_residual"] = time_calls(torch, lambda: h3.linear(
        g, w["w_down"], y, V, h3.H3_EPI_RESIDUAL, resid=x1, gate=mod[:, 5], ld_gate_group=6 * H, workspace=lws),
        kit, 1)

    progress("per-kernel breakdown timed")
    # The online-softmax form on the same shape: q scaled by 8 puts every
    # workgroup's score bound above the fixed-reference range (as trained
    # models with large QK-norm gains would).
    q8 = torch.empty_like(qkv[:, :H])
    q8.copy_(qkv[:, :H]).mul_(8.0)
    k_ms["attention_online"] = time_calls(torch, lambda: h3.attention(
        q8, qkv[:, H:2 * H], qkv[:, 2 * H:], o, V, heads, workspace=vt_ws), kit, 1)
    del q8
    h3.attention(qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], o, V, heads, workspace=vt_ws)  # o back to the block's
    # Measured ceilings on this GPU: a plain device copy (what the memory-bound
    # kernels can hope for) and the vendor library's BF16 GEMM on the QKV shape
    # (hipBLASLt through torch.matmul, no epilogue).
    csrc = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)   # 1 GiB
    cdst = torch.empty_like(csrc)
    copy_ms = time_calls(torch, lambda: cdst.copy_(csrc), 5, 1)
    copy_gbs = 2.0 * csrc.numel() * 2 / (copy_ms * 1e-3) / 1e9
    del csrc, cdst
    hv, wq, qv = hbuf[:V], w["w_qkv"], qkv[:V]
    lib_ms = time_calls(torch, lambda: torch.matmul(hv, wq.t(), out=qv), 3, 1)
    lib_tf = 2.0 * V * H * 3 * H / (lib_ms * 1e-3) / 1e12
    # The matrix cores' sustained BF16 rate on operands with varying bits and
    # no memory traffic (h3_mfma_ceiling: the GEMM tile's register pattern):
    # under load the clock is set by power, which this rate includes.
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    mf_flops = h3.mfma_ceiling(20000, sink)
    mf_ms = time_calls(torch, lambda: h3.mfma_ceiling(20000, sink), 40, 5)
    mf_tf = mf_flops / (mf_ms * 1e-3) / 1e12
    mf8_flops = h3.mfma_ceiling(10000, sink, h3.H3_CEIL_FP8)
    mf8_ms = time_calls(torch, lambda: h3.mfma_ceiling(10000, sink, h3.H3_CEIL_FP8), 40, 5)
    mf8_tf = mf8_flops / (mf8_ms * 1e-3) / 1e12
    del sink

    gemm_f, attn_f = block_flops(V, H, F)
    gflops = {"gemm_qkv": 2.0 * V * H * 3 * H, "gemm_out_residual": 2.0 * V * H * H,
              "gemm_up_swiglu": 2.0 * V * H * 2 * F, "gemm_down_residual": 2.0 * V * F * H, "attention": attn_f,
              "attention_kernel": attn_f, "attention_online": attn_f}
    ebytes = elementwise_bytes(V, H, F)
    kernels = {}
    for k, t in k_ms.items():
        d = {"ms": round(t, 4)}
        if k in gflops:
            tf = gflops[k] / (t * 1e-3) / 1e12
            d.update(tflops=round(tf, 1), frac_mfma=round(tf / PEAK_BF16_TFLOPS, 4),
                     frac_mfma_ceiling=round(tf / mf_tf, 4))
            if k.startswith("gemm"):
                d.update(frac_library_gemm=round(tf / lib_tf, 4))
        if k in ebytes:
            gbs = ebytes[k] / (t * 1e-3) / 1e9
            d.update(gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4), frac_copy=round(gbs / copy_gbs, 4))
        kernels[k] = d

    attn_tf = gflops["attention"] / (k_ms["attention_kernel"] * 1e-3) / 1e12
    gemm_ms = sum(k_ms[k] for k in k_ms if k.startswith("gemm"))
    total_tf = (gemm_f + attn_f) / (ms * 1e-3) / 1e12
    out = {
        "metric": "ms per DiT block at 58,816 tokens",
        "value": round(ms, 3),
        "unit": "ms/block",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "one full-width H3 DiT block forward, 58,758 valid tokens in a 58,816-token "
                               "buffer", "hidden": H, "heads": heads, "head_dim": 128, "ffn": F, "L_buf": L,
                   "valid_len": V, "rot_dim": 64, "weights": "random-init N(0,0.02)"},
        "step_ms": {"median": round(statistics.median(step_ms), 3), "min": round(min(step_ms), 3),
                    "max": round(max(step_ms), 3)},
        "ceilings": {"copy_gbs": round(copy_gbs, 1), "copy_frac_hbm": round(copy_gbs / PEAK_HBM_GBS, 4),
                     "library_gemm_tflops": round(lib_tf, 1),
                     "mfma_varying_operands_tflops": round(mf_tf, 1),
                     "mfma_varying_operands_frac_peak": round(mf_tf / PEAK_BF16_TFLOPS, 4),
                     "mfma_varying_operands": "h3_mfma_ceiling: v_mfma_f32_32x32x16_bf16 in the GEMM tile's register "
                                              "pattern on BF16 operands with varying bits, no memory traffic, "
                                              "one workgroup per CU",
                     "mfma_fp8_varying_operands_tflops": round(mf8_tf, 1),
                     "mfma_fp8_varying_operands_frac_peak": round(mf8_tf / PEAK_FP8_TFLOPS, 4),
                     "library_gemm": "hipBLASLt (torch.matmul) BF16 on the QKV shape, no epilogue"},
        "block_tflops": round(total_tf, 1),
        "block_frac_mfma": round(total_tf / PEAK_BF16_TFLOPS, 4),
        "attention_tflops": round(gflops["attention"] / (k_ms["attention"] * 1e-3) / 1e12, 1),
        "gemm_tflops": round(gemm_f / (gemm_ms * 1e-3) / 1e12, 1),
        "kernels": kernels,
        "roofline": {"kernel": "attention_fwd_kernel<false, true, false> (dense, fixed softmax reference)",
                     "timed_as": "kernels.attention_kernel: the attention launches over K/V staged beforehand; "
                                 "kernels.attention is the whole call with its V^T and key-norm pre-passes",
                     "bound": "mfma", "achieved": round(attn_tf, 1),
                     "measured_ceiling": {"value": round(mf_tf, 1), "unit": "TFLOP/s",
                                          "frac": round(attn_tf / mf_tf, 4),
                                          "what": "ceilings.mfma_varying_operands"},
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": counter_traffic("void attention_fwd_kernel<false, true, false>",
                                                ["attention_fixed.hip", "h3_attention_kernel.h"]),
                     "traffic_unit": "bytes per launch (FETCH_SIZE x2 + WRITE_SIZE x1, copy-calibrated)",
                     "work_per_launch": "4 * 58758^2 * 5376 = 7.424e13 flop (QK^T and PV over valid rows)"},
    }
    if not a.no_configs:
        out["configs"] = {"full_4096": full_4096(torch, h3, dev, gen, dims, weights, w, H, heads, F, kit)}
        progress("4,096-token block timed")
        out["configs"]["streaming_chunk"] = streaming_chunk(torch, h3, dev, gen, dims, weights, H, heads, F, kit)
        progress("streaming chunk timed")
    if not a.no_next:
        out["next"] = {"lora_consumer_fusion": lora_consumers(torch, h3, dev, gen, L, V, H, heads, F, kit)}
        progress("LoRA consumer fusion timed")
        out["next"]["block_sparse_attention"] = block_sparse(torch, h3, dev, qkv[:, :H], qkv[:, H:2 * H],
                                                             qkv[:, 2 * H:], o, V, heads, k_ms["attention"], kit,
                                                             (dims, weights, x, y, mod, ms))
        progress("block-sparse attention timed")
        out["next"]["mxfp8_gemms"] = mxfp8_gemms(torch, h3, dev, w, (hbuf, o, x, x1, h2, g, y), mod, L, V, H, F,
                                                 k_ms, kit, dims, ms, fp8_ceiling=round(mf8_tf, 1))
        progress("MXFP8 GEMMs timed")
        out["next"]["reference_kv_cache"] = reference_kv_cache(torch, h3, dev, dims, weights, mod, gen, L, V, H)
        progress("reference K/V caching timed")
    if not a.no_configs:
        out["configs"]["stacked_denoise"] = stacked_denoise(torch, h3, dev, dims, x, L, V, H, F)
        progress("stacked denoise loop timed")
    if a.calibration_copy:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)   # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = int(src.numel() * 2)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(configs=not a.no_configs)
        progress("CPU oracle sample timed")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
