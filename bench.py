#!/usr/bin/env python3
"""Benchmark of the E2D2 attention hot path on one MI355X.

Headline (``value``): useful TFLOP/s of the training attention forward -- encoder
block-causal attention and fused decoder attention over [clean | noised] keys in ONE
launch -- at B=8, 16 heads, d_head 64, L=1024, block S=16, bf16, N(0,1) synthetic
inputs resident in HBM.  One step = one such launch.  Useful FLOPs = 4 * d * (allowed
pairs of both masks) * B * H: the attention term of the FLOPs table, (L^2 + L S)/2
pairs per mask ("Encoder-Decoder Diffusion Language Models for Efficient Training and
Inference", Paper-Notes page, 方法详解 §4 训练算法).

Also measured in the same run and reported in the same JSON line:
  * ``denoise``: the inference step at B=32, 16 query / 8 KV heads, d_head 128, cache
    2048, block S=32: 32 denoising steps with fresh block tensors, then the KV-cache
    append; microseconds per step and algorithmic GB/s, with the Infinity Cache warm
    (steady state) and swept out by a 1 GiB read before every step (cold);
  * ``long_train``: the same training forward at B=2, 16/8 heads, d_head 128, L=8192,
    S=64, with LSE (MFMA-bound);
  * ``roofline``: the training kernel's useful TFLOP/s against the bf16 MFMA peak,
    with the kernel's average duration from HIP events on its stream;
  * ``cpu_baseline``: the fp64 CPU oracle timed on the host cores on a bounded sample
    of the training workload.

``python bench.py --gpus N --steps K --warmup W``; the benchmark runs on one GPU only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "train_fwd_traffic.json")
KERNEL_SOURCES = ["masked_attention_amd/csrc/attn_train.hip",
                  "masked_attention_amd/csrc/device_common.h",
                  "masked_attention_amd/csrc/schedule.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pairs_blockcausal(L: int, S: int) -> int:
    """Allowed pairs of one mask (encoder or decoder) per head, counted block by block:
    a row of block b sees (b+1) * S keys (clipped at L) in the encoder and, equally,
    b * S earlier clean keys plus its own block in the decoder."""
    total = 0
    for start in range(0, L, S):
        end = min(L, start + S)
        total += (end - start) * end
    return total


def timed_launches(fn, n, stream):
    """Run fn() n times back to back between two HIP events recorded on ``stream`` (the
    stream the kernels run on), with a synchronisation on both sides; returns (total ms,
    mean ms per launch)."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    return total, total / n


def clock_warmup(replay, min_ms=150.0):
    """Keep the GPU busy for at least min_ms with back-to-back replays right before a
    timed region: the MI355X raises its clocks over the first ~50 ms of sustained work
    and lowers them again after idling, so a cold start would time the ramp."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    replay()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-5) * 1e3
    for _ in range(int(min_ms / one) + 1):
        replay()
    torch.cuda.synchronize()


def graph_of(fn, n):
    """A HIP graph holding n back-to-back calls of fn (kernel launches on the current
    stream), so timed replays measure the GPU and not the Python launch overhead."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up launch outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    return g


def bench_train(B, Hq, Hkv, L, S, d, steps, warmup, seed, with_lse=True, cold=False):
    import torch

    import masked_attention_amd as m
    from synth import TensorKind as K, device_fill, tensor_id

    dev = torch.device("cuda:0")

    def fill(kind, H):
        t = torch.empty((B, H, L, d), dtype=torch.bfloat16, device=dev)
        device_fill(t, seed, tensor_id(kind))
        return t

    qd, qe = fill(K.Q_DEC, Hq), fill(K.Q_ENC, Hq)
    kc, vc, kd, vd = (fill(k, Hkv) for k in (K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC))
    od, oe = torch.empty_like(qd), torch.empty_like(qe)
    ld = torch.empty((B, Hq, L), device=dev) if with_lse else None
    le = torch.empty((B, Hq, L), device=dev) if with_lse else None

    def step():
        m.e2d2_attn_train_fwd(qd, kc, vc, kd, vd, od, S, lse_dec=ld, q_enc=qe, o_enc=oe,
                              lse_enc=le)

    step()
    torch.cuda.synchronize()
    ref = (od.clone(), oe.clone())
    # the timed region: `steps` launches replayed from one HIP graph, bracketed by HIP
    # events on the stream they run on.  Warm-up: `warmup` launches (eager and replayed),
    # and at least 150 ms of replays just before the timed one.
    g = graph_of(step, steps)
    for _ in range(max(1, -(-warmup // steps))):
        g.replay()
    clock_warmup(g.replay)
    stream = torch.cuda.current_stream(dev)
    t0 = time.perf_counter()
    total_ms, _ = timed_launches(g.replay, 1, stream)
    wall = time.perf_counter() - t0
    if not (torch.equal(od, ref[0]) and torch.equal(oe, ref[1])):
        raise RuntimeError("graph replay differs from the eager launch")
    useful = 4.0 * d * 2 * pairs_blockcausal(L, S) * B * Hq
    # kernel_ms: the mean launch duration over the timed region (the launches run back to
    # back from the graph; the kernel trace's per-dispatch average agrees)
    out = dict(total_ms=total_ms, ms_per_step=total_ms / steps, kernel_ms=total_ms / steps,
               useful_flop=useful, wall_s=wall)
    if cold:
        out["cold_ms"] = cold_launch_ms(step, 9, stream)
    return out


def cold_launch_ms(fn, n, stream):
    """Duration of one launch of fn with its inputs in HBM: the median time of a read
    sweep over 1 GiB (which leaves the 256 MB Infinity Cache and the L2s holding other,
    clean lines) followed by fn, minus the median time of the sweep alone, each timed as
    one region between HIP events on ``stream``.  No event sits between the sweep and fn,
    so the difference holds the kernel and not an event's dispatch gap."""
    import torch

    flush = torch.ones(1 << 28, dtype=torch.float32, device=stream.device)
    clock_warmup(fn)

    def region(with_fn):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        flush.sum()
        if with_fn:
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    both = sorted(region(True) for _ in range(n))
    sweep = sorted(region(False) for _ in range(n))
    del flush
    return both[n // 2] - sweep[n // 2]


def bench_train_bwd(B, Hq, Hkv, L, S, d, steps, seed):
    """Training backward (e2d2_attn_train_bwd, encoder and decoder) after one forward;
    `steps` backward launches replayed from one HIP graph.  Useful work: the four
    products dV, dP, dQ, dK over the allowed pairs, 8 * d flop per pair (the score
    recomputation is not counted)."""
    import torch

    import masked_attention_amd as m
    from synth import TensorKind as K, device_fill, tensor_id

    dev = torch.device("cuda:0")

    def fill(kind, H):
        t = torch.empty((B, H, L, d), dtype=torch.bfloat16, device=dev)
        device_fill(t, seed, tensor_id(kind))
        return t

    qd, qe, dod, doe = fill(K.Q_DEC, Hq), fill(K.Q_ENC, Hq), fill(K.DO_DEC, Hq), fill(K.DO_ENC, Hq)
    kc, vc, kd, vd = (fill(k, Hkv) for k in (K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC))
    od, oe = torch.empty_like(qd), torch.empty_like(qe)
    ld = torch.empty((B, Hq, L), device=dev)
    le = torch.empty_like(ld)
    m.e2d2_attn_train_fwd(qd, kc, vc, kd, vd, od, S, lse_dec=ld, q_enc=qe, o_enc=oe, lse_enc=le)
    g = [torch.empty_like(t) for t in (qd, kc, vc, kd, vd, qe)]
    ws = torch.empty(m.e2d2_attn_train_bwd_workspace_bytes(m.BF16, B, Hq, L, True),
                     dtype=torch.uint8, device=dev)

    def step():
        m.e2d2_attn_train_bwd(qd, kc, vc, kd, vd, od, ld, dod, S, g[0], g[1], g[2], g[3], g[4], ws,
                              q_enc=qe, o_enc=oe, lse_enc=le, do_enc=doe, dq_enc=g[5])

    step()
    torch.cuda.synchronize()
    graph = graph_of(step, steps)
    clock_warmup(graph.replay)
    stream = torch.cuda.current_stream(dev)
    total_ms, _ = timed_launches(graph.replay, 1, stream)
    ms = total_ms / steps
    useful = 8.0 * d * 2 * pairs_blockcausal(L, S) * B * Hq
    tf = useful / (ms * 1e-3) / 1e12
    return dict(workload=f"training bwd enc+dec, B{B} Hq{Hq} Hkv{Hkv} d{d} L{L} S{S}, bf16",
                ms_per_step=round(ms, 5), tflops=round(tf, 1),
                frac_of_peak=round(tf / PEAK_BF16_TFLOPS, 4), useful_flop=useful)


def bench_layer_split(B, H, L, S, d, steps, seed):
    """Per-layer attention cost of a decoder-only block-diffusion layer (one fused call
    over the 2L tokens: decoder half + encoder half) against an E2D2 encoder layer
    (encoder half alone) and an E2D2 decoder layer (decoder half alone), each timed
    from a HIP graph of `steps` launches."""
    import torch

    import masked_attention_amd as m
    from synth import TensorKind as K, device_fill, tensor_id

    dev = torch.device("cuda:0")

    def fill(kind):
        t = torch.empty((B, H, L, d), dtype=torch.bfloat16, device=dev)
        device_fill(t, seed, tensor_id(kind))
        return t

    qd, qe, kc, vc, kd, vd = (fill(k) for k in (K.Q_DEC, K.Q_ENC, K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC))
    od, oe = torch.empty_like(qd), torch.empty_like(qe)
    ld = torch.empty((B, H, L), device=dev)
    le = torch.empty_like(ld)
    calls = {
        "bd3lm_layer": lambda: m.e2d2_attn_train_fwd(qd, kc, vc, kd, vd, od, S, lse_dec=ld,
                                                     q_enc=qe, o_enc=oe, lse_enc=le),
        "e2d2_encoder_layer": lambda: m.e2d2_attn_encoder_blockcausal(qe, kc, vc, oe, S, lse=le),
        "e2d2_decoder_layer": lambda: m.e2d2_attn_train_fwd(qd, kc, vc, kd, vd, od, S, lse_dec=ld),
    }
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        g = graph_of(fn, steps)
        clock_warmup(g.replay)
        total, _ = timed_launches(g.replay, 1, stream)
        out[name + "_us"] = round(total / steps * 1e3, 2)
    out["workload"] = f"attention per layer, B{B} H{H} d{d} L{L} S{S} bf16"
    out["bd3lm_over_e2d2_mean_layer"] = round(
        out["bd3lm_layer_us"] / ((out["e2d2_encoder_layer_us"] + out["e2d2_decoder_layer_us"]) / 2), 3)
    return out


def bench_denoise_varlen(steps, seed):
    """The denoise workload's heads (B32 Hq16 Hkv8 d128, block 32) with a cache length of
    its own per sequence, drawn once (seeded) from [1024, 2048], read by the kernel from a
    device array: `steps` steps back to back from one HIP graph, as a decode loop over a
    ragged batch runs them."""
    import numpy as np
    import torch

    import masked_attention_amd as m
    from synth import TensorKind as K, device_fill, tensor_id

    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, S, max_len = 32, 16, 8, 128, 32, 2048
    cap = max_len + S
    lens = np.random.RandomState(seed & 0xFFFFFFFF).randint(1024, max_len + 1, size=B)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=dev)

    def fill(shape, kind, rows=None, **kw):
        t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        device_fill(t, seed, tensor_id(kind, **kw), rows=rows)
        return t

    kc = fill((B, Hkv, cap, d), K.K_CACHE, rows=max_len)
    vc = fill((B, Hkv, cap, d), K.V_CACHE, rows=max_len)
    qs = [fill((B, Hq, S, d), K.Q_BLK, step=t) for t in range(steps)]
    ks = [fill((B, Hkv, S, d), K.K_BLK, step=t) for t in range(steps)]
    vs = [fill((B, Hkv, S, d), K.V_BLK, step=t) for t in range(steps)]
    o = torch.empty((B, Hq, S, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, S), device=dev)
    nws = m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, Hq, Hkv, S, d, max_len)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    stream = torch.cuda.current_stream(dev)
    it = [0]

    def next_step():
        t = it[0] % steps
        m.e2d2_attn_denoise_step_varlen(qs[t], kc, vc, lens_t, max_len, ks[t], vs[t], o,
                                        lse_blk=lse, workspace=ws)
        it[0] += 1

    g = graph_of(next_step, steps)
    g.replay()
    clock_warmup(g.replay)
    per_step = []
    for _ in range(4):
        _, ms = timed_launches(g.replay, 1, stream)
        per_step.append(ms / steps)
    us = sorted(per_step)[len(per_step) // 2] * 1e3
    alg = (int(lens.sum()) * 2 * Hkv * d * 2 + 2 * B * Hkv * S * d * 2 + 2 * B * Hq * S * d * 2
           + B * Hq * S * 4)
    gbs = alg / (us * 1e-6) / 1e9
    return dict(workload="denoise step with per-sequence cache lengths, B32 Hq16 Hkv8 d128 block 32, "
                         "lengths uniform in [1024, 2048] (seeded), bf16",
                lens_min=int(lens.min()), lens_mean=round(float(lens.mean()), 1), lens_max=int(lens.max()),
                us_per_step_warm=round(us, 2), algorithmic_bytes_per_step=alg, gbs_warm=round(gbs, 1),
                frac_of_hbm_peak=round(gbs / PEAK_HBM_GBS, 4))


def bench_denoise(steps_per_block, blocks, warm_blocks, seed):
    import torch

    import masked_attention_amd as m
    from synth import TensorKind as K, device_fill, tensor_id

    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, C, S, T = 32, 16, 8, 128, 2048, 32, steps_per_block
    cap = C + S

    def fill(shape, kind, **kw):
        t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        device_fill(t, seed, tensor_id(kind, **kw))
        return t

    kc = torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    device_fill(kc, seed, tensor_id(K.K_CACHE), rows=C)
    device_fill(vc, seed, tensor_id(K.V_CACHE), rows=C)
    qs = [fill((B, Hq, S, d), K.Q_BLK, step=t) for t in range(T)]
    ks = [fill((B, Hkv, S, d), K.K_BLK, step=t) for t in range(T)]
    vs = [fill((B, Hkv, S, d), K.V_BLK, step=t) for t in range(T)]
    kn, vn = fill((B, Hkv, S, d), K.K_NEW), fill((B, Hkv, S, d), K.V_NEW)
    o = torch.empty((B, Hq, S, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, S), device=dev)
    nws = m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, Hq, Hkv, S, d, C)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    stream = torch.cuda.current_stream(dev)

    def step(t):
        m.e2d2_attn_denoise_step(qs[t], kc, vc, C, ks[t], vs[t], o, lse_blk=lse, workspace=ws)

    def append():
        m.e2d2_kv_cache_append(kc, vc, C, kn, vn)

    for _ in range(warm_blocks):
        for t in range(T):
            step(t)
        append()
    torch.cuda.synchronize()
    # warm: the T steps of a block back to back from one HIP graph (as a decode loop
    # runs them), then the append, each bracketed by HIP events on the launch stream
    it = [0]

    def next_step():
        step(it[0] % T)
        it[0] += 1

    g = graph_of(next_step, T)
    g.replay()  # untimed warm-up
    clock_warmup(g.replay)
    step_ms, append_ms = [], []
    for _ in range(blocks):
        _, ms = timed_launches(g.replay, 1, stream)
        step_ms.append(ms / T)
        # the append is timed behind a replay still running on the GPU, so its events
        # bracket the kernel rather than the host's launch path
        torch.cuda.synchronize()
        g.replay()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        append()
        end.record(stream)
        torch.cuda.synchronize()
        append_ms.append(start.elapsed_time(end))
    # cold: each step with its inputs in HBM (cold_launch_ms: a 1 GiB read sweep, which
    # leaves the 256 MB Infinity Cache and the L2s holding other, clean lines, then the
    # step, minus the sweep alone)
    it_cold = [0]

    def cold_step():
        step(it_cold[0] % T)
        it_cold[0] += 1

    cold = cold_launch_ms(cold_step, 9, stream)
    cache_bytes = 2 * B * Hkv * C * d * 2
    blk_bytes = 2 * B * Hkv * S * d * 2
    q_bytes = B * Hq * S * d * 2
    o_bytes = B * Hq * S * d * 2 + B * Hq * S * 4
    alg = cache_bytes + blk_bytes + q_bytes + o_bytes
    warm = sorted(step_ms)[len(step_ms) // 2]
    app = sorted(append_ms)[len(append_ms) // 2]
    app_bytes = 2 * 2 * B * Hkv * S * d * 2
    return dict(
        workload="denoise step, B32 Hq16 Hkv8 d128 cache 2048 block 32, bf16; 32 steps then append",
        us_per_step_warm=warm * 1e3, us_per_step_cold=cold * 1e3,
        us_per_step_mean_warm=sum(step_ms) / len(step_ms) * 1e3,
        gbs_warm=alg / (warm * 1e-3) / 1e9, gbs_cold=alg / (cold * 1e-3) / 1e9,
        algorithmic_bytes_per_step=alg, steps_timed=len(step_ms) * T,
        append_us=app * 1e3, append_gbs=app_bytes / (app * 1e-3) / 1e9,
        roofline=dict(bound="hbm", achieved=round(alg / (cold * 1e-3) / 1e9, 1),
                      peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=round(alg / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      note="cold (Infinity Cache flushed); warm figure in gbs_warm"),
    )


def bench_decoder_layer(steps_per_block, reps, seed):
    """Attention sublayer of a decoder layer per denoising step (QKV projection, the
    denoise attention, output projection) at the denoise workload's shape with model
    width Hq d, over steps_per_block steps with fresh hidden states each."""
    import torch

    import masked_attention_amd as m
    from synth import TensorKind as K, device_draw, device_fill, tensor_id

    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, C, S, T = 32, 16, 8, 128, 2048, 32, steps_per_block
    Dm = Hq * d
    cap = C + S
    kc = torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    device_fill(kc, seed, tensor_id(K.K_CACHE), rows=C)
    device_fill(vc, seed, tensor_id(K.V_CACHE), rows=C)
    xs = []
    for t in range(T):
        x = torch.empty((B, S, Dm), dtype=torch.bfloat16, device=dev)
        device_draw(x, seed, tensor_id(K.X_BLK, step=t))
        xs.append(x)
    w_qkv = torch.empty(((Hq + 2 * Hkv) * d, Dm), dtype=torch.bfloat16, device=dev)
    w_o = torch.empty((Dm, Hq * d), dtype=torch.bfloat16, device=dev)
    device_draw(w_qkv, seed, tensor_id(K.W_QKV))
    device_draw(w_o, seed, tensor_id(K.W_O))
    w_qkv.mul_(2.0 ** -6)  # ~1/sqrt(Dm), a power of two (exact in bf16)
    w_o.mul_(2.0 ** -6)
    q = torch.empty((B, Hq, S, d), dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(q)
    k = torch.empty((B, Hkv, S, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    y = torch.empty((B, S, Dm), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, S), device=dev)
    nws = m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, Hq, Hkv, S, d, C)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    stream = torch.cuda.current_stream(dev)
    it = [0]

    def layer_step():
        m.e2d2_decoder_layer_denoise_step(xs[it[0] % T], w_qkv, w_o, kc, vc, C, q, k, v, o, y,
                                          lse_blk=lse, workspace=ws)
        it[0] += 1

    def attn_step():
        m.e2d2_attn_denoise_step(q, kc, vc, C, k, v, o, lse_blk=lse, workspace=ws)

    x2 = xs[0].view(B * S, Dm)
    o2 = torch.empty((B * S, Hq * d), dtype=torch.bfloat16, device=dev)

    qkv2 = torch.empty((B * S, (Hq + 2 * Hkv) * d), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((B * S, Dm), dtype=torch.bfloat16, device=dev)

    def lib_gemms():  # the same two products through torch (hipBLASLt), for context
        torch.matmul(x2, w_qkv.t(), out=qkv2)
        torch.matmul(o2, w_o.t(), out=y2)

    def lib_gemms_around_attention():
        # The library products in the layer's order with the attention between them, as
        # in the layer step.  Minus the attention alone, this is what they would cost
        # inside the step, measured the way projections_us measures the layer's own.
        torch.matmul(x2, w_qkv.t(), out=qkv2)
        attn_step()
        torch.matmul(o2, w_o.t(), out=y2)

    res = {}
    for name, fn in (("layer", layer_step), ("attention", attn_step), ("torch_gemms", lib_gemms),
                     ("torch_gemms_attention", lib_gemms_around_attention)):
        g = graph_of(fn, T)
        g.replay()
        clock_warmup(g.replay)
        ms = sorted(timed_launches(g.replay, 1, stream)[1] / T for _ in range(reps))
        res[name] = ms[len(ms) // 2]
    M = B * S
    flop = 2 * M * Dm * ((Hq + 2 * Hkv) * d + Hq * d)
    proj_ms = res["layer"] - res["attention"]
    return dict(
        workload="decoder-layer denoise step (QKV projection, attention over cache 2048 + "
                 "block 32, output projection), B32 Hq16 Hkv8 d128 Dm2048, bf16; "
                 f"{T} steps with fresh hidden states",
        us_per_step=round(res["layer"] * 1e3, 2),
        attention_us=round(res["attention"] * 1e3, 2),
        projections_us=round(proj_ms * 1e3, 2),
        projections_tflops=round(flop / (proj_ms * 1e-3) / 1e12, 1),
        projection_flop_per_step=flop,
        torch_hipblaslt_gemms_us=round(res["torch_gemms"] * 1e3, 2),
        torch_hipblaslt_gemms_in_layer_us=round((res["torch_gemms_attention"] - res["attention"]) * 1e3, 2),
    )


def bench_sampling_block(T, reps, seed):
    """One block of the sampling loop ("Encoder-Decoder Diffusion Language Models for
    Efficient Training and Inference", Paper-Notes page, 方法详解 §3 采样算法: T
    decoder steps against the encoder's KV cache, then the finished block through the
    encoder, which extends the cache) at the denoise workload's shape, for one encoder
    layer and one decoder layer in the shared-KV wiring (the decoder layer reads the
    encoder layer's cache):
      * T decoder-layer denoising steps (QKV projection, attention over the cache plus
        the noised block, output projection), fresh hidden states per step;
      * the encoder layer's update of the finished block: the same attention sublayer
        on the block's clean hidden states, whose k/v outputs are the block's rows of
        the cache;
      * the append of those rows.
    Each part and the whole block are replayed from HIP graphs and timed with HIP
    events; the append rewrites the same cache rows on every replay."""
    import torch

    import masked_attention_amd as m
    from synth import TensorKind as K, device_draw, device_fill, tensor_id

    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, C, S = 32, 16, 8, 128, 2048, 32
    Dm = Hq * d
    cap = C + S
    kc = torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    device_fill(kc, seed, tensor_id(K.K_CACHE), rows=C)
    device_fill(vc, seed, tensor_id(K.V_CACHE), rows=C)

    def draw(shape, kind, step=0, block=0, scale=None):
        t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        device_draw(t, seed, tensor_id(kind, step=step, block=block))
        if scale is not None:
            t.mul_(scale)  # ~1/sqrt(fan-in), a power of two (exact in bf16)
        return t

    xs = [draw((B, S, Dm), K.X_BLK, step=t) for t in range(T)]
    x_clean = draw((B, S, Dm), K.X_BLK, block=1)
    w = {}
    for layer, blk in (("dec", 0), ("enc", 1)):
        w[layer] = (draw(((Hq + 2 * Hkv) * d, Dm), K.W_QKV, block=blk, scale=2.0 ** -6),
                    draw((Dm, Hq * d), K.W_O, block=blk, scale=2.0 ** -6))

    def act():
        q = torch.empty((B, Hq, S, d), dtype=torch.bfloat16, device=dev)
        k = torch.empty((B, Hkv, S, d), dtype=torch.bfloat16, device=dev)
        return (q, k, torch.empty_like(k), torch.empty_like(q),
                torch.empty((B, S, Dm), dtype=torch.bfloat16, device=dev),
                torch.empty((B, Hq, S), device=dev))

    a_dec, a_enc = act(), act()
    nws = m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, Hq, Hkv, S, d, C)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    it = [0]

    def dec_steps():
        for t in range(T):
            q, k, v, o, y, lse = a_dec
            m.e2d2_decoder_layer_denoise_step(xs[t], *w["dec"], kc, vc, C, q, k, v, o, y,
                                              lse_blk=lse, workspace=ws)

    def enc_update():
        q, k, v, o, y, lse = a_enc
        m.e2d2_decoder_layer_denoise_step(x_clean, *w["enc"], kc, vc, C, q, k, v, o, y,
                                          lse_blk=lse, workspace=ws)
        m.e2d2_kv_cache_append(kc, vc, C, k, v)

    def block():
        dec_steps()
        enc_update()

    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, fn in (("block", block), ("decoder_steps", dec_steps), ("encoder_update", enc_update)):
        g = graph_of(fn, 1)
        g.replay()
        clock_warmup(g.replay)
        ms = sorted(timed_launches(g.replay, 1, stream)[1] for _ in range(reps))
        res[name] = ms[len(ms) // 2]
    return dict(
        workload=f"one sampling-loop block, B32 Hq16 Hkv8 d128 Dm2048, cache 2048, block 32, "
                 f"bf16: {T} decoder-layer steps + the encoder layer's update of the "
                 "finished block + the KV-cache append (one encoder and one decoder layer)",
        us_per_block=round(res["block"] * 1e3, 2),
        decoder_steps_us=round(res["decoder_steps"] * 1e3, 2),
        decoder_us_per_step=round(res["decoder_steps"] * 1e3 / T, 2),
        encoder_update_us=round(res["encoder_update"] * 1e3, 2),
        encoder_share=round(res["encoder_update"] / res["block"], 4),
        tokens_per_s_per_layer_pair=round(B * S / (res["block"] * 1e-3), 1),
    )


def bench_near_ar(blocks, steps, seed):
    """Near-autoregressive decoding: B64 H32 (MHA) d128, block 4, a cache that starts at
    32768 rows; `blocks` blocks of `steps` denoising steps each, every block followed by
    the KV-cache append of its 4 rows (cache_len grows by 4 per block), with fresh
    block tensors for every step.  Each step streams the whole cache (34 GB), so the
    loop runs eagerly; HIP events bracket every step and append and the whole loop."""
    import torch

    import masked_attention_amd as m
    from synth import TensorKind as K, device_fill, tensor_id

    dev = torch.device("cuda:0")
    B, H, d, C0, S = 64, 32, 128, 32768, 4
    cap = C0 + blocks * S
    kc = torch.empty((B, H, cap, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    device_fill(kc, seed, tensor_id(K.K_CACHE), rows=C0)
    device_fill(vc, seed, tensor_id(K.V_CACHE), rows=C0)

    def fill(kind, t, k):
        x = torch.empty((B, H, S, d), dtype=torch.bfloat16, device=dev)
        device_fill(x, seed, tensor_id(kind, step=t, block=k))
        return x

    blk = [[(fill(K.Q_BLK, t, k), fill(K.K_BLK, t, k), fill(K.V_BLK, t, k)) for t in range(steps)]
           for k in range(blocks)]
    new = [(fill(K.K_NEW, 0, k), fill(K.V_NEW, 0, k)) for k in range(blocks)]
    o = torch.empty((B, H, S, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, S), device=dev)
    assert m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, H, H, S, d, C0) == 0
    stream = torch.cuda.current_stream(dev)

    def step(k, t):
        q, kb, vb = blk[k][t]
        m.e2d2_attn_denoise_step(q, kc, vc, C0 + k * S, kb, vb, o, lse_blk=lse)

    for t in range(steps):  # warm-up at the first length (each step is ms of streaming)
        step(0, t)
    torch.cuda.synchronize()
    ev = []
    e0 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(blocks):
        for t in range(steps):
            step(k, t)
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            ev.append(("step", e))
        m.e2d2_kv_cache_append(kc, vc, C0 + k * S, *new[k])
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev.append(("append", e))
    torch.cuda.synchronize()
    step_ms, app_ms = [], []
    prev = e0
    for kind, e in ev:
        (step_ms if kind == "step" else app_ms).append(prev.elapsed_time(e))
        prev = e
    total = e0.elapsed_time(ev[-1][1])
    alg = 0  # algorithmic bytes of every step: the cache rows read, own K/V, Q, O, LSE
    for k in range(blocks):
        C = C0 + k * S
        alg += steps * (2 * B * H * C * d * 2 + 2 * B * H * S * d * 2 + 2 * B * H * S * d * 2
                        + B * H * S * 4)
    app_bytes = blocks * 2 * 2 * B * H * S * d * 2
    med = sorted(step_ms)[len(step_ms) // 2]
    gbs = alg / (sum(step_ms) * 1e-3) / 1e9
    return dict(workload=f"near-AR decoding, B64 H32 (MHA) d128, cache 32768 + 4 per block, block 4, "
                         f"{blocks} blocks x {steps} steps with an append after each block, bf16",
                total_ms=round(total, 2), steps_timed=len(step_ms),
                ms_per_step_mean=round(sum(step_ms) / len(step_ms), 4), ms_per_step_median=round(med, 4),
                append_us_mean=round(sum(app_ms) / len(app_ms) * 1e3, 2),
                algorithmic_bytes=alg, gbs=round(gbs, 1), frac_of_hbm_peak=round(gbs / PEAK_HBM_GBS, 4),
                total_with_appends_gbs=round((alg + app_bytes) / (total * 1e-3) / 1e9, 1))


def cpu_baseline(budget_s: float = 12.0):
    """fp64 oracle on a bounded sample of the training workload (whole heads, encoder
    and decoder), in useful TFLOP/s like the GPU figure."""
    import numpy as np  # noqa: F401
    from threadpoolctl import threadpool_info

    import oracle
    from synth import TensorKind as K, host_tensor, tensor_id

    B, H, L, S, d, seed = 8, 16, 1024, 16, 64, 0xE2D20002
    heads = [(b, h) for b in range(B) for h in range(H)]
    t_total = 0.0
    done = 0
    for b, h in heads:
        def g(kind):
            return host_tensor(seed, tensor_id(kind), (1, 1, L, d), "bf16", b0=b, h0=h)

        qd, qe, kc, vc, kd, vd = (g(k) for k in (K.Q_DEC, K.Q_ENC, K.K_CTX, K.V_CTX, K.K_DEC,
                                                  K.V_DEC))
        t0 = time.perf_counter()
        oracle.train_fwd(qd, kc, vc, kd, vd, S, 1.0 / math.sqrt(d), q_enc=qe)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    useful = 4.0 * d * 2 * pairs_blockcausal(L, S) * done
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return dict(value=useful / t_total / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{done} of {B * H} (batch, head) pairs of the B8 H16 d64 L1024 S16 "
                       f"training forward, encoder + decoder, fp64 explicit-mask oracle, "
                       f"{t_total:.1f} s; cores = BLAS threads (exp and masking run on one)",
                seconds=round(t_total, 2), host_cpus=os.cpu_count())


def _time_repeat(fn, min_s):
    """Run fn until at least min_s seconds have passed; returns (calls, seconds)."""
    n, t = 0, 0.0
    while t < min_s:
        t0 = time.perf_counter()
        fn()
        t += time.perf_counter() - t0
        n += 1
    return n, t


def cpu_baseline_other(min_s: float = 3.0):
    """The fp64 oracle on the other workloads, each timed on a slice (the oracle's cost
    depends only on the shapes, so a slice's time scales to the whole workload; every
    figure that is scaled says so):
      * denoise step B32 Hq16 Hkv8 d128 C2048 S32: the 16 query heads of one sequence,
        scaled to 32 sequences;
      * long training forward B2 Hq16 Hkv8 d128 L8192 S64: one query head, encoder and
        decoder, scaled to 32 heads;
      * near-AR step B64 H32 d128 C32768 S4: one head, scaled to 2048 heads per step and
        to the 64 steps of 16 blocks x 4 (cache 32768 + 4 per block)."""
    import oracle
    from synth import TensorKind as K, host_tensor, tensor_id

    out = []
    # denoise step
    seed, B, Hq, Hkv, d, C, S = 0xE2D20003, 32, 16, 8, 128, 2048, 32
    g = lambda kind, shape, **kw: host_tensor(seed, tensor_id(kind), shape, "bf16", **kw)
    q = g(K.Q_BLK, (1, Hq, S, d))
    kc, vc = g(K.K_CACHE, (1, Hkv, C, d)), g(K.V_CACHE, (1, Hkv, C, d))
    kb, vb = g(K.K_BLK, (1, Hkv, S, d)), g(K.V_BLK, (1, Hkv, S, d))
    n, t = _time_repeat(lambda: oracle.denoise_step(q, kc, vc, C, kb, vb, 1 / math.sqrt(d)), min_s)
    per_step = t / n * B
    out.append(dict(workload="denoise step, B32 Hq16 Hkv8 d128 cache 2048 block 32", kind="oracle",
                    value=round(per_step * 1e6, 1), unit="us per step (extrapolated)",
                    sample=f"16 query heads of 1 of 32 sequences, {n} calls in {t:.2f} s, x 32"))
    # long training forward
    seed, L, S, d = 0xE2D20004, 8192, 64, 128
    g = lambda kind: host_tensor(seed, tensor_id(kind), (1, 1, L, d), "bf16")
    qd, qe, kc, vc, kd, vd = (g(k) for k in (K.Q_DEC, K.Q_ENC, K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC))
    t0 = time.perf_counter()
    oracle.train_fwd(qd, kc, vc, kd, vd, S, 1 / math.sqrt(d), q_enc=qe)
    t = time.perf_counter() - t0
    useful = 4.0 * d * 2 * pairs_blockcausal(L, S)
    out.append(dict(workload="long training forward, B2 Hq16 Hkv8 d128 L8192 S64, encoder + decoder",
                    kind="oracle", value=round(useful / t / 1e12, 5), unit="TFLOP/s",
                    seconds_per_head=round(t, 2), seconds_whole=round(t * 32, 1),
                    sample="1 of 32 query heads (both masks); seconds_whole = x 32 (extrapolated)"))
    # near-AR step
    seed, d, C0, S = 0xE2D20005, 128, 32768, 4
    g = lambda kind, n: host_tensor(seed, tensor_id(kind), (1, 1, n, d), "bf16")
    q, kb, vb = g(K.Q_BLK, S), g(K.K_BLK, S), g(K.V_BLK, S)
    kc, vc = g(K.K_CACHE, C0), g(K.V_CACHE, C0)
    n, t = _time_repeat(lambda: oracle.denoise_step(q, kc, vc, C0, kb, vb, 1 / math.sqrt(d)), min_s)
    per_step = t / n * 64 * 32
    out.append(dict(workload="near-AR step, B64 H32 d128 cache 32768 block 4", kind="oracle",
                    value=round(per_step * 1e3, 1), unit="ms per step (extrapolated)",
                    seconds_64_steps=round(per_step * 64, 1),
                    sample=f"1 of 2048 heads at cache 32768, {n} calls in {t:.2f} s, x 2048 heads; "
                           "x 64 steps for the 16 blocks x 4 (extrapolated)"))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--only", choices=["all", "train", "bwd", "layers", "denoise", "long", "nearar",
                                       "declayer", "sampling", "copycal"],
                    default="all",
                    help="restrict the run (profiling); 'copycal' runs only a plain 1 GiB "
                         "device copy, the reference for scaling HBM byte counters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the benchmark measures one GPU only (no multi-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import masked_attention_amd as m

    m.lib()  # fail loudly when the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    out = {}
    train = None
    if args.only == "copycal":
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copycal_bytes_read": n, "copycal_bytes_written": n, "launches": 3}))
        return
    if args.only in ("all", "train"):
        B, H, L, S, d = 8, 16, 1024, 16, 64
        train = bench_train(B, H, H, L, S, d, args.steps, args.warmup, 0xE2D20002, cold=True)
        print(f"[bench] train fwd B{B} H{H} d{d} L{L} S{S}: {train['ms_per_step'] * 1e3:.1f} us/step, "
              f"kernel {train['kernel_ms'] * 1e3:.1f} us", file=sys.stderr, flush=True)
    if args.only in ("all", "bwd"):
        out["train_bwd"] = bench_train_bwd(8, 16, 16, 1024, 16, 64, args.steps, 0xE2D20002)
        out["long_train_bwd"] = bench_train_bwd(2, 16, 8, 8192, 64, 128, max(3, args.steps // 10),
                                                0xE2D20004)
        for k in ("train_bwd", "long_train_bwd"):
            print(f"[bench] {k}: {out[k]['ms_per_step'] * 1e3:.1f} us, {out[k]['tflops']} TFLOP/s",
                  file=sys.stderr, flush=True)
    if args.only in ("all", "layers"):
        out["layer_split"] = bench_layer_split(8, 16, 1024, 16, 64, args.steps, 0xE2D20002)
        print(f"[bench] layer split: {out['layer_split']}", file=sys.stderr, flush=True)
    if args.only in ("all", "long"):
        lt = bench_train(2, 16, 8, 8192, 64, 128, max(3, args.steps // 10), 2, 0xE2D20004)
        out["long_train"] = dict(
            workload="training fwd enc+dec, B2 Hq16 Hkv8 d128 L8192 S64, bf16, with LSE",
            ms_per_step=round(lt["ms_per_step"], 4),
            tflops=round(lt["useful_flop"] / (lt["kernel_ms"] * 1e-3) / 1e12, 1),
            frac_of_peak=round(lt["useful_flop"] / (lt["kernel_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))
        print(f"[bench] long train: {lt['kernel_ms']:.3f} ms, {out['long_train']['tflops']} TFLOP/s",
              file=sys.stderr, flush=True)
    if args.only in ("all", "denoise"):
        out["denoise"] = bench_denoise(32, 4, 1, 0xE2D20003)
        print(f"[bench] denoise: warm {out['denoise']['us_per_step_warm']:.1f} us "
              f"({out['denoise']['gbs_warm']:.0f} GB/s), cold {out['denoise']['us_per_step_cold']:.1f} us "
              f"({out['denoise']['gbs_cold']:.0f} GB/s)", file=sys.stderr, flush=True)
        out["denoise_varlen"] = bench_denoise_varlen(32, 0xE2D20009)
        print(f"[bench] denoise varlen: {out['denoise_varlen']['us_per_step_warm']:.1f} us "
              f"({out['denoise_varlen']['gbs_warm']:.0f} GB/s)", file=sys.stderr, flush=True)

    if args.only in ("all", "sampling"):
        out["sampling_block"] = bench_sampling_block(32, 5, 0xE2D20003)
        print(f"[bench] sampling block: {out['sampling_block']}", file=sys.stderr, flush=True)

    if args.only in ("all", "declayer"):
        out["decoder_layer"] = bench_decoder_layer(32, 5, 0xE2D20003)
        print(f"[bench] decoder layer step: {out['decoder_layer']}", file=sys.stderr, flush=True)

    if args.only in ("all", "nearar"):
        out["near_ar"] = bench_near_ar(16, 4, 0xE2D20005)
        print(f"[bench] near-AR: {out['near_ar']['total_ms']:.1f} ms for 64 steps, "
              f"{out['near_ar']['ms_per_step_mean']:.3f} ms/step ({out['near_ar']['gbs']:.0f} GB/s)",
              file=sys.stderr, flush=True)

    if train is None:
        print(json.dumps(out))
        return
    value = train["useful_flop"] / (train["ms_per_step"] * 1e-3) / 1e12
    tB, tH, tL, td = 8, 16, 1024, 64
    alg_bytes = 6 * tB * tH * tL * td * 2 + 2 * tB * tH * tL * td * 2 + 2 * tB * tH * tL * 4
    achieved = train["useful_flop"] / (train["kernel_ms"] * 1e-3) / 1e12
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")
    except (OSError, ValueError):
        pass
    line = {
        "metric": "useful TFLOP/s (masked attn fwd, % MFMA peak); denoise-step us + HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(train["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "E2D2 training attention fwd, encoder block-causal + decoder "
                               "2L-key mask in one launch, B8 H16 d64 L1024 S16 bf16, "
                               "N(0,1) inputs", "global_batch": 8, "seq_len": 1024,
                   "block": 16, "heads": 16, "d_head": 64, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "train_fwd_bf16_kernel<64>",
                     "kernel_us": round(train["kernel_ms"] * 1e3, 2),
                     "useful_flop_per_launch": train["useful_flop"],
                     # six bf16 inputs in, two outputs and two LSE arrays out, each once
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "flop_per_byte": round(train["useful_flop"] / alg_bytes, 1),
                     "hbm_roof_tflops": round(train["useful_flop"] / alg_bytes * PEAK_HBM_GBS / 1e3, 1)},
        "train_cold": {"us": round(train["cold_ms"] * 1e3, 2),
                       "tflops": round(train["useful_flop"] / (train["cold_ms"] * 1e-3) / 1e12, 1),
                       "hbm_gbs": round(alg_bytes / (train["cold_ms"] * 1e-3) / 1e9, 1),
                       "note": "one launch right after a 1 GiB read sweep (inputs from HBM); "
                               "value and roofline are the warm figures (inputs in the "
                               "Infinity Cache after the previous launch)"},
    }
    line.update(out)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
        line["cpu_baseline_other"] = cpu_baseline_other()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
