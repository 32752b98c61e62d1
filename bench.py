#!/usr/bin/env python3
"""Benchmark of the dense-decoder hot path on one MI355X.

One step = one pass of the workload: prefill of a random-id prompt (MFMA GEMM
path), then greedy decode steps at batch 1 that feed the previous step's
on-device argmax back as the next token.  Weights are seeded synthetic
N(0, 0.02) bf16 (or MLX-style 4-bit), resident in HBM before timing starts.

Prints one JSON line: value = decode tok/s (whole job, one GPU), plus prefill
tok/s, a roofline object for the dominant kernel (decode weight streaming,
HBM bound) and one for the prefill GEMMs (MFMA bound), and the CPU oracle's
rate on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix throughput

# Measured HBM traffic per launch of the dominant decode kernel: two rocprofv3
# --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
# each scaled by what the same counter reads for a plain 1 GiB device copy
# (--copy-probe): FETCH_SIZE x 2.0, WRITE_SIZE x 1.0.  A figure is only
# reported while the kernel's sources are the ones it was taken on.
TRAFFIC = {
    ("q8b", "decode.step"): {"fetch_kib": 7563807.7, "write_kib": 50617.4, "fetch_factor": 2.0, "write_factor": 1.0,
                             "sources": ["decoder_prefill_kv_amd/csrc/decode_step.hip",
                                         "decoder_prefill_kv_amd/csrc/gemv_body.h",
                                         "decoder_prefill_kv_amd/csrc/common.h",
                                         "decoder_prefill_kv_amd/csrc/kernels.h"],
                             "sha256": "f2cb8946b099d6d586e5a6d70c67de03aa622fac7dd0567e7a091f16a2995818"},
    # the same step over the int8 cache and with integer-code weights
    ("q8b+kv_i8", "decode.step"): {"fetch_kib": 7500108.5, "write_kib": 50599.4, "fetch_factor": 2.0, "write_factor": 1.0,
                             "sources": ["decoder_prefill_kv_amd/csrc/decode_step.hip", "decoder_prefill_kv_amd/csrc/gemv_body.h",
                              "decoder_prefill_kv_amd/csrc/common.h", "decoder_prefill_kv_amd/csrc/kernels.h"],
                             "sha256": "f2cb8946b099d6d586e5a6d70c67de03aa622fac7dd0567e7a091f16a2995818"},
    ("q8b_i8", "decode.step"): {"fetch_kib": 3874082.5, "write_kib": 14347.1, "fetch_factor": 2.0, "write_factor": 1.0,
                             "sources": ["decoder_prefill_kv_amd/csrc/decode_step.hip", "decoder_prefill_kv_amd/csrc/gemv_body.h",
                              "decoder_prefill_kv_amd/csrc/common.h", "decoder_prefill_kv_amd/csrc/kernels.h"],
                             "sha256": "f2cb8946b099d6d586e5a6d70c67de03aa622fac7dd0567e7a091f16a2995818"},
    ("q8b_q8", "decode.step"): {"fetch_kib": 4486450.6, "write_kib": 14347.1, "fetch_factor": 2.0, "write_factor": 1.0,
                             "sources": ["decoder_prefill_kv_amd/csrc/decode_step.hip", "decoder_prefill_kv_amd/csrc/gemv_body.h",
                              "decoder_prefill_kv_amd/csrc/common.h", "decoder_prefill_kv_amd/csrc/kernels.h"],
                             "sha256": "f2cb8946b099d6d586e5a6d70c67de03aa622fac7dd0567e7a091f16a2995818"},
    ("q8b_q40", "decode.step"): {"fetch_kib": 2258180.2, "write_kib": 14347.1, "fetch_factor": 2.0, "write_factor": 1.0,
                             "sources": ["decoder_prefill_kv_amd/csrc/decode_step.hip", "decoder_prefill_kv_amd/csrc/gemv_body.h",
                              "decoder_prefill_kv_amd/csrc/common.h", "decoder_prefill_kv_amd/csrc/kernels.h"],
                             "sha256": "f2cb8946b099d6d586e5a6d70c67de03aa622fac7dd0567e7a091f16a2995818"},
    # the 0.6B-shaped steps (128 columns per wave and iteration; bf16, MLX 4-bit)
    ("q06b", "decode.step"): {"fetch_kib": 618300.4, "write_kib": 4896.1, "fetch_factor": 2.0, "write_factor": 1.0,
                             "sources": ["decoder_prefill_kv_amd/csrc/decode_step.hip", "decoder_prefill_kv_amd/csrc/gemv_body.h",
                              "decoder_prefill_kv_amd/csrc/common.h", "decoder_prefill_kv_amd/csrc/kernels.h"],
                             "sha256": "f2cb8946b099d6d586e5a6d70c67de03aa622fac7dd0567e7a091f16a2995818"},
    ("q06b_q4", "decode.step"): {"fetch_kib": 287342.3, "write_kib": 6492.1, "fetch_factor": 2.0, "write_factor": 1.0,
                             "sources": ["decoder_prefill_kv_amd/csrc/decode_step.hip", "decoder_prefill_kv_amd/csrc/gemv_body.h",
                              "decoder_prefill_kv_amd/csrc/common.h", "decoder_prefill_kv_amd/csrc/kernels.h"],
                             "sha256": "f2cb8946b099d6d586e5a6d70c67de03aa622fac7dd0567e7a091f16a2995818"},
    # the prefill gate+up GEMM (M = 2048): operands re-read from HBM ~3.5x
    ("q8b", "gemm.gate_up"): {"fetch_kib": 380246.7, "write_kib": 57600.4, "fetch_factor": 2.0, "write_factor": 1.0,
                              "sources": ["decoder_prefill_kv_amd/csrc/gemm.hip",
                                          "decoder_prefill_kv_amd/csrc/common.h",
                                          "decoder_prefill_kv_amd/csrc/kernels.h"],
                              "sha256": "b45210dd7044baea62beaf1d0aa34b5186e72ef00b5c1ecda1fda5cdfcf2ba71"},
}


def measured_traffic(workload, kclass):
    import hashlib
    t = TRAFFIC.get((workload, kclass))
    if not t:
        return None
    h = hashlib.sha256()
    for src in t["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != t["sha256"]:
        return None
    return 1024.0 * (t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"])


WORKLOADS = {
    # name: (config, prompt, decode steps, description)
    "q8b": ("q8b", 2048, 256, "Qwen3-8B-shaped bf16 decoder (36 layers, hidden 4096, 32/8 heads, d 128, MLP 12288, "
                              "vocab 151936, untied head): prefill 2048 random ids, then 256 greedy decode steps, "
                              "batch 1"),
    "q06b": ("q06b", 512, 128, "Qwen3-0.6B-shaped bf16 decoder (28 layers, hidden 1024, 16/8 heads, d 128, "
                               "MLP 3072, vocab 151936, tied head): prefill 512, then 128 greedy decode steps"),
    "q06b_q4": ("q06b_q4", 2048, 128, "Qwen3-0.6B-shaped decoder, MLX 4-bit affine g64 linears incl. tied head: "
                                      "prefill 2048, then 128 greedy decode steps"),
    "q8b_i8": ("q8b_i8", 2048, 64, "Qwen3-8B-shaped decoder, int8 linears with one bf16 scale per output row "
                                   "(incl. head): prefill 2048, then 64 greedy decode steps"),
    "q8b_q8": ("q8b_q8", 2048, 64, "Qwen3-8B-shaped decoder, int8 linears in blocks of 32 with an fp32 scale each "
                                   "(incl. head): prefill 2048, then 64 greedy decode steps"),
    "q8b_q40": ("q8b_q40", 2048, 64, "Qwen3-8B-shaped decoder, GGUF-style Q4_0 linears (blocks of 32 four-bit codes, "
                                     "fp16 scale; incl. head): prefill 2048, then 64 greedy decode steps"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_info():
    """CPUs this process may run on and the host's CPU model."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 0
    return {"nproc": ncpu, "cpu_model": model}


def cpu_baseline(cfg, w, prompt, n_prefix=32):
    """The oracle as it stands (float64, weights widened from bf16 per use) on a
    bounded sample of the workload: the block path over the first n_prefix
    prompt ids (prompt tok/s), then one step-path decode step at position
    n_prefix (decode tok/s)."""
    import torch
    import oracle
    m = oracle.OracleModel(cfg, w, torch.float64, cache_weights=False)
    cache = m.new_cache(n_prefix + 1)
    t0 = time.perf_counter()
    lg = m.forward_block(cache, prompt[:n_prefix], 0)[0]
    t_pre = time.perf_counter() - t0
    t0 = time.perf_counter()
    m.forward_step(cache, oracle.argmax_lowest(lg), n_prefix)
    t_dec = time.perf_counter() - t0
    out = {"value": round(1.0 / t_dec, 5), "unit": "tok/s", "cores": torch.get_num_threads(), "kind": "oracle",
           "prefill_tok_s": round(n_prefix / t_pre, 4),
           "sample": "float64 oracle, weights widened from bf16 per use: block-path prefill of the workload "
                     "prompt's first %d ids (%.1f s), then one step-path decode step at position %d (%.1f s); "
                     "value is that decode rate, prefill_tok_s the prompt rate" % (n_prefix, t_pre, n_prefix, t_dec)}
    out.update(host_info())
    return out


def copy_probe(nbytes):
    """A plain copy kernel of known size: reads and writes nbytes once each.
    Counter runs over it give the factor between what FETCH_SIZE / WRITE_SIZE
    report and the bytes actually moved."""
    import torch
    n = (nbytes + 15) // 16 * 16
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)


def membench(nbytes=2 << 30, reps=5):
    """Achievable HBM rate on this GPU for context: a plain device-to-device
    copy of nbytes (read + write counted), best of reps."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = 1e30
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    del src, dst
    torch.cuda.empty_cache()
    return {"kind": "device copy (read + write)", "bytes": 2 * nbytes, "GBps": round(2 * nbytes / best / 1e9, 1),
            "frac_of_peak": round(2 * nbytes / best / 1e9 / HBM_PEAK_GBS, 4)}


def class_times(stats, passes):
    """{kernel class: [launches per pass, total us per pass, GB/s]} from a
    profile_end() result covering `passes` passes."""
    out = {}
    for k, v in sorted(stats.items(), key=lambda kv: -kv[1]["total_ms"]):
        gbs = v["bytes"] / (v["total_ms"] / 1e3) / 1e9 if v["total_ms"] else 0.0
        out[k] = [v["launches"] // passes, round(1e3 * v["total_ms"] / passes, 1), round(gbs, 1)]
    return out


class DeviceError(RuntimeError):
    pass


def check_device(dpk, dec, what):
    """Raise if the library saw a device-side error (a persistent step's
    bounded barrier wait that gave up, or an out-of-range device token id)
    since the last check: the timed work would not be valid."""
    try:
        dpk.check_device_errors(dec.handle)
    except dpk.DpkError as e:
        raise DeviceError("%s: %s" % (what, e))


def bench_verify(dpk, cfg, w, seed, flags, K=5, rounds=24, warm=4):
    """Speculative verify of K drafts (M = K + 1 rows) against the KV cache of
    an 8192-token prompt: passes/s, and the ratio to one decode step at the
    same context.  Each verify call returns the accept count to the host (one
    synchronisation per pass, as the speculative loop needs it)."""
    import torch
    import synth
    P = 8192
    # room for the timed passes, the profiled pass and the decode steps after them
    dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=P + (K + 1) * (rounds + warm + 1) + 32, max_rows=P, flags=flags)
    lg = dec.logits_buffer(K + 1)
    am = dec.argmax_buffer(K + 1)
    dec.prefill(0, [int(t) for t in synth.prompt_ids(cfg, P, seed)], lg[0:1], am[0:1])
    drafts = [int(t) for t in synth.prompt_ids(cfg, (K + 1) * (rounds + warm), seed, index=99)]
    torch.cuda.synchronize()
    pos = P
    times = []
    for r in range(rounds + warm):
        t0 = time.perf_counter()
        acc = dec.verify(0, drafts[r * (K + 1):(r + 1) * (K + 1)], pos, am, lg)
        dt = time.perf_counter() - t0
        if r >= warm:
            times.append(dt)
        pos += acc + 1
    vt = sum(times) / len(times)
    check_device(dpk, dec, "verify passes")
    # one more pass with per-launch timing: where a verify pass spends its time
    dpk.profile_begin(dec.handle, 100000)
    acc = dec.verify(0, drafts[0:K + 1], pos, am, lg)
    pos += acc + 1
    classes = class_times(dpk.profile_end(dec.handle), 1)
    # one decode step at the same context, for the verify / decode ratio
    a1 = dec.argmax_buffer(1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(3):
        dec.decode_step([0], [drafts[i]], [pos + i], a1)
    torch.cuda.synchronize()
    e0.record()
    for i in range(8):
        dec.decode_step([0], [drafts[i]], [pos + 3 + i], a1)
    e1.record()
    torch.cuda.synchronize()
    dt_dec = e0.elapsed_time(e1) / 8 / 1e3
    check_device(dpk, dec, "verify profiled pass and decode steps")
    dec.close()
    H, L, d = cfg.hidden, cfg.n_layers, cfg.head_dim
    wbytes = (cfg.n_linear_params() + cfg.vocab * H) * 2.0
    kv = (P + K + 1) * 2 * L * cfg.n_kv_heads * d * (1 + 4.0 / d if cfg.kv_i8 else 2.0)
    return {"workload": "verify K=%d (M=%d rows) over the KV cache of an %d-token prompt" % (K, K + 1, P),
            "passes_per_s": round(1.0 / vt, 2), "ms_per_pass": round(vt * 1e3, 3),
            "hbm_frac": round((wbytes + kv) / vt / 1e9 / HBM_PEAK_GBS, 4),
            "decode_ms_same_ctx": round(dt_dec * 1e3, 3), "verify_over_decode": round(vt / dt_dec, 3),
            "note": "per-pass wall time includes the host read of the accept count",
            "kernel_classes_us_per_pass": classes}


def bench_batch16(dpk, cfg, w, seed, flags, B=16, P=4096, N=32):
    """Decode of 16 independent sequences, each with its own 4096-token KV
    cache, one token per sequence per step: aggregate tok/s."""
    import torch
    import synth
    dec = dpk.Decoder(cfg, w, max_batch=B, max_seq=P + N + 8, max_rows=P, flags=flags)
    lg = dec.logits_buffer(B)
    am = dec.argmax_buffer(B)
    for b in range(B):
        dec.prefill(b, [int(t) for t in synth.prompt_ids(cfg, P, seed, index=b)], lg[b:b + 1], am[b:b + 1])
    seqs = list(range(B))
    dec.decode_step(seqs, None, [P] * B, am, lg, ids_dev=am)  # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(N):
        dec.decode_step(seqs, None, [P + 1 + s] * B, am, lg, ids_dev=am)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) / N / 1e3
    check_device(dpk, dec, "batch-16 steps")
    # one more step with per-launch timing: where a batch step spends its time
    dpk.profile_begin(dec.handle, 100000)
    dec.decode_step(seqs, None, [P + 1 + N] * B, am, lg, ids_dev=am)
    classes = class_times(dpk.profile_end(dec.handle), 1)
    check_device(dpk, dec, "batch-16 profiled step")
    dec.close()
    H, L, d = cfg.hidden, cfg.n_layers, cfg.head_dim
    wbytes = (cfg.n_linear_params() + cfg.vocab * H) * 2.0
    kv = B * (P + 1 + N / 2.0) * 2 * L * cfg.n_kv_heads * d * (1 + 4.0 / d if cfg.kv_i8 else 2.0)
    return {"workload": "batched decode: %d sequences x %d-token KV caches, %d steps" % (B, P, N),
            "tok_s": round(B / dt, 1), "ms_per_step": round(dt * 1e3, 3),
            "hbm_frac": round((wbytes + kv) / dt / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_classes_us_per_step": classes}


def run_workload(dpk, name, steps, warmup, seed, flags, decode_steps=None, profile=True, w=None, kv_i8=False):
    """Prefill + greedy batch-1 decode of one workload: steps timed passes after
    warmup untimed ones.  Returns (result dict, host weights)."""
    import torch
    import synth
    cname, P, N, desc = WORKLOADS[name]
    if decode_steps is not None:
        N = decode_steps
    cfg = synth.CONFIGS[cname]
    if kv_i8:
        cfg = cfg.with_(kv_i8=True)
    t0 = time.time()
    if w is None:
        w = synth.make_weights(cfg, seed)
    log("[bench] %s: weights generated in %.1f s" % (name, time.time() - t0))
    prompt = [int(t) for t in synth.prompt_ids(cfg, P, seed)]
    stream = torch.cuda.current_stream()
    t0 = time.time()
    dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=P + N, max_rows=P, flags=flags)
    torch.cuda.synchronize()
    log("[bench] %s: weights on device in %.1f s (kv %.2f GB, scratch %.2f GB, prep %.2f GB)"
        % ((name, time.time() - t0) + tuple(x / 1e9 for x in dec.sizes)))
    lg = dec.logits_buffer(1)
    am = dec.argmax_buffer(1)

    def one_step(ev=None):
        if ev:
            ev[0].record(stream)
        dec.prefill(0, prompt, lg, am)
        if ev:
            ev[1].record(stream)
        for s in range(N):
            dec.decode_step([0], None, [P + s], am, lg, ids_dev=am)
        if ev:
            ev[2].record(stream)

    for i in range(warmup):
        one_step()
        torch.cuda.synchronize()
        log("[bench] %s: warmup %d done" % (name, i))
    check_device(dpk, dec, name + " warmup")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        one_step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    check_device(dpk, dec, name + " timed steps")
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    log("[bench] %s: timed %d steps: %.1f ms/step (prefill %.2f ms, decode %.1f ms)"
        % (name, steps, wall * 1e3 / steps, pre_ms, dec_ms))
    decode_tps = N / (dec_ms / 1e3)
    prefill_tps = P / (pre_ms / 1e3)

    # algorithmic work of the workload
    H, L, d = cfg.hidden, cfg.n_layers, cfg.head_dim
    n_lin = cfg.n_linear_params()
    head_params = cfg.vocab * H
    wbytes = {"bf16": 2.0, "f32": 4.0, "q4": 0.5 + 4.0 / 64, "i8": 1.0 + 2.0 / H, "q8": 1.0 + 4.0 / 32,
              "q4_0": 0.5 + 2.0 / 32}[cfg.weight_format]
    kv_elt = 4 if cfg.weight_format == "f32" else (1 + 4.0 / cfg.head_dim if cfg.kv_i8 else 2)
    kv_per_pos = 2 * L * cfg.n_kv_heads * d * kv_elt
    mean_ctx = P + (N + 1) / 2.0
    decode_bytes_tok = (n_lin + head_params) * wbytes + kv_per_pos * mean_ctx
    prefill_flops = 2.0 * n_lin * P + 4.0 * L * cfg.n_heads * d * P * (P + 1) / 2 + 2.0 * head_params

    roof = roof_prefill = kernels = None
    if profile:
        dpk.profile_begin(dec.handle, 200000)
        one_step()
        stats = dpk.profile_end(dec.handle)
        check_device(dpk, dec, name + " profiled step")
        kernels = {k: {"launches": v["launches"], "avg_us": round(1e3 * v["total_ms"] / v["launches"], 2),
                       "total_ms": round(v["total_ms"], 3)} for k, v in stats.items()}
        dec_cls = {k: v for k, v in stats.items()
                   if k.startswith("gemv") or k.startswith("attn.decode") or k == "decode.step"}
        dom = max(dec_cls, key=lambda k: dec_cls[k]["total_ms"])
        v = stats[dom]
        avg_s = v["total_ms"] / 1e3 / v["launches"]
        ach = v["bytes"] / v["launches"] / avg_s / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(name + ("+kv_i8" if cfg.kv_i8 else ""), dom),
                "bytes_per_launch": v["bytes"] / v["launches"], "avg_launch_us": round(avg_s * 1e6, 2)}
        gem = {k: v for k, v in stats.items() if k.startswith("gemm")}
        if gem:
            domg = max(gem, key=lambda k: gem[k]["total_ms"])
            g = gem[domg]
            avg_g = g["total_ms"] / 1e3 / g["launches"]
            achg = g["flops"] / g["launches"] / avg_g / 1e12
            roof_prefill = {"bound": "mfma", "kernel": domg, "achieved": round(achg, 1), "peak": MFMA_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(achg / MFMA_PEAK_TFLOPS, 4),
                            "traffic": measured_traffic(name + ("+kv_i8" if cfg.kv_i8 else ""), domg),
                            "flops_per_launch": g["flops"] / g["launches"], "avg_launch_us": round(avg_g * 1e6, 2)}
    dec.close()
    del dec
    torch.cuda.empty_cache()
    res = {"workload": desc, "prompt_tokens": P, "decode_steps": N,
           "decode_tok_s": round(decode_tps, 2), "prefill_tok_s": round(prefill_tps, 1),
           "prefill_ms": round(pre_ms, 3), "decode_ms_per_token": round(dec_ms / N, 4),
           "ms_per_step": round(wall * 1e3 / steps, 3),
           "decode_hbm_frac": round(decode_bytes_tok * decode_tps / 1e9 / HBM_PEAK_GBS, 4),
           "decode_bytes_per_token": decode_bytes_tok,
           "prefill_mfma_frac": round(prefill_flops / (pre_ms / 1e3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
           "prefill_flops": prefill_flops,
           "roofline": roof, "roofline_prefill": roof_prefill, "kernels": kernels}
    return res, w, cfg, prompt


# The pages' own figures for this path (Apple M2 Pro Neural Engine, fp16;
# "LLMs on the ANE", ANEForge docs): context, not the target.
PAGES_CONTEXT = {"hardware": "Apple M2 Pro Neural Engine, fp16 weights",
                 "source": "LLMs on the ANE (ANEForge docs), prefill / decode figures",
                 "qwen3_0.6b_prefill_tok_s": 8600, "qwen3_0.6b_decode_tok_s": 75, "qwen3_8b_decode_tok_s": 7.5}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="q8b", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel profiled pass")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the verify (K=5 over 8192 tokens), batch-16 decode and 0.6B-shaped measurements")
    ap.add_argument("--decode-path", choices=["auto", "multi"], default="auto",
                    help="auto: one persistent launch per decode step where the shapes allow it; "
                         "multi: one launch per kernel")
    ap.add_argument("--kv-i8", action="store_true",
                    help="int8 KV cache (one fp32 scale per position and KV head); decode then runs one launch "
                         "per kernel; the verify and batch-16 extras use it too")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="override the workload's decode step count (for counter runs; not a bench figure)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import decoder_prefill_kv_amd as dpk

    torch.cuda.init()
    flags = 2 if args.decode_path == "multi" else 0  # DPK_FLAG_DECODE_MULTI
    try:
        head, w, cfg, prompt = run_workload(dpk, args.workload, args.steps, args.warmup, args.seed, flags,
                                            args.decode_steps, not args.no_profile, kv_i8=args.kv_i8)
        extra = {}
        if not args.no_extra and args.workload == "q8b" and args.decode_steps is None:
            log("[bench] verify K=5 over an 8192-token cache ...")
            extra["verify"] = bench_verify(dpk, cfg, w, args.seed, flags)
            log("[bench] verify: %s" % extra["verify"])
            torch.cuda.empty_cache()
            log("[bench] batch-16 decode over 4096-token caches ...")
            extra["batch16"] = bench_batch16(dpk, cfg, w, args.seed, flags)
            log("[bench] batch16: %s" % extra["batch16"])
            torch.cuda.empty_cache()
            # the 0.6B-shaped workloads (bf16 and 4-bit), same measurement
            for name in ("q06b", "q06b_q4"):
                r, _, _, _ = run_workload(dpk, name, 2, 1, args.seed, flags)
                extra[name] = r
                log("[bench] %s: decode %.1f tok/s, prefill %.0f tok/s"
                    % (name, r["decode_tok_s"], r["prefill_tok_s"]))
            # the 8B-shaped model with integer-code weights (prefill 2048 + 64 decode steps)
            for name in ("q8b_i8", "q8b_q8", "q8b_q40"):
                r, _, _, _ = run_workload(dpk, name, 1, 1, args.seed, flags)
                extra[name] = r
                log("[bench] %s: decode %.1f tok/s, prefill %.0f tok/s"
                    % (name, r["decode_tok_s"], r["prefill_tok_s"]))
                torch.cuda.empty_cache()
    except DeviceError as e:
        print("bench.py: device-side error, no result reported: %s" % e, file=sys.stderr, flush=True)
        sys.exit(3)

    mem = membench()
    log("[bench] membench: %s" % mem)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(cfg, w, prompt)
        log("[bench] cpu oracle: %s" % cpu)

    out = {
        "metric": "decode tok/s & prefill tok/s, 8B-shaped bf16, 1 MI355X; % HBM / MFMA peak",
        "value": head["decode_tok_s"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.weight_format == "bf16" else cfg.weight_format,
        "data": "synthetic (seeded N(0,0.02) weights, uniform random prompt ids)",
        "config": {"workload": head["workload"], "prompt_tokens": head["prompt_tokens"],
                   "decode_steps": head["decode_steps"], "batch": 1, "decode_path": args.decode_path,
                   "kv_cache": "int8 + fp32 scale per position" if args.kv_i8 else "fp16"},
        "prefill_dtype": "fp16 operands, fp32 accumulation",
    }
    for k in ("decode_tok_s", "prefill_tok_s", "prefill_ms", "decode_ms_per_token", "decode_hbm_frac",
              "decode_bytes_per_token", "prefill_mfma_frac", "prefill_flops", "roofline", "roofline_prefill",
              "kernels"):
        out[k] = head[k]
    out["cpu_baseline"] = cpu
    out["membench"] = mem
    out["pages_context"] = PAGES_CONTEXT
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
