"""Shared helpers of the parity tests: oracle runs and GPU teacher-forced runs.

Tolerances (logits max-abs): 1e-4 for the fp32 model, 2e-2 for bf16 / 4-bit /
int8 weights.  Greedy ids must match except where the oracle's top-2 gap is below
3e-3 of its max |logit| (tie-margin rule)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

TOL = {"f32": 1e-4, "bf16": 2e-2, "q4": 2e-2, "i8": 2e-2, "q8": 2e-2, "q4_0": 2e-2}


def oracle_greedy(cfg, weights, prompt, n_steps):
    m = oracle.OracleModel(cfg, weights)
    run = oracle.greedy_run(m, prompt, n_steps)
    return m, run


def compare_logits(gpu, ref, tol, what=""):
    ref = ref.to(torch.float64)
    gpu = gpu.to(torch.float64)
    d = (gpu - ref).abs()
    mx = float(d.max())
    assert torch.isfinite(gpu).all(), "%s: non-finite GPU logits" % what
    assert mx <= tol, "%s: max-abs %.3g > %.3g (at %d)" % (what, mx, tol, int(d.argmax()))
    return mx


def check_ids(gpu_ids, ref_logits_list, ref_ids, what=""):
    bad = []
    for i, (g, r) in enumerate(zip(gpu_ids, ref_ids)):
        if int(g) != int(r) and not oracle.tie_exempt(ref_logits_list[i]):
            bad.append((i, int(g), int(r)))
    assert not bad, "%s: greedy ids differ at non-tie steps %s" % (what, bad[:5])


def gpu_teacher_forced(dec, prompt, forced, n_steps, seq=0):
    """Prefill, then n_steps decode steps feeding forced[s] at position P+s."""
    P = len(prompt)
    lg = dec.logits_buffer(1)
    am = dec.argmax_buffer(1)
    dec.prefill(seq, [int(t) for t in prompt], lg, am)
    logits = [lg[0].cpu()]
    ids = [int(am.cpu()[0])]
    for s in range(n_steps):
        dec.decode_step([seq], [int(forced[s])], [P + s], am, lg)
        logits.append(lg[0].cpu())
        ids.append(int(am.cpu()[0]))
    return logits, ids


def small(cfg: synth.ModelConfig, **kw) -> synth.ModelConfig:
    return cfg.with_(**kw)
