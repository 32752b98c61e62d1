"""Write the full-size reference fixtures tests/golden/<name>.npz.

Calls only the CPU oracle and the seeded input generator.  For each workload
it stores, for every compared logit vector (prefill, each decode step, each
verify row): the oracle's greedy id, its top-16 (index, value), max |logit|,
the tie-margin flag, and the logits at a fixed seeded subset of 2048 vocab
indices; the prefill logits are stored in full, and so are the whole logit
vectors of a few chosen records (``full_rows`` / ``full_logits``: decode steps
0, 1, the middle and the last one; every row of the first verify round).

Precision: float64 for the 0.6B-shaped models; the 8B-shaped model uses the
oracle's float32 path (same code, float32 tensors).  ``q8b_f64`` re-runs the
8B-shaped prefill and its first two decode steps in float64 (teacher-forced on
the float32 run's greedy ids), so the float32 path is pinned against the
definition at full depth (tests/test_oracle.py compares the two files).

Usage: python tests/golden/make_goldens.py q06b q06b_q4 q8b q8b_f64 q8b_verify q8b_batch16
"""
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402
import synth  # noqa: E402

N_SAMPLE = 2048
TOPK = 16


def sample_idx(vocab):
    return np.sort(synth.uniform_int(synth.key_of(0, "golden/sample"), N_SAMPLE, vocab)).astype(np.int32)


def summarize(lg, idx):
    lg = lg.to(torch.float64)
    tv, ti = torch.topk(lg, TOPK)
    return dict(id=oracle.argmax_lowest(lg), top_idx=ti.numpy().astype(np.int32), top_val=tv.numpy(),
                maxabs=float(lg.abs().max()), exempt=oracle.tie_exempt(lg), sample=lg.numpy()[idx])


def stack(recs):
    out = {}
    for k in recs[0]:
        out[k] = np.array([r[k] for r in recs])
    return out


def log(*a):
    print(*a, flush=True)


def full_steps(N):
    """Decode steps whose whole logit vector is kept: 0, 1, N/2 - 1, N - 1."""
    return sorted({0, min(1, N - 1), max(0, N // 2 - 1), N - 1})


def greedy_golden(name, cfg, P, N, dtype, prompt_index=0):
    w = synth.make_weights(cfg, 0)
    prompt = synth.prompt_ids(cfg, P, 0, index=prompt_index)
    m = oracle.OracleModel(cfg, w, dtype)
    idx = sample_idx(cfg.vocab)
    cache = m.new_cache(P + N)
    t = time.time()
    lg0 = m.forward_block(cache, prompt, 0)[0]
    log("[%s] prefill %d in %.0f s" % (name, P, time.time() - t))
    recs = [summarize(lg0, idx)]
    keep = full_steps(N)
    full = []
    for s in range(N):
        lg = m.forward_step(cache, recs[-1]["id"], P + s)
        recs.append(summarize(lg, idx))
        if s in keep:
            full.append(lg.numpy().astype(np.float32))
        if s % 16 == 0:
            log("[%s] step %d (%.0f s)" % (name, s, time.time() - t))
    out = stack(recs)
    # full_rows are record indices: record 0 is the prefill, record s + 1 decode step s
    out.update(prefill_logits=lg0.numpy().astype(np.float32), sample_idx=idx, prompt_len=P, n_steps=N,
               prompt_index=prompt_index, full_rows=np.array([s + 1 for s in keep], dtype=np.int32),
               full_logits=np.stack(full))
    return out, m, cache


def verify_golden(cfg, P, K, rounds, dtype):
    w = synth.make_weights(cfg, 0)
    prompt = synth.prompt_ids(cfg, P, 0)
    m = oracle.OracleModel(cfg, w, dtype)
    idx = sample_idx(cfg.vocab)
    cache = m.new_cache(P + (K + 1) * rounds + 1)
    t = time.time()
    lg0 = m.forward_block(cache, prompt, 0)[0]
    log("[verify] prefill %d in %.0f s" % (P, time.time() - t))
    first = summarize(lg0, idx)
    t_last, pos = first["id"], P
    rows, meta, full = [], [], []
    for r in range(rounds):
        # the oracle's greedy continuation (step path) gives the drafts
        greedy = []
        tok = t_last
        for i in range(K):
            lg = m.forward_step(cache, tok, pos + i)
            tok = oracle.argmax_lowest(lg)
            greedy.append(tok)
        cache.length = pos
        drafts = synth.corrupt_drafts(cfg, np.array(greedy), 0.3, 0, r)
        ids_in = [t_last] + [int(x) for x in drafts]
        res = oracle.verify(m, cache, ids_in, pos)
        for i in range(K + 1):
            rows.append(summarize(res["logits"][i], idx))
            if r == 0:
                full.append(res["logits"][i].numpy().astype(np.float32))
        meta.append((pos, res["accepted"], res["bonus"]) + tuple(ids_in))
        log("[verify] round %d pos %d accepted %d (%.0f s)" % (r, pos, res["accepted"], time.time() - t))
        t_last = res["bonus"]
        pos = pos + res["accepted"] + 1
    out = stack(rows)
    out.update(prefill=np.array([first["id"]]), prefill_logits=lg0.numpy().astype(np.float32), sample_idx=idx,
               prompt_len=P, K=K, rounds=np.array(meta, dtype=np.int64),
               full_rows=np.arange(K + 1, dtype=np.int32), full_logits=np.stack(full))
    return out


def f64_golden(cfg, P, ref_name):
    """float64 prefill of the same prompt and decode steps 0 and 1 fed the
    float32 run's greedy ids (weights widened per use, not cached)."""
    ref = np.load(os.path.join(HERE, ref_name + ".npz"))
    assert int(ref["prompt_len"]) == P
    w = synth.make_weights(cfg, 0)
    prompt = synth.prompt_ids(cfg, P, 0)
    m = oracle.OracleModel(cfg, w, torch.float64, cache_weights=False)
    cache = m.new_cache(P + 2)
    t = time.time()
    lg0 = m.forward_block(cache, prompt, 0)[0]
    log("[f64] prefill %d in %.0f s" % (P, time.time() - t))
    rows = [lg0.numpy()]
    for s in range(2):
        rows.append(m.forward_step(cache, int(ref["id"][s]), P + s).numpy())
        log("[f64] step %d (%.0f s)" % (s, time.time() - t))
    return dict(records=np.arange(3, dtype=np.int32), logits=np.stack(rows), prompt_len=P,
                fed_ids=ref["id"][:2].astype(np.int32))


def main():
    names = sys.argv[1:] or ["q06b", "q06b_q4", "q8b", "q8b_f64", "q8b_verify", "q8b_batch16"]
    torch.set_num_threads(int(os.environ.get("GOLDEN_THREADS", "6")))
    for name in names:
        t = time.time()
        if name == "q06b":
            out, _, _ = greedy_golden(name, synth.Q06B, 512, 128, torch.float64)
        elif name == "q06b_q4":
            out, _, _ = greedy_golden(name, synth.Q06B_Q4, 2048, 128, torch.float64)
        elif name == "q8b":
            out, _, _ = greedy_golden(name, synth.Q8B, 2048, 256, torch.float32)
        elif name == "q8b_f64":
            out = f64_golden(synth.Q8B, 2048, "q8b")
        elif name == "q8b_verify":
            out = verify_golden(synth.Q8B, 8192, 5, 8, torch.float32)
        elif name == "q8b_batch16":
            parts = {}
            for b in (0, 15):
                o, _, _ = greedy_golden("%s/%d" % (name, b), synth.Q8B, 4096, 32, torch.float32, prompt_index=b)
                for k, v in o.items():
                    parts["s%d_%s" % (b, k)] = v
            out = parts
        else:
            raise SystemExit("unknown golden " + name)
        np.savez_compressed(os.path.join(HERE, name + ".npz"), **out)
        log("[%s] written in %.0f s" % (name, time.time() - t))


if __name__ == "__main__":
    main()
