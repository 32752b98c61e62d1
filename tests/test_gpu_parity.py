"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Every comparison is element-wise over full logit vectors, teacher-forced on
the oracle's greedy ids (prefill logits, then each decode step)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, check_ids, compare_logits, gpu_teacher_forced, oracle_greedy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dpk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_prefill_kv_amd as dpk
    return dpk


STREAM = 1  # DPK_FLAG_PREFILL_STREAM: prefill through the decode kernels
MULTI = 2   # DPK_FLAG_DECODE_MULTI: decode as one launch per kernel (these
            # shapes otherwise decode in one persistent launch)
CASES = [
    # (name, config, prompt length, decode steps, Decoder kwargs); weight-
    # streaming prefill first, then the MFMA GEMM prefill path
    ("tiny", synth.TINY, 16, 16, {}),
    ("q06b-L2-stream", synth.Q06B.with_(n_layers=2), 40, 8, dict(flags=STREAM)),
    ("q06b_q4-L2-stream", synth.Q06B_Q4.with_(n_layers=2), 37, 6, dict(flags=STREAM)),
    ("q8b-L1-v4096-stream", synth.Q8B.with_(n_layers=1, vocab=4096), 21, 5, dict(flags=STREAM)),
    ("q06b-L2-gemm", synth.Q06B.with_(n_layers=2), 40, 8, {}),
    ("q06b_q4-L2-gemm", synth.Q06B_Q4.with_(n_layers=2), 37, 6, {}),
    ("q8b-L1-v4096-gemm", synth.Q8B.with_(n_layers=1, vocab=4096), 21, 5, {}),
    ("q06b-L2-chunked", synth.Q06B.with_(n_layers=2), 300, 4, dict(max_rows=128)),
    ("q06b-L2-multi", synth.Q06B.with_(n_layers=2), 40, 8, dict(flags=MULTI)),
    ("q06b_q4-L2-multi", synth.Q06B_Q4.with_(n_layers=2), 37, 6, dict(flags=MULTI)),
    ("q06b_q4-L2-persistent-ctx300", synth.Q06B_Q4.with_(n_layers=2), 290, 12, dict(max_rows=128)),
    # hidden 1024 with 4 query heads per KV head: the 128-column persistent step for G = 4
    ("h1024-g4-L2-v4096", synth.Q06B.with_(n_layers=2, n_kv_heads=4, vocab=4096), 260, 6, dict(max_rows=128)),
    ("h1024-g4-q4-L2-v4096", synth.Q06B_Q4.with_(n_layers=2, n_kv_heads=4, vocab=4096), 260, 6, dict(max_rows=128)),
    ("q8b-L2-v4096-chunked", synth.Q8B.with_(n_layers=2, vocab=4096), 600, 4, dict(max_rows=256)),
    ("q8b-L2-v4096-multi", synth.Q8B.with_(n_layers=2, vocab=4096), 250, 12, dict(flags=MULTI, max_rows=256)),
    ("q8b-L2-v4096-persistent", synth.Q8B.with_(n_layers=2, vocab=4096), 250, 12, dict(max_rows=256)),
    # prompts long enough for the QKV projection to run on 256 x 256 tiles, whose
    # epilogue applies QK-norm / RoPE and writes the cache (one chunk; chunks
    # at offsets 0 and 1400 plus a short tail)
    ("q8b-L1-v4096-qkv-epilogue", synth.Q8B.with_(n_layers=1, vocab=4096), 1400, 3, dict(max_rows=1400)),
    ("q8b-L1-v4096-qkv-epilogue-chunked", synth.Q8B.with_(n_layers=1, vocab=4096), 2900, 3, dict(max_rows=1400)),
    # int8 per-channel weights: GEMM prefill from the fp16 copy, weight-streaming decode
    ("q06b_i8-L2-gemm", synth.Q06B_I8.with_(n_layers=2), 40, 8, {}),
    ("q06b_i8-L2-stream", synth.Q06B_I8.with_(n_layers=2), 37, 6, dict(flags=STREAM)),
    ("q8b_i8-L1-v4096-gemm", synth.Q8B_I8.with_(n_layers=1, vocab=4096), 21, 5, {}),
    ("q8b_i8-L2-v4096-chunked", synth.Q8B_I8.with_(n_layers=2, vocab=4096), 300, 4, dict(max_rows=128)),
    # int8 in blocks of 32 with fp32 scales: the same paths, a scale per MFMA k-step
    ("q06b_q8-L2-gemm", synth.Q06B_Q8.with_(n_layers=2), 40, 8, {}),
    ("q06b_q8-L2-stream", synth.Q06B_Q8.with_(n_layers=2), 37, 6, dict(flags=STREAM)),
    ("q8b_q8-L1-v4096-gemm", synth.Q8B_Q8.with_(n_layers=1, vocab=4096), 21, 5, {}),
    ("q8b_q8-L2-v4096-chunked", synth.Q8B_Q8.with_(n_layers=2, vocab=4096), 300, 4, dict(max_rows=128)),
    # int8 KV cache: prefill (GEMM, streamed, chunked over the cache), decode; bf16 and Q8 weights
    ("q06b-kvi8-L2-gemm", synth.Q06B.with_(n_layers=2, kv_i8=True), 40, 8, {}),
    ("q06b-kvi8-L2-stream", synth.Q06B.with_(n_layers=2, kv_i8=True), 37, 6, dict(flags=STREAM)),
    ("q8b-kvi8-L1-v4096-chunked", synth.Q8B.with_(n_layers=1, vocab=4096, kv_i8=True), 300, 6, dict(max_rows=128)),
    # the persistent step over the int8 cache (bf16 weights with the fused O
    # projection, int8 weights): positions crossing a 256-position chunk boundary
    ("q8b-kvi8-L2-v4096-persistent", synth.Q8B.with_(n_layers=2, vocab=4096, kv_i8=True), 510, 6, dict(max_rows=256)),
    ("q8b_i8-kvi8-L2-v4096-persistent", synth.Q8B_I8.with_(n_layers=2, vocab=4096, kv_i8=True), 250, 8,
     dict(max_rows=256)),
    ("q06b_q8-kvi8-L2-gemm", synth.Q06B_Q8.with_(n_layers=2, kv_i8=True), 40, 8, {}),
    # GGUF-style Q4_0 blocks: the same paths with 4-bit codes around 8 and fp16 scales
    ("q06b_q40-L2-gemm", synth.Q06B_Q40.with_(n_layers=2), 40, 8, {}),
    ("q06b_q40-L2-stream", synth.Q06B_Q40.with_(n_layers=2), 37, 6, dict(flags=STREAM)),
    ("q8b_q40-L1-v4096-gemm", synth.Q8B_Q40.with_(n_layers=1, vocab=4096), 21, 5, {}),
    ("q8b_q40-L2-v4096-chunked", synth.Q8B_Q40.with_(n_layers=2, vocab=4096), 300, 4, dict(max_rows=128)),
    # Q4_0 in the persistent step (decode positions crossing a 256-position
    # chunk), over the fp16 and the int8 cache (the prefill's K and V then
    # include the fp16 copy's rounding residuals)
    ("q8b_q40-L2-v4096-persistent", synth.Q8B_Q40.with_(n_layers=2, vocab=4096), 250, 8, dict(max_rows=256)),
    ("q8b_q40-kvi8-L2-v4096-persistent", synth.Q8B_Q40.with_(n_layers=2, vocab=4096, kv_i8=True), 250, 8,
     dict(max_rows=256)),
    ("q8b_q40-kvi8-L2-v4096-short", synth.Q8B_Q40.with_(n_layers=2, vocab=4096, kv_i8=True), 40, 4, {}),
    ("q06b_q4-kvi8-L2-gemm", synth.Q06B_Q4.with_(n_layers=2, kv_i8=True), 40, 4, {}),
    # Q8 in the persistent step, over the fp16 and the int8 cache
    ("q8b_q8-L2-v4096-persistent", synth.Q8B_Q8.with_(n_layers=2, vocab=4096), 250, 8, dict(max_rows=256)),
    ("q8b_q8-kvi8-L2-v4096-persistent", synth.Q8B_Q8.with_(n_layers=2, vocab=4096, kv_i8=True), 250, 8,
     dict(max_rows=256)),
    # the 128-column persistent step over the int8 cache (0.6B shapes, bf16 and
    # MLX 4-bit), contexts of three attention chunks
    ("q06b-kvi8-L2-persistent-ctx600", synth.Q06B.with_(n_layers=2, kv_i8=True), 590, 8, dict(max_rows=256)),
    ("q06b_q4-kvi8-L2-persistent-ctx600", synth.Q06B_Q4.with_(n_layers=2, kv_i8=True), 590, 8, dict(max_rows=256)),
    # the int8 cache at a long context in the persistent step: 16 attention
    # chunks per (row, KV head) and their merge
    ("q8b-kvi8-L1-v4096-ctx4100", synth.Q8B.with_(n_layers=1, vocab=4096, kv_i8=True), 4080, 4,
     dict(max_rows=2048)),
    # the persistent step's other query-group sizes: the int8 cache with 2 and 1
    # query heads per KV head (bf16, fused O projection), Q4_0 with 2, Q8 with 1
    ("h2048-g2-kvi8-L2-v4096-persistent",
     synth.Q8B.with_(n_layers=2, hidden=2048, n_heads=16, n_kv_heads=8, intermediate=4096, vocab=4096, kv_i8=True),
     250, 6, dict(max_rows=256)),
    ("h2048-g1-kvi8-L2-v4096-persistent",
     synth.Q8B.with_(n_layers=2, hidden=2048, n_heads=16, n_kv_heads=16, intermediate=4096, vocab=4096, kv_i8=True),
     250, 6, dict(max_rows=256)),
    ("q8b_q40-g2-L2-v4096-persistent", synth.Q8B_Q40.with_(n_layers=2, n_kv_heads=16, intermediate=4096, vocab=4096),
     250, 6, dict(max_rows=256)),
    ("q8b_q8-g1-L2-v4096-persistent", synth.Q8B_Q8.with_(n_layers=2, n_kv_heads=32, intermediate=4096, vocab=4096),
     250, 6, dict(max_rows=256)),
]


@pytest.mark.parametrize("name,cfg,P,N,kw", CASES, ids=[c[0] for c in CASES])
def test_prefill_and_decode_match_oracle(dpk, name, cfg, P, N, kw):
    print("\n[parity] %s P=%d N=%d %s" % (name, P, N, kw), flush=True)
    w = synth.make_weights(cfg, 0)
    prompt = synth.prompt_ids(cfg, P, 0)
    _, run = oracle_greedy(cfg, w, prompt, N)
    args = dict(max_rows=64)
    args.update(kw)
    dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=P + N, **args)
    logits, ids = gpu_teacher_forced(dec, prompt, run["ids"], N)
    torch.cuda.synchronize()
    tol = TOL[cfg.weight_format]
    worst = 0.0
    for i in range(N + 1):
        worst = max(worst, compare_logits(logits[i], run["logits"][i], tol, "%s step %d" % (name, i)))
    check_ids(ids, run["logits"], run["ids"], name)
    dpk.check_device_errors(dec.handle)
    print("[parity] %s worst max-abs %.3g" % (name, worst), flush=True)
    dec.close()


# hidden size 2048, bf16: the persistent step runs the O projection inside
# the attention phase (split by KV head, fixed-point sums); with 4 and 8 KV
# heads its items are 32- and 64-row blocks shared by 4 and 2 waves per row
# tile
H2048_G4 = synth.Q8B.with_(n_layers=2, hidden=2048, n_heads=16, n_kv_heads=4, intermediate=4096, vocab=4096)
H2048_G2 = synth.Q8B.with_(n_layers=2, hidden=2048, n_heads=16, n_kv_heads=8, intermediate=4096, vocab=4096)

PERSISTENT_CFGS = [
    # (name, config, prompt length): contexts P .. P + 31 cross a 256-position
    # attention chunk boundary; the long ones merge 17 chunks
    ("q8b-L2-v4096", synth.Q8B.with_(n_layers=2, vocab=4096), 250),          # 256 columns per wave step
    ("q06b-L2-v4096", synth.Q06B.with_(n_layers=2, vocab=4096), 250),        # 128 columns, bf16
    ("q06b_q4-L2-v4096", synth.Q06B_Q4.with_(n_layers=2, vocab=4096), 250),  # 128 columns, 4-bit
    ("h2048-g4-L2-v4096", H2048_G4, 250),                                   # O projection in the attention phase
    ("h2048-g2-L2-v4096", H2048_G2, 250),
    ("q8b-L1-v4096-ctx4100", synth.Q8B.with_(n_layers=1, vocab=4096), 4080),
    ("q06b_q4-L1-v4096-ctx4100", synth.Q06B_Q4.with_(n_layers=1, vocab=4096), 4080),
    ("q8b_i8-L2-v4096", synth.Q8B_I8.with_(n_layers=2, vocab=4096), 250),    # int8 codes, one scale per row
    ("q8b_q40-L2-v4096", synth.Q8B_Q40.with_(n_layers=2, vocab=4096), 250),  # Q4_0 blocks
    ("q8b_q8-L2-v4096", synth.Q8B_Q8.with_(n_layers=2, vocab=4096), 250),    # Q8 blocks
]


@pytest.mark.parametrize("name,cfg,P", PERSISTENT_CFGS, ids=[c[0] for c in PERSISTENT_CFGS])
def test_persistent_decode_matches_multi_launch(dpk, name, cfg, P):
    """The one-launch decode step against the one-launch-per-kernel path on
    the same model and tokens, across attention chunk boundaries and with
    several chunks merged."""
    w = synth.make_weights(cfg, 0)
    N = 32
    prompt = [int(t) for t in synth.prompt_ids(cfg, P, 0)]
    feed = [int(t) for t in synth.prompt_ids(cfg, N, 1)]  # the same tokens for both paths
    outs = []
    for flags in (0, MULTI):
        print("\n[parity] persistent-vs-multi %s flags=%d" % (name, flags), flush=True)
        dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=(P + N + 63) // 64 * 64, max_rows=256, flags=flags)
        lg = dec.logits_buffer(1)
        am = dec.argmax_buffer(1)
        dec.prefill(0, prompt, lg, am)
        rows = []
        for s in range(N):
            dec.decode_step([0], [feed[s]], [P + s], am, lg)
            rows.append(lg[0].clone())
        torch.cuda.synchronize()
        dpk.check_device_errors(dec.handle)
        outs.append(torch.stack(rows).cpu())
        dec.close()
    d = (outs[0] - outs[1]).abs().max().item()
    print("[parity] %s persistent vs multi-launch decode max-abs %.3g" % (name, d), flush=True)
    assert d <= 1e-3


PATH_CASES = [
    ("q8b-L1-v4096", synth.Q8B.with_(n_layers=1, vocab=4096), True),
    ("q06b-L1", synth.Q06B.with_(n_layers=1), True),
    ("q06b_q4-L1", synth.Q06B_Q4.with_(n_layers=1), True),
    ("tiny-f32", synth.TINY, False),
    ("q06b_i8-L1", synth.Q06B_I8.with_(n_layers=1), False),
    ("q06b_q8-L1", synth.Q06B_Q8.with_(n_layers=1), False),
    ("q06b_q40-L1", synth.Q06B_Q40.with_(n_layers=1), False),
    ("q06b-kvi8-L1", synth.Q06B.with_(n_layers=1, kv_i8=True), True),
    ("q8b-kvi8-L1-v4096", synth.Q8B.with_(n_layers=1, vocab=4096, kv_i8=True), True),
    ("q8b_i8-kvi8-L1-v4096", synth.Q8B_I8.with_(n_layers=1, vocab=4096, kv_i8=True), True),
    ("q8b_q40-L1-v4096", synth.Q8B_Q40.with_(n_layers=1, vocab=4096), True),
    ("q8b_q8-L1-v4096", synth.Q8B_Q8.with_(n_layers=1, vocab=4096), True),
    ("h2048-g1-kvi8-L1-v4096",
     synth.Q8B.with_(n_layers=1, hidden=2048, n_heads=16, n_kv_heads=16, intermediate=4096, vocab=4096, kv_i8=True), True),
    ("q8b_q8-g1-L1-v4096", synth.Q8B_Q8.with_(n_layers=1, n_kv_heads=32, intermediate=4096, vocab=4096), True),
    ("q8b_i8-L1-v4096", synth.Q8B_I8.with_(n_layers=1, vocab=4096), True),
]


@pytest.mark.parametrize("name,cfg,persistent", PATH_CASES, ids=[c[0] for c in PATH_CASES])
def test_decode_path_taken(dpk, name, cfg, persistent):
    """Which decode path a batch-1 step takes: one persistent launch
    ('decode.step' in the profile) for bf16 / 4-bit models whose shapes it
    supports, one launch per kernel otherwise."""
    w = synth.make_weights(cfg, 0)
    P = 24
    dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=P + 8, max_rows=64)
    lg, am = dec.logits_buffer(1), dec.argmax_buffer(1)
    dec.prefill(0, [int(t) for t in synth.prompt_ids(cfg, P, 0)], lg, am)
    dpk.profile_begin(dec.handle, 10000)
    dec.decode_step([0], None, [P], am, lg, ids_dev=am)
    stats = dpk.profile_end(dec.handle)
    dpk.check_device_errors(dec.handle)
    dec.close()
    print("\n[parity] %s decode classes %s" % (name, sorted(stats)), flush=True)
    assert ("decode.step" in stats) == persistent, sorted(stats)
    if persistent:
        assert not any(k.startswith("gemv.") or k.startswith("attn.") for k in stats), sorted(stats)


KV_I8_CASES = [
    # (name, config, decoder flags): the cache writers are the prefill rows kernel
    # and the decode attention (bf16), the streamed prefill's per-row kernel, and
    # the int8-code GEMV's QKV epilogue (Q8 weights)
    ("bf16-gemm", synth.Q06B.with_(n_layers=2, kv_i8=True), 0),
    ("bf16-stream", synth.Q06B.with_(n_layers=2, kv_i8=True), STREAM),
    ("q8-gemm", synth.Q06B_Q8.with_(n_layers=2, kv_i8=True), 0),
    # (8B shapes: the decode positions written by the persistent step)
    ("bf16-8b-persistent", synth.Q8B.with_(n_layers=1, vocab=4096, kv_i8=True), 0),
]


@pytest.mark.parametrize("name,cfg,flags", KV_I8_CASES, ids=[c[0] for c in KV_I8_CASES])
def test_int8_kv_cache_holds_the_oracle_codes(dpk, name, cfg, flags):
    """The int8 cache itself, read back from the device: layer 0's keys and
    values (which do not depend on the cache) after a 40-token prefill and 4
    decode steps, against the oracle's quantized cache -- scales within fp32
    rounding, codes equal but for rare +-1 at near-ties."""
    w = synth.make_weights(cfg, 0)
    P, N = 40, 4
    prompt = synth.prompt_ids(cfg, P, 0)
    m, run = oracle_greedy(cfg, w, prompt, N)
    dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=P + N + 8, max_rows=64, flags=flags)
    lg, am = dec.logits_buffer(1), dec.argmax_buffer(1)
    dec.prefill(0, [int(t) for t in prompt], lg, am)
    for s in range(N):
        dec.decode_step([0], [run["ids"][s]], [P + s], am, lg)
    torch.cuda.synchronize()
    dpk.check_device_errors(dec.handle)
    raw = dec.kv.cpu().numpy()
    dec.close()
    L, Hkv, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    S = (P + N + 8 + 63) // 64 * 64
    n = L * 2 * Hkv * S * d  # one sequence slot
    codes = raw[:n].view(np.int8).reshape(L, 2, Hkv, S, d)
    off = (n + 255) // 256 * 256
    scales = raw[off:off + L * 2 * Hkv * S * 4].view(np.float32).reshape(L, 2, Hkv, S)
    T = P + N
    for which, ref in ((0, run["cache"].k[0]), (1, run["cache"].v[0])):
        ref = ref[:, :T, :].numpy()                                   # [Hkv, T, d], values s * q
        gs = scales[0, which, :, :T].astype(np.float64)              # [Hkv, T]
        gq = codes[0, which] if which == 0 else codes[0, which].reshape(Hkv, d, S).transpose(0, 2, 1)
        gq = gq[:, :T, :].astype(np.int64)
        rs = np.abs(ref).max(axis=2) / 127.0                         # the oracle's scale (s * 127 = max |s q|)
        # bf16 weights are exact in the fp16 prefill copy; Q8's s * q is rounded
        # to fp16 there (2^-11 relative per weight), which moves k and v as much
        rtol = 2e-5 if cfg.weight_format == "bf16" else 2e-3
        rel = float((np.abs(gs - rs) / np.maximum(rs, 1e-30)).max())
        print("\n[kv-i8] %s %s: scale rel. diff %.3g" % (name, "KV"[which], rel), flush=True)
        assert rel <= rtol, "%s %d: scales %.3g" % (name, which, rel)
        rq = np.rint(ref / np.where(rs > 0, rs, 1.0)[..., None]).astype(np.int64)
        diff = np.abs(gq - rq)
        print("[kv-i8] %s %s: codes off by one %.4f" % (name, "KV"[which], float(diff.mean())), flush=True)
        assert diff.max() <= 1 and diff.mean() < (5e-3 if cfg.weight_format == "bf16" else 5e-2), \
            "%s %d: codes differ (%d, %.4f)" % (name, which, int(diff.max()), float(diff.mean()))


def test_prefill_without_outputs_then_decode(dpk):
    # prefill with neither logits nor argmax buffers (both optional)
    cfg = synth.Q06B.with_(n_layers=2)
    w = synth.make_weights(cfg, 0)
    prompt = synth.prompt_ids(cfg, 20, 0)
    _, run = oracle_greedy(cfg, w, prompt, 1)
    dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=24, max_rows=64)
    for flags_prompt in (prompt[:5], prompt):   # stream-sized and GEMM-sized
        dec.prefill(0, [int(t) for t in flags_prompt])
    lg, am = dec.logits_buffer(1), dec.argmax_buffer(1)
    dec.decode_step([0], [run["ids"][0]], [20], am, lg)
    compare_logits(lg[0].cpu(), run["logits"][1], TOL["bf16"], "decode after bare prefill")
    dec.close()


VERIFY_CASES = [
    # (id, config, prompt length, drafts K): one group of rows per KV head;
    # 4-bit weights with two row groups; ready-made-activation GEMVs with two
    # row groups across the 256-position chunk edge; 16 rows across 512
    ("q06b-L2-k5", synth.Q06B.with_(n_layers=2), 33, 5),
    ("q06b_q4-L2-k11", synth.Q06B_Q4.with_(n_layers=2), 300, 11),
    ("q8b-L1-v4096-k5", synth.Q8B.with_(n_layers=1, vocab=4096), 254, 5),
    ("q8b-L1-v4096-k15", synth.Q8B.with_(n_layers=1, vocab=4096), 500, 15),
    ("q06b_i8-L2-k5", synth.Q06B_I8.with_(n_layers=2), 70, 5),
    ("q06b_q8-L2-k5", synth.Q06B_Q8.with_(n_layers=2), 70, 5),
    ("q06b_q40-L2-k5", synth.Q06B_Q40.with_(n_layers=2), 70, 5),
    ("q06b-kvi8-L2-k5", synth.Q06B.with_(n_layers=2, kv_i8=True), 70, 5),
    ("q8b-kvi8-L1-v4096-k15", synth.Q8B.with_(n_layers=1, vocab=4096, kv_i8=True), 500, 15),
]


@pytest.mark.parametrize("case", VERIFY_CASES, ids=[c[0] for c in VERIFY_CASES])
def test_verify_matches_oracle(dpk, case):
    _, cfg, P, K = case
    w = synth.make_weights(cfg, 0)
    prompt = synth.prompt_ids(cfg, P, 0)
    m, run = oracle_greedy(cfg, w, prompt, K + 1)
    g = run["ids"]
    drafts = synth.corrupt_drafts(cfg, np.array(g[1:K + 1]), 0.3, 0, 0)
    drafts[3] = (g[4] + 1) % cfg.vocab  # at least one rejection
    ids_in = [g[0]] + [int(x) for x in drafts]
    c = m.new_cache(P + K + 1)
    m.forward_block(c, prompt, 0)
    ref = oracle.verify(m, c, ids_in, P)
    dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=(P + K + 64) // 64 * 64, max_rows=512)
    lg = dec.logits_buffer(K + 1)
    am = dec.argmax_buffer(K + 1)
    dec.prefill(0, [int(t) for t in prompt])
    acc = dec.verify(0, ids_in, P, am, lg)
    for i in range(K + 1):
        compare_logits(lg[i].cpu(), ref["logits"][i], TOL[cfg.weight_format], "verify row %d" % i)
    check_ids(am.cpu().tolist(), list(ref["logits"]), ref["argmax"], "verify")
    dpk.check_device_errors(dec.handle)
    assert acc == ref["accepted"]
    assert dec.seq_length(0) == P + acc + 1
    dec.close()


def test_batched_decode_matches_oracle(dpk):
    cfg = synth.Q06B.with_(n_layers=2)
    w = synth.make_weights(cfg, 0)
    lens = [9, 23, 17]
    N = 4
    prompts = [synth.prompt_ids(cfg, L, 0, index=b) for b, L in enumerate(lens)]
    runs = [oracle_greedy(cfg, w, p, N)[1] for p in prompts]
    dec = dpk.Decoder(cfg, w, max_batch=4, max_seq=64, max_rows=64)
    B = len(lens)
    for b in range(B):
        dec.prefill(b + 1, [int(t) for t in prompts[b]])  # slots 1..3
    lg = dec.logits_buffer(B)
    am = dec.argmax_buffer(B)
    for s in range(N):
        toks = [runs[b]["ids"][s] for b in range(B)]
        dec.decode_step([b + 1 for b in range(B)], toks, [lens[b] + s for b in range(B)], am, lg)
        for b in range(B):
            compare_logits(lg[b].cpu(), runs[b]["logits"][s + 1], TOL["bf16"], "batch row %d step %d" % (b, s))
    dec.close()


BATCHED_PERSISTENT = [("q06b-L2", synth.Q06B.with_(n_layers=2)), ("q06b_q4-L2", synth.Q06B_Q4.with_(n_layers=2)),
                      ("h2048-g4-L2-v4096", H2048_G4), ("h2048-g2-L2-v4096", H2048_G2)]


def test_batched_decode_int8_8b_rows(dpk):
    """Two sequences of an 8B-shaped int8 model decoded together in one
    persistent launch (contexts of one and two chunks; the staged activations
    of two rows fit its LDS beside the int8 mode's buffers)."""
    cfg = synth.Q8B_I8.with_(n_layers=1, vocab=4096)
    w = synth.make_weights(cfg, 0)
    lens, N = [200, 300], 3
    prompts = [synth.prompt_ids(cfg, L, 0, index=b) for b, L in enumerate(lens)]
    runs = [oracle_greedy(cfg, w, p, N)[1] for p in prompts]
    dec = dpk.Decoder(cfg, w, max_batch=2, max_seq=320, max_rows=256)
    for b in range(2):
        dec.prefill(b, [int(t) for t in prompts[b]])
    lg, am = dec.logits_buffer(2), dec.argmax_buffer(2)
    for s in range(N):
        toks = [runs[b]["ids"][s] for b in range(2)]
        if s == 0:
            dpk.profile_begin(dec.handle, 10000)
        dec.decode_step([0, 1], toks, [lens[b] + s for b in range(2)], am, lg)
        if s == 0:
            stats = dpk.profile_end(dec.handle)
            assert "decode.step" in stats, sorted(stats)
        for b in range(2):
            compare_logits(lg[b].cpu(), runs[b]["logits"][s + 1], TOL["i8"], "int8 row %d step %d" % (b, s))
    dpk.check_device_errors(dec.handle)
    dec.close()


@pytest.mark.parametrize("name,cfg", [("q8", synth.Q8B_Q8.with_(n_layers=1, vocab=4096)),
                                      ("q4_0", synth.Q8B_Q40.with_(n_layers=1, vocab=4096))], ids=["q8", "q4_0"])
def test_batched_persistent_decode_block_formats_8b_rows(dpk, name, cfg):
    """Two sequences of an 8B-shaped Q8 / Q4_0 model decoded together in one
    persistent launch (contexts of one and two chunks): the block modes' D rows
    1..M-1, which batch-1 steps never use."""
    w = synth.make_weights(cfg, 0)
    lens, N = [200, 300], 3
    prompts = [synth.prompt_ids(cfg, L, 0, index=b) for b, L in enumerate(lens)]
    runs = [oracle_greedy(cfg, w, p, N)[1] for p in prompts]
    dec = dpk.Decoder(cfg, w, max_batch=2, max_seq=320, max_rows=256)
    for b in range(2):
        dec.prefill(b, [int(t) for t in prompts[b]])
    lg, am = dec.logits_buffer(2), dec.argmax_buffer(2)
    worst = 0.0
    for s in range(N):
        toks = [runs[b]["ids"][s] for b in range(2)]
        if s == 0:
            dpk.profile_begin(dec.handle, 10000)
        dec.decode_step([0, 1], toks, [lens[b] + s for b in range(2)], am, lg)
        if s == 0:
            stats = dpk.profile_end(dec.handle)
            assert "decode.step" in stats, sorted(stats)
        for b in range(2):
            worst = max(worst, compare_logits(lg[b].cpu(), runs[b]["logits"][s + 1], TOL[cfg.weight_format],
                                              "%s row %d step %d" % (name, b, s)))
    dpk.check_device_errors(dec.handle)
    dec.close()
    print("\n[parity] %s 2-row persistent worst max-abs %.3g" % (name, worst), flush=True)


@pytest.mark.parametrize("name,cfg", BATCHED_PERSISTENT, ids=[c[0] for c in BATCHED_PERSISTENT])
def test_batched_persistent_decode_long_contexts(dpk, name, cfg):
    """Three sequences decoded together through the persistent step (M = 3
    rows, each with its own position and cache), with contexts of one, two
    and three attention chunks."""
    w = synth.make_weights(cfg, 0)
    lens = [200, 300, 530]
    N = 3
    prompts = [synth.prompt_ids(cfg, L, 0, index=b) for b, L in enumerate(lens)]
    runs = [oracle_greedy(cfg, w, p, N)[1] for p in prompts]
    dec = dpk.Decoder(cfg, w, max_batch=3, max_seq=576, max_rows=256)
    B = len(lens)
    for b in range(B):
        dec.prefill(b, [int(t) for t in prompts[b]])
    lg = dec.logits_buffer(B)
    am = dec.argmax_buffer(B)
    worst = 0.0
    for s in range(N):
        toks = [runs[b]["ids"][s] for b in range(B)]
        if s == 0:
            dpk.profile_begin(dec.handle, 10000)
        dec.decode_step(list(range(B)), toks, [lens[b] + s for b in range(B)], am, lg)
        if s == 0:
            stats = dpk.profile_end(dec.handle)
            assert "decode.step" in stats, sorted(stats)  # the persistent kernel took all three rows
        for b in range(B):
            worst = max(worst, compare_logits(lg[b].cpu(), runs[b]["logits"][s + 1], TOL[cfg.weight_format],
                                              "%s row %d step %d" % (name, b, s)))
    dpk.check_device_errors(dec.handle)
    print("\n[parity] %s batched persistent worst max-abs %.3g" % (name, worst), flush=True)
    dec.close()



BATCH16_CASES = [
    # (name, config, prompt lengths): independent sequences decoded together on
    # the ready-made-activation GEMVs (more rows than the persistent step
    # stages); contexts of one and two attention chunks.  With more than 8 rows
    # the lm_head runs on two workgroups per compute unit, more than a small
    # vocabulary has row blocks: its argmax candidates must still fit.
    ("q8b-L1-v4096-M16", synth.Q8B.with_(n_layers=1, vocab=4096), [5 + 17 * b for b in range(16)]),
    ("q06b-L2-v4096-M16", synth.Q06B.with_(n_layers=2, vocab=4096), [300 - 19 * b for b in range(16)]),
    ("q8b-L1-v4096-M2", synth.Q8B.with_(n_layers=1, vocab=4096), [270, 31]),
    # 4-bit weights: the rows go through the 4-bit skinny GEMVs
    ("q06b_q4-L2-v4096-M16", synth.Q06B_Q4.with_(n_layers=2, vocab=4096), [40 + 13 * b for b in range(16)]),
    ("q06b_i8-L2-v4096-M16", synth.Q06B_I8.with_(n_layers=2, vocab=4096), [40 + 13 * b for b in range(16)]),
    ("q06b_q8-L2-v4096-M16", synth.Q06B_Q8.with_(n_layers=2, vocab=4096), [40 + 13 * b for b in range(16)]),
    ("q06b_q40-L2-v4096-M16", synth.Q06B_Q40.with_(n_layers=2, vocab=4096), [40 + 13 * b for b in range(16)]),
    ("q06b-kvi8-L2-v4096-M16", synth.Q06B.with_(n_layers=2, vocab=4096, kv_i8=True), [40 + 13 * b for b in range(16)]),
]


@pytest.mark.parametrize("name,cfg,lens", BATCH16_CASES, ids=[c[0] for c in BATCH16_CASES])
def test_batched_decode_many_rows_match_oracle(dpk, name, cfg, lens):
    """Every row of a batched decode step against the oracle, teacher-forced
    on each sequence's own greedy ids."""
    w = synth.make_weights(cfg, 0)
    N = 3
    B = len(lens)
    prompts = [synth.prompt_ids(cfg, L, 0, index=b) for b, L in enumerate(lens)]
    runs = [oracle_greedy(cfg, w, p, N)[1] for p in prompts]
    print("\n[parity] %s rows=%d" % (name, B), flush=True)
    dec = dpk.Decoder(cfg, w, max_batch=B, max_seq=(max(lens) + N + 63) // 64 * 64, max_rows=256)
    for b in range(B):
        dec.prefill(b, [int(t) for t in prompts[b]])
    lg = dec.logits_buffer(B)
    am = dec.argmax_buffer(B)
    worst = 0.0
    for s in range(N):
        toks = [runs[b]["ids"][s] for b in range(B)]
        if s == 0:
            dpk.profile_begin(dec.handle, 10000)
        dec.decode_step(list(range(B)), toks, [lens[b] + s for b in range(B)], am, lg)
        if s == 0:
            stats = dpk.profile_end(dec.handle)
            assert any(k.endswith("head") for k in stats), sorted(stats)
        ids = am.cpu().tolist()
        for b in range(B):
            worst = max(worst, compare_logits(lg[b].cpu(), runs[b]["logits"][s + 1], TOL[cfg.weight_format],
                                              "%s row %d step %d" % (name, b, s)))
            check_ids([ids[b]], [runs[b]["logits"][s + 1]], [runs[b]["ids"][s + 1]], "%s row %d" % (name, b))
    dpk.check_device_errors(dec.handle)
    print("[parity] %s worst max-abs %.3g" % (name, worst), flush=True)
    dec.close()
