"""GPU parity of prefill onto an existing cache (dpk_prefill_at) against the
CPU oracle's block path at the same offsets.

A prompt is fed in pieces: each piece's rows attend causally within the piece
and to every cached position before it, and the last row's logits are
compared with the oracle's forward_block over the same piece at the same
start.  Pieces longer than max_rows are chunked inside the library, so some
pieces cross a chunk boundary at an offset; pieces of at most 16 rows take
the weight-streaming path.  A piece may also start before the cursor (the
positions after its start are dropped, as a rollback)."""
import pytest
import torch

import oracle
import synth
from helpers import TOL, compare_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dpk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_prefill_kv_amd as dpk
    return dpk


# (name, config, pieces as (start, length), decode steps after, Decoder kwargs)
CASES = [
    ("q06b-L2-gemm", synth.Q06B.with_(n_layers=2), [(0, 37), (37, 150), (187, 5), (192, 70)], 4,
     dict(max_rows=64)),
    ("q06b-L2-rollback", synth.Q06B.with_(n_layers=2), [(0, 100), (60, 90), (150, 3), (120, 40)], 3,
     dict(max_rows=64)),
    ("q06b_q4-L2", synth.Q06B_Q4.with_(n_layers=2), [(0, 20), (20, 131), (151, 9)], 4, dict(max_rows=64)),
    ("q8b-L2-v4096", synth.Q8B.with_(n_layers=2, vocab=4096), [(0, 300), (300, 257), (557, 16)], 4,
     dict(max_rows=256)),
    ("tiny", synth.TINY, [(0, 7), (7, 12), (19, 1), (20, 9)], 4, {}),
    # a piece long enough for the QKV epilogue path, at an odd offset
    ("q8b-L1-v4096-qkv-epilogue", synth.Q8B.with_(n_layers=1, vocab=4096), [(0, 37), (37, 1400), (1437, 3)], 2,
     dict(max_rows=1400)),
]


@pytest.mark.parametrize("name,cfg,pieces,N,kw", CASES, ids=[c[0] for c in CASES])
def test_prefill_at_matches_oracle(dpk, name, cfg, pieces, N, kw):
    print("\n[prefill_at] %s pieces=%s" % (name, pieces), flush=True)
    w = synth.make_weights(cfg, 0)
    total = max(s + n for s, n in pieces)
    max_seq = total + N
    ids = synth.prompt_ids(cfg, 2 * max_seq, 0, index=3)
    m = oracle.OracleModel(cfg, w)
    cache = m.new_cache(max_seq)
    dec = dpk.Decoder(cfg, w, max_batch=2, max_seq=max_seq, **kw)
    lg = dec.logits_buffer(1)
    am = dec.argmax_buffer(1)
    tol = TOL[cfg.weight_format]
    worst = 0.0
    k = 0
    for start, n in pieces:
        piece = [int(t) for t in ids[k:k + n]]
        k += n
        ref = m.forward_block(cache, piece, start)[0]
        # slot 1: the piece API at every offset, including start 0
        dec.prefill_at(1, start, piece, lg, am)
        worst = max(worst, compare_logits(lg[0].cpu(), ref, tol, "%s piece at %d" % (name, start)))
        assert dec.seq_length(1) == start + n
        g = int(am.cpu()[0])
        assert g == oracle.argmax_lowest(ref) or oracle.tie_exempt(ref), "%s argmax at %d" % (name, start)
    # greedy decode after the last piece, teacher-forced on the oracle
    pos = cache.length
    tok = oracle.argmax_lowest(ref)
    for s in range(N):
        ref = m.forward_step(cache, tok, pos + s)
        dec.decode_step([1], [tok], [pos + s], am, lg)
        worst = max(worst, compare_logits(lg[0].cpu(), ref, tol, "%s decode %d" % (name, s)))
        tok = oracle.argmax_lowest(ref)
    dpk.check_device_errors(dec.handle)
    print("[prefill_at] %s worst max-abs %.3g" % (name, worst), flush=True)
    dec.close()


def test_prefill_at_rejects_bad_offsets(dpk):
    cfg = synth.Q06B.with_(n_layers=1, vocab=4096)
    w = synth.make_weights(cfg, 0)
    dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=64, max_rows=32)
    dec.prefill(0, list(range(10)))
    for start, n in ((11, 4), (-1, 4), (10, 55), (0, 65)):
        with pytest.raises(dpk.DpkError) as e:
            dec.prefill_at(0, start, list(range(n)))
        assert e.value.status == dpk.DPK_ERANGE, (start, n)
        assert dec.seq_length(0) == 10  # unchanged
    dec.prefill_at(0, 10, list(range(54)))
    assert dec.seq_length(0) == 64
    dec.close()
