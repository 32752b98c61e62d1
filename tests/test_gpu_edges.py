"""GPU edge cases through the C ABI: the degenerate and boundary inputs of the
prefill / decode / verify calls, each against the oracle, and the argument
checks that reject a call before anything is launched (the model stays
usable and its cursors unchanged after such a rejection)."""
import pytest
import torch

import oracle
import synth
from helpers import TOL, compare_logits

pytestmark = pytest.mark.gpu

CFG = synth.Q06B.with_(n_layers=2, vocab=4096)
MAX_SEQ = 64


@pytest.fixture(scope="module")
def dpk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_prefill_kv_amd as dpk
    return dpk


@pytest.fixture(scope="module")
def weights():
    return synth.make_weights(CFG, 0)


@pytest.fixture(scope="module")
def model(weights):
    return oracle.OracleModel(CFG, weights)


def status_of(dpk, call):
    with pytest.raises(dpk.DpkError) as e:
        call()
    return e.value.status


def test_one_token_prompt_boundary_ids_and_last_position(dpk, weights, model):
    """A one-token prompt; ids 0 and vocab - 1 fed as decode tokens; decoding
    up to the last position max_seq - 1; one step past it is rejected."""
    V = CFG.vocab
    dec = dpk.Decoder(CFG, weights, max_batch=1, max_seq=MAX_SEQ, max_rows=64)
    lg, am = dec.logits_buffer(1), dec.argmax_buffer(1)
    cache = model.new_cache(MAX_SEQ)
    dec.prefill(0, [V - 1], lg, am)
    compare_logits(lg[0].cpu(), model.forward_block(cache, [V - 1], 0)[0], TOL["bf16"], "1-token prefill")
    feed = [0, V - 1] + [int(t) for t in synth.prompt_ids(CFG, MAX_SEQ, 3)]
    worst = 0.0
    for pos in range(1, MAX_SEQ):
        tok = feed[pos - 1]
        dec.decode_step([0], [tok], [pos], am, lg)
        worst = max(worst, compare_logits(lg[0].cpu(), model.forward_step(cache, tok, pos), TOL["bf16"],
                                          "decode pos %d" % pos))
    assert dec.seq_length(0) == MAX_SEQ
    assert status_of(dpk, lambda: dec.decode_step([0], [1], [MAX_SEQ], am, lg)) == dpk.DPK_ERANGE
    # a verify block that would end past max_seq
    assert status_of(dpk, lambda: dec.verify(0, [1, 2, 3], MAX_SEQ - 2, am, lg)) == dpk.DPK_ERANGE
    assert dec.seq_length(0) == MAX_SEQ
    dpk.check_device_errors(dec.handle)
    print("\n[edges] positions 0..%d worst max-abs %.3g" % (MAX_SEQ - 1, worst), flush=True)
    dec.close()


def test_rejected_calls_leave_the_model_usable(dpk, weights, model):
    V = CFG.vocab
    dec = dpk.Decoder(CFG, weights, max_batch=2, max_seq=MAX_SEQ, max_rows=64)
    lg, am = dec.logits_buffer(2), dec.argmax_buffer(2)
    prompt = [int(t) for t in synth.prompt_ids(CFG, 10, 0)]
    dec.prefill(0, prompt, lg, am)
    dec.prefill(1, prompt[:4], lg, am)
    E, R = dpk.DPK_EINVAL, dpk.DPK_ERANGE
    rejected = [
        (lambda: dec.prefill(0, []), E),                                   # n < 1
        (lambda: dec.prefill(0, [1] * (MAX_SEQ + 1)), R),                  # beyond max_seq
        (lambda: dec.prefill(0, [1, V, 2]), R),                            # id outside the vocabulary
        (lambda: dec.prefill(2, [1, 2]), R),                               # slot >= max_batch
        (lambda: dec.decode_step([0], [1], [11], am, lg), R),              # pos beyond the cursor
        (lambda: dec.decode_step([0], [-1], [10], am, lg), R),             # negative id
        (lambda: dec.decode_step([0, 0], [1, 2], [10, 10], am, lg), E),    # a slot twice
        (lambda: dec.decode_step([5], [1], [0], am, lg), R),               # slot >= max_batch
        (lambda: dec.decode_step(list(range(17)), [1] * 17, [0] * 17, am, lg), E),  # batch > 16
        (lambda: dec.verify(0, [1] * 17, 10, am, lg), E),                  # k + 1 > 16
        (lambda: dec.verify(0, [], 10, am, lg), E),                        # k + 1 < 1
        (lambda: dec.verify(0, [1, 2], 11, am, lg), R),                    # pos beyond the cursor
        (lambda: dec.verify(0, [1, V], 10, am, lg), R),                    # draft outside the vocabulary
        (lambda: dec.verify(1, [1, -1], 4, am, lg), R),                    # negative draft
    ]
    for i, (call, want) in enumerate(rejected):
        assert status_of(dpk, call) == want, "case %d" % i
        assert dec.seq_length(0) == 10 and dec.seq_length(1) == 4, "case %d moved a cursor" % i
    # still usable: both slots continue exactly as the oracle does
    c0, c1 = model.new_cache(MAX_SEQ), model.new_cache(MAX_SEQ)
    model.forward_block(c0, prompt, 0)
    model.forward_block(c1, prompt[:4], 0)
    dec.decode_step([1, 0], [7, 9], [4, 10], am, lg)
    compare_logits(lg[0].cpu(), model.forward_step(c1, 7, 4), TOL["bf16"], "slot 1 after rejections")
    compare_logits(lg[1].cpu(), model.forward_step(c0, 9, 10), TOL["bf16"], "slot 0 after rejections")
    dpk.check_device_errors(dec.handle)
    dec.close()


def test_verify_without_drafts_is_a_decode_step(dpk, weights, model):
    """k_plus_1 = 1: no drafts, nothing to accept; the row's logits are the
    next-token logits and the cursor advances by one."""
    dec = dpk.Decoder(CFG, weights, max_batch=1, max_seq=MAX_SEQ, max_rows=64)
    lg, am = dec.logits_buffer(1), dec.argmax_buffer(1)
    prompt = [int(t) for t in synth.prompt_ids(CFG, 12, 1)]
    dec.prefill(0, prompt)
    cache = model.new_cache(MAX_SEQ)
    model.forward_block(cache, prompt, 0)
    acc = dec.verify(0, [17], 12, am, lg)
    assert acc == 0
    assert dec.seq_length(0) == 13
    ref = model.forward_step(cache, 17, 12)
    compare_logits(lg[0].cpu(), ref, TOL["bf16"], "verify k=0")
    assert int(am.cpu()[0]) == oracle.argmax_lowest(ref) or oracle.tie_exempt(ref)
    dpk.check_device_errors(dec.handle)
    dec.close()


def test_out_of_range_device_id_is_reported_and_read_as_zero(dpk, weights, model):
    """A device-side token id outside the vocabulary is replaced by 0 (the
    step's results are those of token 0) and reported once by the error
    check."""
    dec = dpk.Decoder(CFG, weights, max_batch=1, max_seq=MAX_SEQ, max_rows=64)
    lg, am = dec.logits_buffer(1), dec.argmax_buffer(1)
    prompt = [int(t) for t in synth.prompt_ids(CFG, 8, 2)]
    dec.prefill(0, prompt)
    cache = model.new_cache(MAX_SEQ)
    model.forward_block(cache, prompt, 0)
    bad = torch.tensor([CFG.vocab + 5], dtype=torch.int32, device="cuda")
    dec.decode_step([0], None, [8], am, lg, ids_dev=bad)
    assert status_of(dpk, lambda: dpk.check_device_errors(dec.handle)) == dpk.DPK_ERANGE
    dpk.check_device_errors(dec.handle)  # cleared
    compare_logits(lg[0].cpu(), model.forward_step(cache, 0, 8), TOL["bf16"], "id read as 0")
    dec.close()


def test_rollback_replays_a_step(dpk, weights):
    """Decoding again at an earlier position (rollback) with the same token
    gives that step's logits again: positions past the cursor are never
    read."""
    dec = dpk.Decoder(CFG, weights, max_batch=1, max_seq=MAX_SEQ, max_rows=64)
    lg, am = dec.logits_buffer(1), dec.argmax_buffer(1)
    prompt = [int(t) for t in synth.prompt_ids(CFG, 20, 4)]
    dec.prefill(0, prompt)
    dec.decode_step([0], [3], [20], am, lg)
    first = lg[0].clone()
    for s, tok in enumerate([11, 12, 13]):
        dec.decode_step([0], [tok], [21 + s], am, lg)
    assert dec.seq_length(0) == 24
    dec.decode_step([0], [3], [20], am, lg)
    assert dec.seq_length(0) == 21
    d = (lg[0] - first).abs().max().item()
    print("\n[edges] rollback replay max-abs %.3g" % d, flush=True)
    assert d <= 1e-5
    dpk.check_device_errors(dec.handle)
    dec.close()


def test_verify_at_the_maximum_block(dpk, weights, model):
    """k_plus_1 = 16 (the largest verify block): drafts are the oracle's own
    greedy continuation with one wrong token planted at draft 10, so exactly 9
    drafts are accepted (unless a step is a near tie); every row's logits
    against the oracle's block pass."""
    dec = dpk.Decoder(CFG, weights, max_batch=1, max_seq=MAX_SEQ, max_rows=64)
    lg, am = dec.logits_buffer(16), dec.argmax_buffer(16)
    prompt = [int(t) for t in synth.prompt_ids(CFG, 20, 5)]
    run = oracle.greedy_run(model, prompt, 16)
    g = run["ids"]
    ids_in = [g[0]] + [g[i] for i in range(1, 16)]
    ids_in[10] = (ids_in[10] + 1) % CFG.vocab  # draft 10 (index 10) is wrong
    dec.prefill(0, prompt)
    cache = model.new_cache(MAX_SEQ)
    model.forward_block(cache, prompt, 0)
    ref = oracle.verify(model, cache, ids_in, 20)
    acc = dec.verify(0, ids_in, 20, am, lg)
    for i in range(16):
        compare_logits(lg[i].cpu(), ref["logits"][i], TOL["bf16"], "verify-16 row %d" % i)
    assert acc == ref["accepted"]
    assert dec.seq_length(0) == 20 + acc + 1
    print("\n[edges] verify k+1=16 accepted %d" % acc, flush=True)
    dpk.check_device_errors(dec.handle)
    dec.close()


@pytest.mark.parametrize("name,cfg", [
    ("q8b-L2-v4096", synth.Q8B.with_(n_layers=2, vocab=4096)),      # 256-column persistent step
    ("q06b-L2-v4096", synth.Q06B.with_(n_layers=2, vocab=4096)),    # 128-column persistent step
])
def test_barrier_abort_is_reported_and_recovered(dpk, name, cfg):
    """A persistent step run with the abort word set (as after a barrier wait
    that gave up) passes every barrier at once and finishes; the error is
    reported, the counters are reset, and decoding again from the same
    position reproduces the undisturbed steps exactly.  The 600-token context
    spans three attention chunks, so the chunk-merge counters are exercised."""
    P, N = 600, 4
    w = synth.make_weights(cfg, 0)
    prompt = [int(t) for t in synth.prompt_ids(cfg, P, 0)]
    dec = dpk.Decoder(cfg, w, max_batch=1, max_seq=P + N, max_rows=256)
    lg, am = dec.logits_buffer(1), dec.argmax_buffer(1)
    feed = [int(t) for t in synth.prompt_ids(cfg, N, 0, index=5)]
    dec.prefill(0, prompt, lg, am)
    ref = []
    for s in range(N):
        dec.decode_step([0], [feed[s]], [P + s], am, lg)
        ref.append(lg[0].cpu().clone())
    dpk.check_device_errors(dec.handle)
    print("\n[abort] %s: forcing the abort word before a step at pos %d" % (name, P), flush=True)
    dpk.test_set_barrier_abort(dec.handle)
    dec.decode_step([0], [feed[0]], [P], am, lg)
    assert status_of(dpk, lambda: dpk.check_device_errors(dec.handle)) == dpk.DPK_EHIP
    assert "barrier" in dpk.last_error()
    dpk.check_device_errors(dec.handle)  # cleared
    for s in range(N):
        dec.decode_step([0], [feed[s]], [P + s], am, lg)
        assert torch.equal(lg[0].cpu(), ref[s]), "%s step %d after recovery" % (name, s)
    dpk.check_device_errors(dec.handle)
    dec.close()
