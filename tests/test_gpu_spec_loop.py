"""GPU test of the greedy speculative loop (dpk_spec_generate): a draft model
proposes, the target verifies, and the emitted tokens must be the target's
greedy continuation, checked against the CPU oracle's free-running greedy run
(up to the first near-tie step, after which either continuation is correct)
and against the GPU's own plain greedy decode.  After the loop the caches
must be consistent: one more decode step matches the oracle."""
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


TARGET = synth.Q8B.with_(n_layers=2, vocab=4096)
CASES = [
    # (name, target config, draft config or None for a self-draft, n_new, k_init, k_min, k_max)
    ("self-draft", TARGET, None, 40, 4, 2, 6),
    ("qwen06b-draft", TARGET, synth.Q06B.with_(n_layers=2, vocab=4096), 23, 4, 2, 6),
    ("q4-target-bf16-draft", synth.Q06B_Q4.with_(n_layers=2, vocab=4096), synth.Q06B.with_(n_layers=2, vocab=4096),
     30, 2, 1, 15),
]


@pytest.mark.parametrize("name,tcfg,dcfg,n_new,k0,kmin,kmax", CASES, ids=[c[0] for c in CASES])
def test_spec_generate_is_the_target_greedy_run(dpk, name, tcfg, dcfg, n_new, k0, kmin, kmax):
    P = 40
    max_seq = P + n_new + kmax + 2
    wt = synth.make_weights(tcfg, 0)
    wd = wt if dcfg is None else synth.make_weights(dcfg, 0)
    prompt = [int(t) for t in synth.prompt_ids(tcfg, P, 0)]
    om = oracle.OracleModel(tcfg, wt)
    run = oracle.greedy_run(om, prompt, n_new + 1)
    tgt = dpk.Decoder(tcfg, wt, max_batch=1, max_seq=max_seq, max_rows=64)
    drf = dpk.Decoder(dcfg or tcfg, wd, max_batch=1, max_seq=max_seq, max_rows=64)
    lg, am = tgt.logits_buffer(1), tgt.argmax_buffer(1)
    tgt.prefill(0, prompt, lg, am)
    drf.prefill(0, prompt)
    g0 = int(am.cpu()[0])
    assert g0 == run["ids"][0] or oracle.tie_exempt(run["logits"][0])
    ids, stats = dpk.spec_generate(tgt.handle, drf.handle, 0, P, g0, n_new, k0, kmin, kmax)
    dpk.check_device_errors(tgt.handle)
    dpk.check_device_errors(drf.handle)
    rate = stats["accepted"] / max(1, stats["drafted"])
    print("\n[spec-loop] %s: %s, acceptance %.2f" % (name, stats, rate), flush=True)
    # against the oracle's free-running greedy run, up to the first near-tie
    for s in range(n_new):
        if oracle.tie_exempt(run["logits"][s + 1]) or oracle.tie_exempt(run["logits"][s]):
            print("[spec-loop] %s: near-tie at step %d, compared %d tokens" % (name, s, s), flush=True)
            break
        assert ids[s] == run["ids"][s + 1], "%s: token %d: spec %d oracle %d" % (name, s, ids[s], run["ids"][s + 1])
    assert tgt.seq_length(0) == P + n_new and drf.seq_length(0) == P + n_new
    if dcfg is None:
        assert rate >= 0.9
    # against the GPU's own plain greedy decode of the same prompt
    plain = dpk.Decoder(tcfg, wt, max_batch=1, max_seq=max_seq, max_rows=64)
    plain.prefill(0, prompt, lg, am)
    tok = g0
    plain_ids = []
    for s in range(n_new):
        plain.decode_step([0], [tok], [P + s], am, lg)
        tok = int(am.cpu()[0])
        plain_ids.append(tok)
    n_same = next((s for s in range(n_new) if plain_ids[s] != ids[s]), n_new)
    if n_same < n_new:
        assert oracle.tie_exempt(run["logits"][n_same + 1]) or oracle.tie_exempt(run["logits"][n_same])
    plain.close()
    # the caches are consistent: one more step of both continues the oracle's run
    if n_same == n_new and ids == [int(t) for t in run["ids"][1:n_new + 1]]:
        tgt.decode_step([0], [ids[-1]], [P + n_new], am, lg)
        compare_logits(lg[0].cpu(), run["logits"][n_new + 1], TOL[tcfg.weight_format], "%s step after" % name)
        drf.decode_step([0], [ids[-1]], [P + n_new], am)
        dpk.check_device_errors(drf.handle)
    tgt.close()
    drf.close()


def test_spec_generate_rejects_bad_arguments(dpk):
    w = synth.make_weights(TARGET, 0)
    a = dpk.Decoder(TARGET, w, max_batch=1, max_seq=64, max_rows=32)
    b = dpk.Decoder(TARGET, w, max_batch=1, max_seq=64, max_rows=32)
    a.prefill(0, list(range(10)))
    b.prefill(0, list(range(10)))
    for kw, status in ((dict(k_init=1, k_min=2, k_max=6), dpk.DPK_EINVAL),
                       (dict(k_init=4, k_min=2, k_max=16), dpk.DPK_EINVAL),
                       (dict(pos=11), dpk.DPK_ERANGE),
                       (dict(n_new=60), dpk.DPK_ERANGE),
                       (dict(token=4096), dpk.DPK_ERANGE)):
        args = dict(pos=10, token=1, n_new=5, k_init=4, k_min=2, k_max=6)
        args.update(kw)
        with pytest.raises(dpk.DpkError) as e:
            dpk.spec_generate(a.handle, b.handle, 0, args["pos"], args["token"], args["n_new"], args["k_init"],
                              args["k_min"], args["k_max"])
        assert e.value.status == status, kw
    with pytest.raises(dpk.DpkError):
        dpk.spec_generate(a.handle, a.handle, 0, 10, 1, 5)
    assert a.seq_length(0) == 10 and b.seq_length(0) == 10
    a.close()
    b.close()
