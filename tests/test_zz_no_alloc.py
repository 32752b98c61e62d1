"""GPU test of dpk_spec_accept_noalloc (speculative-sampling acceptance with
the library's built-in workspace) against dpk_spec_accept (caller-provided
workspace) through the C ABI: identical accepted counts and tokens on two
calls in a row, the second with fewer drafts and a smaller vocabulary, and a
clear rejection of more drafts than the built-in workspace holds."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dpk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_prefill_kv_amd as dpk
    return dpk


def _case(tag, K, V):
    key = lambda s: synth.key_of(0, "noalloc/%s/%s" % (tag, s))
    tl = synth.normal_f32(key("t"), (K + 1, V), 1.3)
    dl = (0.7 * tl[:K] + 0.3 * synth.normal_f32(key("d"), (K, V), 1.3)).astype(np.float32)
    drafts = synth.uniform_int(key("ids"), K, V)
    drafts[0] = int(np.argmax(dl[0]))  # a likely draft
    r = synth.uniform_f64(key("r"), K).astype(np.float32)
    u = synth.uniform_f64(key("u"), K + 1).astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dev(tl), dev(dl), dev(drafts.astype(np.int32)), dev(r), dev(u)


@pytest.mark.parametrize("T,top_k,top_p", [(0.9, 0, 1.0), (0.8, 40, 0.9), (0.0, 0, 1.0)])
def test_noalloc_matches_workspace_entry_point(dpk, T, top_k, top_p):
    print("\n[noalloc] T=%g top_k=%d top_p=%g" % (T, top_k, top_p), flush=True)
    for call, (K, V) in enumerate(((7, 151936), (3, 4096))):  # the second call is smaller
        args = _case("%g-%d-%g-%d" % (T, top_k, top_p, call), K, V)
        ws = torch.empty(dpk.spec_accept_workspace_size(K), dtype=torch.uint8, device="cuda")
        want = torch.full((2,), -1, dtype=torch.int32, device="cuda")
        got = torch.full((2,), -1, dtype=torch.int32, device="cuda")
        dpk.spec_accept(*args, want, ws, T, top_k, top_p)
        dpk.spec_accept_noalloc(*args, got, T, top_k, top_p)
        torch.cuda.synchronize()
        print("[noalloc] call %d K=%d V=%d: %s vs %s" % (call, K, V, got.tolist(), want.tolist()), flush=True)
        assert got.tolist() == want.tolist()
        assert 0 <= got[0].item() <= K and 0 <= got[1].item() < V


def test_noalloc_rejects_more_drafts_than_it_holds(dpk):
    args = _case("big", 17, 64)
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(dpk.DpkError) as e:
        dpk.spec_accept_noalloc(*args, out, 1.0)
    assert e.value.status == dpk.DPK_EINVAL and "16" in dpk.last_error()
