"""GPU parity of sampling (dpk_sample) and speculative-sampling acceptance
(dpk_spec_accept) against the CPU oracle (oracle/sampling.py), through the
C ABI.

The sampled token is an integer decided by floating point: the GPU computes
z and the weights in fp32 (weights summed in exact fixed point), the oracle
in fp64.  So a token must equal the oracle's unless the oracle's uniform lies
within EPS of a boundary of its cumulative distribution (and no oracle mass
lies between the two tokens), or the oracle's own kept set is decided by a
margin below EPS (a top-p cut or a top-k tie); such rows are counted and
reported.  Acceptance decisions follow the same rule for r against p / q.
Distribution checks use a stratified grid of uniforms, where each token's
count must equal N * p to within one."""
import numpy as np
import pytest
import torch

import oracle
from oracle import sampling as S
import synth

pytestmark = pytest.mark.gpu
EPS = 2e-5


@pytest.fixture(scope="module")
def dpk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_prefill_kv_amd as dpk
    return dpk


def uniforms(tag, n):
    return synth.uniform_f64(synth.key_of(0, "sampling-test/" + tag), n)


def logit_rows(tag, rows, V, scale=1.3):
    return synth.normal_f32(synth.key_of(0, "sampling-test/logits/" + tag), (rows, V), scale)


def margins_ok(x64, T, top_k, top_p):
    """False when the oracle's kept set is decided by a margin below EPS."""
    if T == 0.0:
        top2 = torch.topk(x64, 2).values
        return bool(top2[0] - top2[1] > EPS)
    z = x64 / T
    if 0 < top_k < z.numel():
        sv = torch.sort(z, descending=True).values
        if float(sv[top_k - 1] - sv[top_k]) < EPS * max(1.0, float(sv[top_k - 1].abs())):
            return False
    if top_p < 1.0:
        p = S.sampling_probs(x64, T, top_k, 1.0)
        run = torch.cumsum(torch.sort(p, descending=True).values, 0)
        if float((run - top_p).abs().min()) < EPS:
            return False
    return True


def allowed_mismatch(probs, u, i, j):
    c = torch.cumsum(probs, 0).numpy()
    lo, hi = min(i, j), max(i, j)
    between = c[hi - 1] - c[lo]
    return between < EPS and abs(u - c[lo]) < 2 * EPS


PARAMS = [(0.0, 0, 1.0), (1.0, 0, 1.0), (0.7, 50, 1.0), (0.8, 0, 0.9), (1.3, 200, 0.6), (0.5, 1, 1.0),
          (0.25, 0, 0.5), (1.0, 5000, 0.95)]


@pytest.mark.parametrize("V", [151936, 4096, 37])
@pytest.mark.parametrize("T,top_k,top_p", PARAMS)
def test_sample_matches_oracle(dpk, V, T, top_k, top_p):
    rows = 24 if V > 10000 else 64
    x = logit_rows("%d" % V, rows, V)
    u = uniforms("u/%d/%g/%d/%g" % (V, T, top_k, top_p), rows)
    xd = torch.from_numpy(x).cuda()
    ud = torch.from_numpy(u.astype(np.float32)).cuda()
    out = torch.empty(rows, dtype=torch.int32, device="cuda")
    dpk.sample(xd, ud, out, T, top_k, top_p)
    got = out.cpu().tolist()
    same, near, skipped = 0, 0, 0
    for r in range(rows):
        x64 = torch.from_numpy(x[r]).to(torch.float64)
        uf = float(np.float32(u[r]))
        probs = S.sampling_probs(x64, T, top_k, top_p)
        want = S.draw(probs, uf)
        assert 0 <= got[r] < V
        if got[r] == want:
            same += 1
            continue
        if not margins_ok(x64, T, top_k, top_p):
            skipped += 1
            continue
        assert probs[got[r]] > 0, "row %d: GPU token %d outside the kept set" % (r, got[r])
        assert allowed_mismatch(probs, uf, want, got[r]), "row %d: GPU %d oracle %d (u %.9f)" % (r, got[r], want, uf)
        near += 1
    print("[sample] V=%d T=%g k=%d p=%g: %d equal, %d at a boundary, %d margin-skipped"
          % (V, T, top_k, top_p, same, near, skipped), flush=True)
    assert same >= rows - 2


@pytest.mark.parametrize("V,T,top_k,top_p", [(4096, 1.0, 0, 1.0), (4096, 0.6, 0, 0.8), (151936, 0.25, 0, 0.9),
                                             (151936, 0.9, 40, 1.0)])
def test_sample_stratified_counts(dpk, V, T, top_k, top_p):
    """N copies of one row with uniforms (j + 1/2) / N: each token's count is
    N times its oracle probability to within one."""
    N = 4096
    x = logit_rows("strat%d" % V, 1, V)
    xd = torch.from_numpy(x).cuda().expand(N, V).contiguous()
    ud = ((torch.arange(N, dtype=torch.float64) + 0.5) / N).to(torch.float32).cuda()
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    dpk.sample(xd, ud, out, T, top_k, top_p)
    counts = np.bincount(out.cpu().numpy(), minlength=V)
    p = S.sampling_probs(torch.from_numpy(x[0]).to(torch.float64), T, top_k, top_p).numpy()
    dev = np.abs(counts - N * p)
    print("[sample] stratified V=%d T=%g k=%d p=%g: kept %d, max |count - Np| %.3f"
          % (V, T, top_k, top_p, int((p > 0).sum()), dev.max()), flush=True)
    assert counts[p == 0].sum() == 0
    assert dev.max() <= 1.0 + 1e-3


def _spec_case(tag, K, V, T, top_k, top_p, draft_from_q=True):
    tl = logit_rows("spec-t/" + tag, K + 1, V)
    dl = logit_rows("spec-d/" + tag, K, V)
    # make the draft close to the target so that some drafts are accepted
    dl = (0.7 * tl[:K] + 0.3 * dl).astype(np.float32)
    ur = uniforms("spec-r/" + tag, K).astype(np.float32)
    uu = uniforms("spec-u/" + tag, K + 1).astype(np.float32)
    ud = uniforms("spec-d/" + tag, K)
    drafts = []
    for i in range(K):
        q = S.sampling_probs(torch.from_numpy(dl[i]).double(), T, top_k, top_p)
        drafts.append(S.draw(q, float(ud[i])) if draft_from_q else int(ud[i] * V))
    return tl, dl, drafts, ur, uu


@pytest.mark.parametrize("V", [4096, 151936])
@pytest.mark.parametrize("T,top_k,top_p", [(0.0, 0, 1.0), (1.0, 0, 1.0), (0.8, 30, 1.0), (0.9, 0, 0.85)])
def test_spec_accept_matches_oracle(dpk, V, T, top_k, top_p):
    K = 5
    trials = 40 if V < 10000 else 12
    ws = torch.empty(dpk.spec_accept_workspace_size(K), dtype=torch.uint8, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    hist = {}
    same = near = 0
    for t in range(trials):
        tag = "%d/%g/%d/%g/%d" % (V, T, top_k, top_p, t)
        tl, dl, drafts, ur, uu = _spec_case(tag, K, V, T, top_k, top_p, draft_from_q=(t % 4 != 3))
        dpk.spec_accept(torch.from_numpy(tl).cuda(), torch.from_numpy(dl).cuda(),
                        torch.tensor(drafts, dtype=torch.int32, device="cuda"), torch.from_numpy(ur).cuda(),
                        torch.from_numpy(uu).cuda(), out, ws, T, top_k, top_p)
        m, tok = out.cpu().tolist()
        ref = S.spec_accept(torch.from_numpy(tl).double(), torch.from_numpy(dl).double(), drafts,
                            [float(v) for v in ur], [float(v) for v in uu], T, top_k, top_p)
        hist[m] = hist.get(m, 0) + 1
        if (m, tok) == (ref["accepted"], ref["token"]):
            same += 1
            continue
        # a decision within EPS of the oracle's: r against p / q at the first
        # differing draft, or the final draw at a CDF boundary
        i = min(m, ref["accepted"])
        ok = False
        if i < K:
            p = S.sampling_probs(torch.from_numpy(tl[i]).double(), T, top_k, top_p)
            q = S.sampling_probs(torch.from_numpy(dl[i]).double(), T, top_k, top_p)
            d = drafts[i]
            ok = q[d] > 0 and abs(float(ur[i]) - float(p[d] / q[d])) < EPS
        if not ok and m == ref["accepted"]:
            rows = [torch.from_numpy(tl[m]).double()]
            dist = (S.residual(S.sampling_probs(rows[0], T, top_k, top_p),
                               S.sampling_probs(torch.from_numpy(dl[m]).double(), T, top_k, top_p))
                    if m < K else S.sampling_probs(rows[0], T, top_k, top_p))
            ok = allowed_mismatch(dist, float(uu[m]), ref["token"], tok)
        assert ok, "trial %d: GPU (%d, %d) oracle (%d, %d)" % (t, m, tok, ref["accepted"], ref["token"])
        near += 1
    print("[spec] V=%d T=%g k=%d p=%g: %d equal, %d at a boundary; accepted-count histogram %s"
          % (V, T, top_k, top_p, same, near, dict(sorted(hist.items()))), flush=True)
    assert same >= trials - 1


def test_spec_accept_greedy_is_the_verify_rule(dpk):
    """Temperature 0: accept while the draft equals the target row's argmax;
    the next token is the argmax of the first rejected row (or the bonus)."""
    K, V = 6, 4096
    ws = torch.empty(dpk.spec_accept_workspace_size(K), dtype=torch.uint8, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    for t in range(30):
        tl = logit_rows("greedy-t/%d" % t, K + 1, V)
        dl = logit_rows("greedy-d/%d" % t, K, V)
        greedy = [oracle.argmax_lowest(torch.from_numpy(tl[i])) for i in range(K + 1)]
        coin = uniforms("greedy-c/%d" % t, K)
        drafts = [greedy[i] if coin[i] < 0.7 else (greedy[i] + 1) % V for i in range(K)]
        r = torch.rand(K, device="cuda")
        u = torch.rand(K + 1, device="cuda")
        dpk.spec_accept(torch.from_numpy(tl).cuda(), torch.from_numpy(dl).cuda(),
                        torch.tensor(drafts, dtype=torch.int32, device="cuda"), r, u, out, ws, 0.0)
        m, tok = out.cpu().tolist()
        want = oracle.accept_length([0] + drafts, greedy)
        assert (m, tok) == (want, greedy[want]), "trial %d" % t


def test_spec_accept_first_token_follows_the_target(dpk):
    """Monte Carlo through the GPU rule (K = 1, V = 8): the first emitted
    token's frequencies against the target row's distribution (chi-square)."""
    V, T, n = 8, 0.9, 3000
    tl = logit_rows("mc-t", 2, V)
    dl = logit_rows("mc-d", 1, V)
    q = S.sampling_probs(torch.from_numpy(dl[0]).double(), T)
    ds = uniforms("mc-draft", n)
    rs = uniforms("mc-r", n).astype(np.float32)
    us = uniforms("mc-u", 2 * n).astype(np.float32)
    ws = torch.empty(dpk.spec_accept_workspace_size(1), dtype=torch.uint8, device="cuda")
    out = torch.empty(2 * n, dtype=torch.int32, device="cuda")
    tld, dld = torch.from_numpy(tl).cuda(), torch.from_numpy(dl).cuda()
    drafts = torch.tensor([S.draw(q, float(v)) for v in ds], dtype=torch.int32, device="cuda")
    rd, ud = torch.from_numpy(rs).cuda(), torch.from_numpy(us).cuda()
    for j in range(n):
        dpk.spec_accept(tld, dld, drafts[j:j + 1], rd[j:j + 1], ud[2 * j:2 * j + 2], out[2 * j:2 * j + 2], ws, T)
    res = out.view(n, 2).cpu().numpy()
    dr = drafts.cpu().numpy()
    first = np.where(res[:, 0] >= 1, dr, res[:, 1])
    counts = np.bincount(first, minlength=V)
    p = S.sampling_probs(torch.from_numpy(tl[0]).double(), T).numpy()
    chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
    print("[spec] first-token chi-square %.2f (7 dof), acceptance %.3f" % (chi2, float((res[:, 0] >= 1).mean())))
    assert chi2 < 24.3  # 7 degrees of freedom, p = 0.001


def test_sampling_rejects_bad_arguments(dpk):
    x = torch.zeros(2, 16, device="cuda")
    u = torch.zeros(2, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    for T, k, p in ((-1.0, 0, 1.0), (float("inf"), 0, 1.0), (1.0, -1, 1.0), (1.0, 0, 0.0), (1.0, 0, 1.5)):
        with pytest.raises(dpk.DpkError) as e:
            dpk.sample(x, u, out, T, k, p)
        assert e.value.status == dpk.DPK_EINVAL
    with pytest.raises(dpk.DpkError):
        dpk.spec_accept_workspace_size(0)
