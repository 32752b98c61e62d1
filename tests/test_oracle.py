"""Pins of the CPU oracle to facts other than itself (closed forms, library
routines, brute force on tiny inputs, structural invariants).  CPU only."""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from oracle.decoder import (apply_rope, argmax_lowest, dequant_q4, rms_norm, silu, softmax,
                            unpack_q4)

F64 = torch.float64


def small_cfg(**kw):
    base = dict(family="pin", n_layers=2, hidden=8, n_heads=4, n_kv_heads=2, head_dim=4,
                intermediate=12, vocab=16, weight_format="f32", qk_norm=True, tied=False,
                init_std=0.3, rope_theta=10000.0)
    base.update(kw)
    return synth.ModelConfig(**base)


# ---------------------------------------------------------------- generator
def test_splitmix64_published_vector(synth_built):
    # SplitMix64 seeded with 0: the first outputs are 0xE220A8397B1DCDAF,
    # 0x6E789E6AA1B965F4, 0x06C45D188009454F (reference sequence of the
    # published generator).
    assert synth.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert synth.splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert synth.splitmix64(0, 2) == 0x06C45D188009454F


def test_generator_statistics_and_determinism(synth_built):
    k = synth.key_of(0, "stat/test")
    a = synth.normal_f64(k, (200000,), 0.02)
    assert abs(a.mean()) < 3 * 0.02 / math.sqrt(len(a))
    assert abs(a.std() - 0.02) < 0.0003
    b = synth.normal_f64(k, (1000,), 0.02)
    np.testing.assert_array_equal(a[:1000], b)          # counter based: prefix-stable
    ids = synth.uniform_int(k, 100000, 151936)
    assert ids.min() >= 0 and ids.max() < 151936
    bf = synth.normal_bf16(k, (1000,), 0.02)
    np.testing.assert_array_equal(bf, synth.f32_to_bf16_bits(a[:1000].astype(np.float32)))


def test_generator_golden_checksum(synth_built):
    # Guards the input recipe against accidental change (values written by
    # this generator when the recipe was fixed).
    w = synth.make_weights(synth.TINY, 0, names=["layers.0.self_attn.q_proj"])
    q = w["layers.0.self_attn.q_proj"]
    assert q.shape == (256, 256)
    ids = synth.prompt_ids(synth.TINY, 16, 0)
    assert ids.tolist() == GOLDEN_TINY_PROMPT
    assert float(np.float64(q.astype(np.float64).sum())) == pytest.approx(GOLDEN_TINY_Q0_SUM, abs=1e-9)


GOLDEN_TINY_PROMPT = None  # filled below from tests/golden/generator.txt
GOLDEN_TINY_Q0_SUM = None


def _load_golden():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "generator.txt")
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    return [int(x) for x in vals["tiny_prompt"].split()], float(vals["tiny_q0_sum"])


GOLDEN_TINY_PROMPT, GOLDEN_TINY_Q0_SUM = _load_golden()


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_form_constant_vector():
    for c in (0.5, -3.0, 1e-4):
        x = torch.full((7,), c, dtype=F64)
        g = torch.linspace(0.5, 2.0, 7, dtype=F64)
        y = rms_norm(x, g, 1e-6)
        expect = g * c / math.sqrt(c * c + 1e-6)
        assert torch.allclose(y, expect, rtol=1e-14, atol=0)


def test_rmsnorm_scale_invariance_and_unit_rms():
    x = torch.randn(5, 64, dtype=F64, generator=torch.Generator().manual_seed(1))
    g = torch.ones(64, dtype=F64)
    y = rms_norm(x, g, 0.0)
    assert torch.allclose((y * y).mean(-1), torch.ones(5, dtype=F64), atol=1e-14)
    assert torch.allclose(rms_norm(37.0 * x, g, 0.0), y, atol=1e-13)


# ---------------------------------------------------------------- RoPE
def test_rope_identity_at_position_zero():
    x = torch.randn(3, 5, 128, dtype=F64, generator=torch.Generator().manual_seed(2))
    y = apply_rope(x, torch.zeros(3, dtype=torch.long), 1e6)
    assert torch.equal(x, y)


def test_rope_matches_complex_rotation():
    # (x_i, x_{i+d/2}) as the complex number x_i + j x_{i+d/2}, multiplied by
    # exp(j * pos * theta^(-2i/d)).
    d, theta = 16, 1e6
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 2, d))
    pos = np.array([0, 1, 17, 8191])
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    ang = pos[:, None] * theta ** (-2.0 * np.arange(d // 2) / d)
    zr = z * np.exp(1j * ang)[:, None, :]
    expect = np.concatenate([zr.real, zr.imag], axis=-1)
    got = apply_rope(torch.from_numpy(x), torch.from_numpy(pos), theta).numpy()
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-12)


def test_rope_hand_value():
    # d = 4, theta = 10000, pos = 1: inv_freq = [1, 0.01]
    x = torch.tensor([[[1.0, 2.0, 3.0, 4.0]]], dtype=F64)
    y = apply_rope(x, torch.tensor([1]), 10000.0)[0, 0]
    c0, s0, c1, s1 = math.cos(1), math.sin(1), math.cos(0.01), math.sin(0.01)
    expect = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    assert torch.allclose(y, torch.tensor(expect, dtype=F64), atol=1e-15)


def test_rope_norm_and_relative_position():
    g = torch.Generator().manual_seed(4)
    q = torch.randn(1, 1, 128, dtype=F64, generator=g)
    k = torch.randn(1, 1, 128, dtype=F64, generator=g)
    for m, n, s in [(3, 9, 100), (0, 50, 4000), (1000, 1, 7)]:
        a = (apply_rope(q, torch.tensor([m]), 1e6) * apply_rope(k, torch.tensor([n]), 1e6)).sum()
        b = (apply_rope(q, torch.tensor([m + s]), 1e6) * apply_rope(k, torch.tensor([n + s]), 1e6)).sum()
        assert abs(float(a - b)) < 1e-11
        assert abs(float(apply_rope(q, torch.tensor([m]), 1e6).norm() - q.norm())) < 1e-12


# ---------------------------------------------------------------- softmax / silu / argmax
def test_softmax_rows_and_library():
    s = torch.randn(6, 33, dtype=F64, generator=torch.Generator().manual_seed(5)) * 10
    p = softmax(s)
    assert torch.all(p >= 0)
    assert torch.allclose(p.sum(-1), torch.ones(6, dtype=F64), atol=1e-12)
    np.testing.assert_allclose(p.numpy(), scipy.special.softmax(s.numpy(), axis=-1), atol=1e-15)
    assert torch.allclose(softmax(s + 123.0), p, atol=1e-15)
    s2 = s.clone()
    s2[:, 5:] = float("-inf")
    assert torch.all(softmax(s2)[:, 5:] == 0)


def test_silu_properties():
    z = torch.linspace(-20, 20, 101, dtype=F64)
    assert float(silu(torch.zeros(1, dtype=F64))) == 0.0
    assert torch.allclose(silu(z) - silu(-z), z, atol=1e-14)
    np.testing.assert_allclose(silu(z).numpy(), z.numpy() * scipy.special.expit(z.numpy()),
                               atol=1e-15)


def test_argmax_lowest_index_on_ties():
    x = torch.tensor([1.0, 5.0, 2.0, 5.0, 5.0], dtype=F64)
    assert argmax_lowest(x) == 1
    assert oracle.tie_exempt(torch.tensor([3.0, 2.995, 1.0], dtype=F64))
    assert not oracle.tie_exempt(torch.tensor([3.0, 2.9, 1.0], dtype=F64))


# ---------------------------------------------------------------- 4-bit
def test_q4_pack_unpack_roundtrip(synth_built):
    codes = synth.q4_codes(synth.key_of(0, "q4/pin"), 5, 128)
    c = unpack_q4(codes)
    assert c.shape == (5, 128) and c.max() <= 15
    words = np.zeros((5, 16), dtype=np.uint32)
    for j in range(8):
        words |= c[:, j::8].astype(np.uint32) << np.uint32(4 * j)
    np.testing.assert_array_equal(words, codes)
    # every code value occurs (uniform codes)
    assert set(np.unique(c).tolist()) == set(range(16))


def test_q4_dequant_exact_and_requant(synth_built):
    cfg = synth.Q06B_Q4.with_(family="q4pin")
    w = synth._linear(cfg, 0, "t", (3, 192))
    codes, s, b = w["t.codes"], w["t.scales"], w["t.biases"]
    W = dequant_q4(codes, s, b).numpy()
    c = unpack_q4(codes)
    sf = synth.bf16_bits_to_f32(s).astype(np.float64)
    bf = synth.bf16_bits_to_f32(b).astype(np.float64)
    for n in range(3):
        for k in range(192):
            assert W[n, k] == c[n, k] * sf[n, k // 64] + bf[n, k // 64]
    rq = np.rint((W - np.repeat(bf, 64, 1)) / np.repeat(sf, 64, 1))
    np.testing.assert_array_equal(rq, c)
    # regrouped dot: s * sum(c x) + b * sum(x) per group (oxinfer, MLX checkpoints)
    x = np.random.default_rng(6).standard_normal(192)
    direct = W @ x
    regroup = np.zeros(3)
    for g in range(3):
        xs = x[64 * g:64 * g + 64]
        regroup += sf[:, g] * (c[:, 64 * g:64 * g + 64] @ xs) + bf[:, g] * xs.sum()
    np.testing.assert_allclose(regroup, direct, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- brute force tiny decoder
def brute_force_logits(cfg, w, toks):
    """Pure-Python scalar loops; explicit causal score rows."""
    H, d, Hq, Hkv = cfg.hidden, cfg.head_dim, cfg.n_heads, cfg.n_kv_heads
    G, eps = Hq // Hkv, cfg.rms_eps

    def mat(n):
        return np.asarray(w[n], dtype=np.float64).tolist()

    def matvec(Wm, x):
        return [sum(Wm[r][c] * x[c] for c in range(len(x))) for r in range(len(Wm))]

    def norm(x, g):
        ms = sum(v * v for v in x) / len(x)
        s = 1.0 / math.sqrt(ms + eps)
        return [x[i] * s * g[i] for i in range(len(x))]

    def rope(x, p):
        out = list(x)
        for i in range(d // 2):
            f = p * cfg.rope_theta ** (-2.0 * i / d)
            a, b = x[i], x[i + d // 2]
            out[i] = a * math.cos(f) - b * math.sin(f)
            out[i + d // 2] = b * math.cos(f) + a * math.sin(f)
        return out

    E = mat("embed_tokens")
    hs = [list(E[t]) for t in toks]
    for l in range(cfg.n_layers):
        p = "layers.%d." % l
        Wq, Wk, Wv, Wo = (mat(p + "self_attn.%s_proj" % n) for n in "qkvo")
        if cfg.qk_norm:
            qn, kn = mat(p + "self_attn.q_norm"), mat(p + "self_attn.k_norm")
            qnorm, knorm = (lambda x: norm(x, qn)), (lambda x: norm(x, kn))
        else:
            qnorm = knorm = (lambda x: x)
        ys = [norm(h, mat(p + "input_layernorm")) for h in hs]
        qs, ks, vs = [], [], []
        for i, y in enumerate(ys):
            q, k, v = matvec(Wq, y), matvec(Wk, y), matvec(Wv, y)
            qs.append([rope(qnorm(q[h * d:(h + 1) * d]), i) for h in range(Hq)])
            ks.append([rope(knorm(k[h * d:(h + 1) * d]), i) for h in range(Hkv)])
            vs.append([v[h * d:(h + 1) * d] for h in range(Hkv)])
        for i in range(len(hs)):
            o = []
            for h in range(Hq):
                g = h // G
                sc = [sum(qs[i][h][c] * ks[j][g][c] for c in range(d)) / math.sqrt(d)
                      for j in range(i + 1)]
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                Z = sum(e)
                o += [sum(e[j] / Z * vs[j][g][c] for j in range(i + 1)) for c in range(d)]
            att = matvec(Wo, o)
            hs[i] = [hs[i][c] + att[c] for c in range(H)]
            y = norm(hs[i], mat(p + "post_attention_layernorm"))
            gt, up = matvec(mat(p + "mlp.gate_proj"), y), matvec(mat(p + "mlp.up_proj"), y)
            a = [gt[c] / (1.0 + math.exp(-gt[c])) * up[c] for c in range(len(gt))]
            dn = matvec(mat(p + "mlp.down_proj"), a)
            hs[i] = [hs[i][c] + dn[c] for c in range(H)]
    head = mat("embed_tokens" if cfg.tied else "lm_head")
    return matvec(head, norm(hs[-1], mat("norm")))


@pytest.mark.parametrize("qk_norm", [True, False])
def test_oracle_matches_brute_force(synth_built, qk_norm):
    cfg = small_cfg(qk_norm=qk_norm, gain_std=0.2)
    w = synth.make_weights(cfg, 7)
    toks = [3, 1, 15, 0, 7]
    m = oracle.OracleModel(cfg, w)
    got = m.forward_block(m.new_cache(8), toks, 0)[0].numpy()
    expect = brute_force_logits(cfg, w, toks)
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-12)
    # the step path too, one token at a time
    c = m.new_cache(8)
    for i, t in enumerate(toks):
        step = m.forward_step(c, t, i)
    np.testing.assert_allclose(step.numpy(), expect, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- structural invariants
def tiny_model(cfg=None, seed=0):
    cfg = cfg or synth.TINY
    w = synth.make_weights(cfg, seed)
    return oracle.OracleModel(cfg, w), w


def test_prefill_equals_stepwise_decode(synth_built):
    m, _ = tiny_model()
    prompt = synth.prompt_ids(synth.TINY, 16, 0)
    block = m.forward_block(m.new_cache(16), prompt, 0)[0]
    c = m.new_cache(16)
    for i, t in enumerate(prompt):
        step = m.forward_step(c, int(t), i)
    assert float((block - step).abs().max()) < 1e-9


def test_prefill_equals_stepwise_decode_qwen_shape(synth_built):
    cfg = synth.Q06B.with_(family="pin06", n_layers=2, vocab=2048)
    m, _ = tiny_model(cfg)
    prompt = synth.prompt_ids(cfg, 24, 0)
    block = m.forward_block(m.new_cache(24), prompt, 0)[0]
    c = m.new_cache(24)
    for i, t in enumerate(prompt):
        step = m.forward_step(c, int(t), i)
    assert float((block - step).abs().max()) < 1e-9


def test_attention_over_one_key_returns_v(synth_built):
    # With a single cached key the softmax weight is exactly 1, so the
    # attention output is V whatever q is: changing W_q must not change the
    # logits of a one-token prompt, while it does change a two-token prompt.
    cfg = small_cfg(family="onekey")
    w = synth.make_weights(cfg, 1)
    w2 = dict(w)
    for l in range(cfg.n_layers):
        w2["layers.%d.self_attn.q_proj" % l] = w["layers.%d.self_attn.q_proj" % l] * -3.0 + 0.1
    a = oracle.OracleModel(cfg, w).forward_block(oracle.KVCache(cfg, 2, F64), [5], 0)
    b = oracle.OracleModel(cfg, w2).forward_block(oracle.KVCache(cfg, 2, F64), [5], 0)
    assert torch.equal(a, b)
    a2 = oracle.OracleModel(cfg, w).forward_block(oracle.KVCache(cfg, 2, F64), [5, 9], 0)
    b2 = oracle.OracleModel(cfg, w2).forward_block(oracle.KVCache(cfg, 2, F64), [5, 9], 0)
    assert float((a2 - b2).abs().max()) > 1e-6


def test_gqa_equals_mha_with_duplicated_kv_heads(synth_built):
    cfg = small_cfg(family="gqa", n_heads=4, n_kv_heads=2, head_dim=4)
    w = synth.make_weights(cfg, 2)
    mha = cfg.with_(n_kv_heads=4)
    w2 = dict(w)
    d = cfg.head_dim
    for l in range(cfg.n_layers):
        for n in ("k_proj", "v_proj"):
            W = w["layers.%d.self_attn.%s" % (l, n)]
            # MHA kv head j copies GQA kv head j // G (contiguous groups)
            w2["layers.%d.self_attn.%s" % (l, n)] = np.concatenate(
                [W[(j // cfg.group) * d:(j // cfg.group + 1) * d] for j in range(4)])
    toks = [1, 2, 3, 4, 5, 6]
    a = oracle.OracleModel(cfg, w).forward_block(oracle.KVCache(cfg, 6, F64), toks, 0)
    b = oracle.OracleModel(mha, w2).forward_block(oracle.KVCache(mha, 6, F64), toks, 0)
    assert float((a - b).abs().max()) < 1e-13


def test_zero_projection_layers_are_identity(synth_built):
    cfg = small_cfg(family="ident")
    w = synth.make_weights(cfg, 3)
    for l in range(cfg.n_layers):
        w["layers.%d.self_attn.o_proj" % l] = np.zeros_like(w["layers.%d.self_attn.o_proj" % l])
        w["layers.%d.mlp.down_proj" % l] = np.zeros_like(w["layers.%d.mlp.down_proj" % l])
    toks = [4, 8, 15]
    got = oracle.OracleModel(cfg, w).forward_block(oracle.KVCache(cfg, 3, F64), toks, 0)[0]
    # zero-layer model by hand: W_head . RMSNorm(E[last id])
    e = w["embed_tokens"][15].astype(np.float64)
    g = w["norm"].astype(np.float64)
    y = e / np.sqrt(np.mean(e * e) + cfg.rms_eps) * g
    expect = w["lm_head"].astype(np.float64) @ y
    np.testing.assert_allclose(got.numpy(), expect, rtol=0, atol=1e-13)


def test_tied_head_equals_untied_copy(synth_built):
    cfg = small_cfg(family="tie", tied=True)
    w = synth.make_weights(cfg, 4)
    untied = cfg.with_(tied=False)
    w2 = dict(w)
    w2["lm_head"] = w["embed_tokens"].copy()
    toks = [2, 9, 11]
    a = oracle.OracleModel(cfg, w).forward_block(oracle.KVCache(cfg, 3, F64), toks, 0)
    b = oracle.OracleModel(untied, w2).forward_block(oracle.KVCache(untied, 3, F64), toks, 0)
    assert torch.equal(a, b)


def test_block_is_causal(synth_built):
    m, _ = tiny_model()
    toks = [int(t) for t in synth.prompt_ids(synth.TINY, 8, 1)]
    a = m.forward_block(m.new_cache(8), toks, 0, all_rows=True)
    toks2 = list(toks)
    toks2[6] = (toks2[6] + 1) % synth.TINY.vocab
    b = m.forward_block(m.new_cache(8), toks2, 0, all_rows=True)
    assert torch.equal(a[:6], b[:6])
    assert not torch.equal(a[6], b[6])


def test_verify_equals_greedy_and_accept_rule(synth_built):
    m, _ = tiny_model()
    prompt = synth.prompt_ids(synth.TINY, 16, 0)
    run = oracle.greedy_run(m, prompt, 8)
    g = run["ids"]
    K = 5
    c = m.new_cache(32)
    m.forward_block(c, prompt, 0)
    res = oracle.verify(m, c, [g[0]] + g[1:K + 1], 16)
    for i in range(K + 1):
        assert float((res["logits"][i] - run["logits"][i + 1]).abs().max()) < 1e-9
    assert res["accepted"] == K and res["bonus"] == g[K + 1]
    assert c.length == 16 + K + 1
    # a corrupted third draft: accept 2, bonus is the greedy token there
    c = m.new_cache(32)
    m.forward_block(c, prompt, 0)
    drafts = list(g[1:K + 1])
    drafts[2] = (drafts[2] + 1) % synth.TINY.vocab
    res = oracle.verify(m, c, [g[0]] + drafts, 16)
    assert res["accepted"] == 2 and res["bonus"] == g[3] and c.length == 16 + 3
    # rollback then decode continues exactly as greedy
    lg = m.forward_step(c, g[3], 16 + 3)
    assert float((lg - run["logits"][4]).abs().max()) < 1e-9


def test_q4_model_embedding_and_tied_head(synth_built):
    cfg = synth.Q06B_Q4.with_(family="q4tie", n_layers=1, vocab=256, hidden=128, n_heads=2,
                              n_kv_heads=1, head_dim=64, intermediate=192)
    w = synth.make_weights(cfg, 5)
    m = oracle.OracleModel(cfg, w)
    full = dequant_q4(w["embed_tokens.codes"], w["embed_tokens.scales"], w["embed_tokens.biases"])
    assert torch.equal(m.embed_rows([7, 200])[1], full[200])
    assert torch.equal(m.W("embed_tokens"), full)
    logits = m.forward_block(m.new_cache(4), [7, 200, 3], 0)
    assert logits.shape == (1, 256)


def test_fp32_path_agrees_with_fp64(synth_built):
    cfg = synth.Q06B.with_(family="fp32pin", n_layers=2, vocab=4096)
    w = synth.make_weights(cfg, 0)
    prompt = synth.prompt_ids(cfg, 64, 0)
    a = oracle.OracleModel(cfg, w, torch.float64)
    b = oracle.OracleModel(cfg, w, torch.float32)
    la = a.forward_block(a.new_cache(64), prompt, 0)[0]
    lb = b.forward_block(b.new_cache(64), prompt, 0)[0].double()
    assert float((la - lb).abs().max()) < 2e-3


# ---------------------------------------------------------------------------
# The float32 path at depth.  The 8B-shaped fixtures are written by the
# oracle's float32 path (the float64 definition is too slow for their sizes),
# so that path is pinned against float64 where the error could grow: the full
# 28-layer 0.6B-shaped run, a 4-layer 8B-shaped model, and the full 36-layer
# 8B-shaped prefill and first decode steps.  Bound: 2e-3 max-abs, ten times
# inside the GPU tolerance.
# ---------------------------------------------------------------------------
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FP32_BOUND = 2e-3


def _fp32_gap_report(name, gaps):
    print("\n[fp32 vs fp64] %s: %s" % (name, ", ".join("%s %.3g" % kv for kv in gaps.items())))


def test_fp32_path_full_qwen06b_against_stored_fp64(synth_built):
    """28 layers, 512-token prefill and decode steps 0 and 1 (teacher-forced on
    the stored greedy ids) against the float64 fixture's whole logit rows."""
    with np.load(os.path.join(GOLDEN, "q06b.npz")) as z:
        g = {k: z[k] for k in z.files}
    cfg = synth.Q06B
    P = int(g["prompt_len"])
    w = synth.make_weights(cfg, 0)
    m = oracle.OracleModel(cfg, w, torch.float32)
    cache = m.new_cache(P + 2)
    gaps = {"prefill": float(np.abs(m.forward_block(cache, synth.prompt_ids(cfg, P, 0), 0)[0].double().numpy()
                                    - g["prefill_logits"].astype(np.float64)).max())}
    full_rows = [int(r) for r in g["full_rows"]]
    for s in range(2):
        lg = m.forward_step(cache, int(g["id"][s]), P + s).double().numpy()
        gaps["step %d" % s] = float(np.abs(lg - g["full_logits"][full_rows.index(s + 1)]).max())
    _fp32_gap_report("q06b full", gaps)
    assert max(gaps.values()) < FP32_BOUND, gaps


def test_fp32_path_4layer_qwen8b_against_fp64(synth_built):
    """The 8B shape (hidden 4096, 32/8 heads, MLP 12288, vocab 151936) with 4
    layers: 256-token prefill and two decode steps, float32 against float64."""
    cfg = synth.Q8B.with_(n_layers=4)
    w = synth.make_weights(cfg, 0)
    prompt = synth.prompt_ids(cfg, 256, 0)
    runs = {}
    for dt in (torch.float64, torch.float32):
        m = oracle.OracleModel(cfg, w, dt, cache_weights=False)
        cache = m.new_cache(258)
        rows = [m.forward_block(cache, prompt, 0)[0].double()]
        toks = runs[torch.float64][1] if dt == torch.float32 else None
        fed = []
        for s in range(2):
            t = toks[s] if toks else oracle.argmax_lowest(rows[-1])
            fed.append(t)
            rows.append(m.forward_step(cache, t, 256 + s).double())
        runs[dt] = (rows, fed)
    gaps = {k: float((a - b).abs().max()) for k, a, b in
            zip(("prefill", "step 0", "step 1"), runs[torch.float64][0], runs[torch.float32][0])}
    _fp32_gap_report("q8b 4 layers", gaps)
    assert max(gaps.values()) < FP32_BOUND, gaps


def test_fp32_fixture_full_qwen8b_against_fp64_fixture():
    """The 36-layer 8B-shaped fixture (float32 path: prefill of 2048 ids and
    decode steps 0 and 1) against the float64 re-run of the same records."""
    with np.load(os.path.join(GOLDEN, "q8b.npz")) as z:
        g = {k: z[k] for k in z.files}
    with np.load(os.path.join(GOLDEN, "q8b_f64.npz")) as z:
        h = {k: z[k] for k in z.files}
    assert list(h["fed_ids"]) == [int(x) for x in g["id"][:2]]
    full_rows = [int(r) for r in g["full_rows"]]
    refs = [g["prefill_logits"], g["full_logits"][full_rows.index(1)], g["full_logits"][full_rows.index(2)]]
    gaps = {k: float(np.abs(a.astype(np.float64) - b).max())
            for k, a, b in zip(("prefill", "step 0", "step 1"), refs, h["logits"])}
    _fp32_gap_report("q8b full (fixtures)", gaps)
    assert max(gaps.values()) < FP32_BOUND, gaps


# ---------------------------------------------------------------- int8 weights
def test_i8_dequant_hand_values_and_requant(synth_built):
    from oracle.decoder import dequant_i8
    q = np.array([[3, -5, 127], [0, -127, 1]], dtype=np.int8)
    sc = synth.f32_to_bf16_bits(np.array([[0.5], [0.015625]], dtype=np.float32))
    W = dequant_i8(q, sc)
    assert W.tolist() == [[1.5, -2.5, 63.5], [0.0, -1.984375, 0.015625]]
    cfg = synth.Q06B.with_(family="i8pin", weight_format="i8", n_layers=1, vocab=512)
    w = synth.make_weights(cfg, 3)
    for name in ("layers.0.mlp.down_proj", "embed_tokens"):
        q, sc = w[name + ".q"], w[name + ".scales"]
        s = torch.from_numpy(synth.bf16_bits_to_f32(sc)).double()
        Wd = dequant_i8(q, sc)
        assert torch.equal(torch.round(Wd / s).to(torch.int64), torch.from_numpy(q.astype(np.int64)))
        assert int(np.abs(q.astype(np.int32)).max(axis=1).min()) >= 126  # per-row absmax scaling
        # within half a step of the N(0, std) draw it was quantised from
        ref = synth.normal_f32(synth.key_of(3, cfg.family + "/" + name), q.shape, cfg.init_std)
        assert float((Wd - torch.from_numpy(ref).double()).abs().div(s).max()) <= 0.5 + 1e-3


def test_q8_dequant_hand_values_blocks_and_requant(synth_built):
    """Each run of 32 weights along a row takes its own float32 scale: column
    k uses scale[n, k // 32] (a scale indexed k % 32, or per row, fails)."""
    from oracle.decoder import dequant_q8
    q = np.zeros((2, 64), dtype=np.int8)
    q[0, 0], q[0, 31], q[0, 32], q[0, 63] = 3, -5, 127, 1
    q[1, 1], q[1, 33] = -127, 2
    sc = np.array([[0.5, 0.25], [0.1, 3.0]], dtype=np.float32)
    W = dequant_q8(q, sc)
    assert W[0, 0] == 1.5 and W[0, 31] == -2.5 and W[0, 32] == 31.75 and W[0, 63] == 0.25
    assert W[1, 1] == -127 * float(np.float32(0.1)) and W[1, 33] == 6.0
    assert int((W != 0).sum()) == 6
    cfg = synth.Q06B.with_(family="q8pin", weight_format="q8", n_layers=1, vocab=512)
    w = synth.make_weights(cfg, 3)
    for name in ("layers.0.mlp.down_proj", "embed_tokens"):
        q, sc = w[name + ".q"], w[name + ".scales"]
        assert sc.dtype == np.float32 and sc.shape == (q.shape[0], q.shape[1] // 32)
        s = torch.repeat_interleave(torch.from_numpy(sc).double(), 32, dim=1)
        Wd = dequant_q8(q, sc)
        assert torch.equal(torch.round(Wd / s).to(torch.int64), torch.from_numpy(q.astype(np.int64)))
        # per-block absmax scaling: every block holds a code of magnitude 127
        assert int(np.abs(q.astype(np.int32)).reshape(q.shape[0], -1, 32).max(axis=2).min()) == 127
        # within half a step of the N(0, std) draw it was quantised from
        ref = synth.normal_f32(synth.key_of(3, cfg.family + "/" + name), q.shape, cfg.init_std)
        assert float((Wd - torch.from_numpy(ref).double()).abs().div(s).max()) <= 0.5 + 1e-3


def test_q8_model_equals_f64_weight_model_with_the_dequantized_weights(synth_built):
    """The block-scaled model must equal a plain-format model that holds the
    products scale * q in float64 (exact: 24-bit scale times 8-bit code)."""
    from oracle.decoder import dequant_q8
    cfg = synth.Q06B.with_(family="q8pin2", weight_format="q8", n_layers=2, vocab=512, hidden=256, n_heads=4,
                           n_kv_heads=2, intermediate=512)
    w = synth.make_weights(cfg, 1)
    f = {}
    for k, v in w.items():
        if k.endswith(".q"):
            f[k[:-2]] = dequant_q8(v, w[k[:-2] + ".scales"]).numpy()
        elif not k.endswith(".scales"):
            f[k] = synth.bf16_bits_to_f32(v)
    cf = cfg.with_(weight_format="f32")
    prompt = synth.prompt_ids(cfg, 12, 0)
    ma = oracle.OracleModel(cfg, w)
    a = ma.forward_block(ma.new_cache(12), prompt, 0)
    mb = oracle.OracleModel(cf, f)
    b = mb.forward_block(mb.new_cache(12), prompt, 0)
    assert float((a - b).abs().max()) == 0.0


def test_q40_dequant_hand_values_nibble_order_and_requant(synth_built):
    """Byte j of a block holds code j (low nibble) and code j + 16 (high
    nibble); w = d * (c - 8) with the block's fp16 d (a swapped nibble order,
    a missing -8 or a scale indexed by column fails)."""
    from oracle.decoder import dequant_q40
    packed = np.full((1, 32), 0x88, dtype=np.uint8)  # two blocks, every code 8 -> w = 0
    packed[0, 0] = 0x3F   # block 0: element 0 code 15, element 16 code 3
    packed[0, 15] = 0x08  # element 15 code 8, element 31 code 0
    packed[0, 16] = 0xA1  # block 1: element 32 code 1, element 48 code 10
    d = np.array([[0.5, 0.25]], dtype=np.float16)
    W = dequant_q40(packed, d)
    assert W[0, 0] == 3.5 and W[0, 16] == -2.5 and W[0, 15] == 0.0 and W[0, 31] == -4.0
    assert W[0, 32] == -1.75 and W[0, 48] == 0.5
    assert int((W != 0).sum()) == 5
    cfg = synth.Q06B.with_(family="q40pin", weight_format="q4_0", n_layers=1, vocab=512)
    w = synth.make_weights(cfg, 3)
    for name in ("layers.0.mlp.down_proj", "embed_tokens"):
        q, d = w[name + ".q"], w[name + ".scales"]
        assert q.dtype == np.uint8 and d.dtype == np.float16 and d.shape == (q.shape[0], q.shape[1] // 16)
        s = torch.repeat_interleave(torch.from_numpy(d.astype(np.float64)), 32, dim=1)
        Wd = dequant_q40(q, d)
        ref = synth.normal_f32(synth.key_of(3, cfg.family + "/" + name), Wd.shape, cfg.init_std)
        # requantisation returns the codes, and each weight is within half a
        # step of its draw (a block's largest magnitude maps to code 1 or 15)
        b = q.reshape(q.shape[0], -1, 16).astype(np.int64)
        codes = np.concatenate([b & 0xF, b >> 4], axis=2).reshape(Wd.shape)
        assert torch.equal(torch.round(Wd / s).to(torch.int64) + 8, torch.from_numpy(codes))
        assert float((Wd - torch.from_numpy(ref).double()).abs().div(s).max()) <= 0.5 + 1e-3
        assert set(np.unique(np.abs(codes.reshape(codes.shape[0], -1, 32) - 8).max(axis=2))) <= {7, 8}


def test_q40_model_equals_f64_weight_model_with_the_dequantized_weights(synth_built):
    from oracle.decoder import dequant_q40
    cfg = synth.Q06B.with_(family="q40pin2", weight_format="q4_0", n_layers=2, vocab=512, hidden=256, n_heads=4,
                           n_kv_heads=2, intermediate=512)
    w = synth.make_weights(cfg, 1)
    f = {}
    for k, v in w.items():
        if k.endswith(".q"):
            f[k[:-2]] = dequant_q40(v, w[k[:-2] + ".scales"]).numpy()
        elif not k.endswith(".scales"):
            f[k] = synth.bf16_bits_to_f32(v)
    cf = cfg.with_(weight_format="f32")
    prompt = synth.prompt_ids(cfg, 12, 0)
    ma = oracle.OracleModel(cfg, w)
    a = ma.forward_block(ma.new_cache(12), prompt, 0)
    mb = oracle.OracleModel(cf, f)
    b = mb.forward_block(mb.new_cache(12), prompt, 0)
    assert float((a - b).abs().max()) == 0.0


def test_kv_i8_quantization_hand_values_and_properties():
    """int8 KV cache: per head vector s = fp32(max|x| / 127), q = round(x / s)
    half to even, clipped to +-127; read back s * q."""
    from oracle.decoder import quantize_kv
    x = torch.tensor([[1.0, -0.5, 0.25, 0.0], [0.0, 0.0, 0.0, 0.0], [-2.0, 1.0, 0.0, 0.0]], dtype=torch.float64)
    y = quantize_kv(x)
    s0 = float(np.float32(1.0 / 127.0))
    assert y[0].tolist() == [127 * s0, -64 * s0, 32 * s0, 0.0]  # -63.5 and 31.75 round to -64 and 32
    assert y[1].tolist() == [0.0] * 4
    s2 = float(np.float32(2.0 / 127.0))
    assert y[2].tolist() == [-127 * s2, 64 * s2, 0.0, 0.0]  # 63.5 rounds half to even: 64
    g = torch.Generator().manual_seed(5)
    x = torch.randn(3, 7, 128, generator=g, dtype=torch.float64) * torch.rand(3, 7, 1, generator=g, dtype=torch.float64)
    y = quantize_kv(x)
    s = (x.abs().amax(-1, keepdim=True) / 127).float().double()
    assert float(((x - y).abs() / s).max()) <= 0.5 + 1e-6          # within half a step
    assert torch.equal(y.abs().amax(-1, keepdim=True), 127 * s)     # the largest maps to +-127
    assert torch.equal(quantize_kv(y), y)                           # idempotent
    assert torch.equal(quantize_kv(4 * x), 4 * y)                   # power-of-two scale invariance


def test_kv_i8_cache_holds_the_quantized_vectors_per_position_and_head(synth_built):
    """Layer 0's keys and values do not depend on the cache, so the int8
    cache must hold exactly the quantized float cache, vector by vector; the
    logits move by a bounded amount."""
    from oracle.decoder import quantize_kv
    cfg = synth.Q06B.with_(family="kvq", n_layers=2, vocab=512, hidden=256, n_heads=4, n_kv_heads=2, intermediate=512)
    w = synth.make_weights(cfg, 2)
    prompt = synth.prompt_ids(cfg, 20, 0)
    mf, mq = oracle.OracleModel(cfg, w), oracle.OracleModel(cfg.with_(kv_i8=True), w)
    cf, cq = mf.new_cache(24), mq.new_cache(24)
    lf, lq = mf.forward_block(cf, prompt, 0), mq.forward_block(cq, prompt, 0)
    sf, sq = mf.forward_step(cf, 7, 20), mq.forward_step(cq, 7, 20)
    for a, b in ((cf.k[0], cq.k[0]), (cf.v[0], cq.v[0])):
        assert torch.equal(quantize_kv(a[:, :21, :]), b[:, :21, :])
        assert not torch.equal(a[:, :21, :], b[:, :21, :])
    assert 0 < float((lf - lq).abs().max()) < 0.05 and 0 < float((sf - sq).abs().max()) < 0.05


def test_i8_model_equals_f32_model_with_the_dequantized_weights(synth_built):
    """scale (bf16, 8 significant bits) times q (int8) is exact in fp32, so
    the int8 model must equal an fp32-format model holding those products."""
    from oracle.decoder import dequant_i8
    cfg = synth.Q06B.with_(family="i8pin2", weight_format="i8", n_layers=2, vocab=512, hidden=256, n_heads=4,
                           n_kv_heads=2, intermediate=512)
    w = synth.make_weights(cfg, 1)
    f = {}
    for k, v in w.items():
        if k.endswith(".q"):
            f[k[:-2]] = dequant_i8(v, w[k[:-2] + ".scales"], torch.float32).numpy()
        elif not k.endswith(".scales"):
            f[k] = synth.bf16_bits_to_f32(v)
    cf = cfg.with_(weight_format="f32")
    prompt = synth.prompt_ids(cfg, 12, 0)
    a = oracle.OracleModel(cfg, w).forward_block(oracle.OracleModel(cfg, w).new_cache(12), prompt, 0)
    mb = oracle.OracleModel(cf, f)
    b = mb.forward_block(mb.new_cache(12), prompt, 0)
    assert float((a - b).abs().max()) == 0.0
