"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and validates configurations and call order before touching
the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "dpk.h")).read()
    return sorted(set(re.findall(r"\b(dpk_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def dpk():
    import decoder_prefill_kv_amd as dpk
    return dpk


def test_library_exports_every_header_symbol(dpk):
    dpk.lib()
    lib = ctypes.CDLL(dpk.library_path())
    names = header_functions()
    assert "dpk_prefill" in names and "dpk_verify" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dpk.SYMBOLS)


def cfg_ok(dpk, **kw):
    c = dict(n_layers=2, hidden=1024, n_heads=16, n_kv_heads=8, head_dim=128, intermediate=3072,
             vocab=151936, rms_eps=1e-6, rope_theta=1e6, qk_norm=1, tied_embedding=1,
             weight_format=dpk.FMT_BF16, max_batch=2, max_seq=640, max_rows=64, flags=0)
    c.update(kw)
    return dpk.Config(**c)


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(n_kv_heads=3), dict(hidden=1000),
                                 dict(max_rows=8), dict(weight_format=7), dict(weight_format=6), dict(vocab=0),
                                 dict(n_heads=32, n_kv_heads=2), dict(vocab=151937)])
def test_create_rejects_bad_config(dpk, bad):
    with pytest.raises(dpk.DpkError) as e:
        dpk.create(cfg_ok(dpk, **bad))
    assert e.value.status == dpk.DPK_EINVAL
    assert dpk.last_error()


def test_workspace_sizes_and_call_order(dpk):
    h = dpk.create(cfg_ok(dpk))
    try:
        kv, sc, pr = dpk.workspace_size(h)
        # 2 slots x 2 layers x {K,V} x 8 heads x 640 x 128 x fp16
        assert kv == 2 * 2 * 2 * 8 * 640 * 128 * 2
        per_layer = (4096 * 1024 + 1024 * 2048 + 2 * 3072 * 1024 + 1024 * 3072) * 2
        # fp16 prefill operands + fragment-order bf16 decode copy, plus the tiled head
        assert sc > 0 and pr == 2 * (2 * per_layer) + 151936 * 1024 * 2
        for call in (lambda: dpk.prefill(h, 0, [1, 2, 3], stream=0),
                     lambda: dpk.decode_step(h, [0], [1], [0], None, stream=0),
                     lambda: dpk.verify(h, 0, [1, 2], 0, None, stream=0)):
            with pytest.raises(dpk.DpkError) as e:
                call()
            assert e.value.status in (dpk.DPK_ESTATE, dpk.DPK_EINVAL)
        with pytest.raises(dpk.DpkError) as e:
            dpk.prefill(h, 0, [1, 2, 3], stream=0)
        assert e.value.status == dpk.DPK_ESTATE and "not bound" in dpk.last_error()
        with pytest.raises(dpk.DpkError) as e:
            dpk.load_weights(h, [], stream=0)
        assert e.value.status == dpk.DPK_ESTATE
    finally:
        dpk.destroy(h)


@pytest.mark.parametrize("fmt", ["FMT_I8", "FMT_Q8", "FMT_Q40"])
def test_int8_code_formats_prep_holds_fp16_operands_and_fragment_order_codes(dpk, fmt):
    """The prep buffer of an int8-code model holds the fp16 prefill operands
    (2 bytes per weight) and a fragment-order copy of the codes (1 byte per
    weight, the tied head included; q8 also its block scales); per-row i8
    scales are read where the caller keeps them."""
    h = dpk.create(cfg_ok(dpk, weight_format=getattr(dpk, fmt)))
    try:
        kv, sc, pr = dpk.workspace_size(h)
        per_layer = 4096 * 1024 + 1024 * 2048 + 2 * 3072 * 1024 + 1024 * 3072  # weights
        # q8 / q4_0: and a fragment-order copy of the block scales (4 / 2 bytes per 32 weights);
        # q4_0 codes take half a byte
        per_w = {"FMT_I8": 1, "FMT_Q8": 1 + 4 / 32, "FMT_Q40": 0.5 + 2 / 32}[fmt]
        assert pr == 2 * (per_layer * 2 + per_layer * per_w) + 151936 * 1024 * per_w
        assert kv == 2 * 2 * 2 * 8 * 640 * 128 * 2
    finally:
        dpk.destroy(h)


@pytest.mark.parametrize("fmt,lo", [("FMT_BF16", False), ("FMT_I8", False), ("FMT_Q8", True), ("FMT_Q40", True),
                                    ("FMT_Q4G64", True)])
def test_int8_kv_cache_adds_kv_residuals_for_block_formats(dpk, fmt, lo):
    """Over an int8 KV cache the prep buffer of a block-scaled model (MLX
    4-bit, Q8, Q4_0) also holds the fp16 rounding residuals of the K and V
    projections (2 bytes per weight of those rows); exact fp16 copies (bf16,
    int8 codes) need none."""
    sizes = []
    for flags in (0, dpk.FLAG_KV_I8):
        h = dpk.create(cfg_ok(dpk, weight_format=getattr(dpk, fmt), flags=flags))
        try:
            sizes.append(dpk.workspace_size(h)[2])
        finally:
            dpk.destroy(h)
    kv_rows = 2 * 8 * 128  # K and V rows of a layer (8 KV heads of 128)
    assert sizes[1] - sizes[0] == (2 * kv_rows * 1024 * 2 if lo else 0)


def test_int8_kv_cache_sizes_and_format_check(dpk):
    """int8 KV cache: one byte per cached element, then (at a 256-byte
    boundary) one fp32 scale per position of every slab; refused for fp32
    weights."""
    h = dpk.create(cfg_ok(dpk, flags=dpk.FLAG_KV_I8))
    try:
        kv, sc, pr = dpk.workspace_size(h)
        codes = 2 * 2 * 2 * 8 * 640 * 128
        assert kv == (codes + 255) // 256 * 256 + 2 * 2 * 2 * 8 * 640 * 4
    finally:
        dpk.destroy(h)
    with pytest.raises(dpk.DpkError) as e:
        dpk.create(cfg_ok(dpk, weight_format=dpk.FMT_F32, head_dim=64, n_heads=4, n_kv_heads=2, hidden=256,
                          intermediate=768, vocab=4096, qk_norm=0, flags=dpk.FLAG_KV_I8))
    assert e.value.status == dpk.DPK_EINVAL


def test_fp32_format_needs_no_prep(dpk):
    h = dpk.create(cfg_ok(dpk, weight_format=dpk.FMT_F32, head_dim=64, n_heads=4, n_kv_heads=2, hidden=256,
                          intermediate=768, vocab=4096, qk_norm=0, tied_embedding=0))
    try:
        kv, sc, pr = dpk.workspace_size(h)
        assert pr == 0 and kv == 2 * 2 * 2 * 2 * 640 * 64 * 4  # 640 is a multiple of 64
    finally:
        dpk.destroy(h)
