"""Seeded synthetic inputs for the dense decoder workloads.

This module is the only code the CPU oracle and the GPU library share.  It
holds no decoder arithmetic: it describes model shapes and writes weights,
prompts and uniform draws into host numpy arrays from a counter-based
generator (``gen.c``: SplitMix64 + Box-Muller, bf16 by round-to-nearest-even).

Weight tensors use the ``[out, in]`` row-major layout of a transformers-style
checkpoint.  Storage formats:

* ``f32``  - numpy float32.
* ``bf16`` - numpy uint16 holding bfloat16 bit patterns.
* ``q4``   - MLX-style 4-bit affine, group 64 along the input dimension
  (oxinfer docs page, "MLX checkpoints": eight codes per uint32, one bf16
  scale and bias per 64 weights, w = scale * code + bias).  A tensor ``name``
  becomes three arrays: ``name.codes`` uint32 ``[out, in/8]`` (element 8w+j in
  bits 4j..4j+3 of word w), ``name.scales`` and ``name.biases`` uint16 (bf16)
  ``[out, in/64]``.
* ``i8``   - int8 with one scale per output row (symmetric per-channel
  quantisation of the N(0, std) weights: scale = bf16(max |w| / 127),
  q = round(w / scale) clipped to [-127, 127]).  A tensor ``name`` becomes
  ``name.q`` int8 ``[out, in]`` and ``name.scales`` uint16 (bf16) ``[out, 1]``.
* ``q8``   - int8 in blocks of 32 along the input dimension with one float32
  scale per block (oxinfer docs page, "Build and run", the q8 quantization
  flag; its pre-quantized files store the same blocks as int8 codes plus
  float32 scales): scale = max |w| / 127 over the block (float32),
  q = round(w / scale) clipped to [-127, 127].  A tensor ``name`` becomes
  ``name.q`` int8 ``[out, in]`` and ``name.scales`` float32 ``[out, in/32]``.
* ``q4_0`` - GGUF-style 4-bit blocks of 32 along the input dimension with one
  fp16 scale d each (oxinfer docs page, "Build and run", the q4 quantization
  flag; its pre-quantized files hold two codes per byte plus fp16 scales):
  w = d * (c - 8), c in 0..15; d = fp16(max |w| / 7) over the block,
  c = clip(round(w / d), -8, 7) + 8.  Within a block's 16 bytes, byte j holds
  element j in its low nibble and element j + 16 in its high nibble.  A tensor
  ``name`` becomes ``name.q`` uint8 ``[out, in/2]`` and ``name.scales``
  float16 ``[out, in/32]``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_synth.so")
_lib = None


def build() -> str:
    """Compile gen.c into _synth.so (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    vp = ctypes.c_void_p
    lib.synth_fnv1a64.restype = u64
    lib.synth_fnv1a64.argtypes = [ctypes.c_char_p]
    lib.synth_splitmix64.restype = u64
    lib.synth_splitmix64.argtypes = [u64, u64]
    lib.synth_normal_bf16.argtypes = [u64, i64, dbl, ctypes.c_int, vp]
    lib.synth_normal_f32.argtypes = [u64, i64, dbl, vp]
    lib.synth_normal_f64.argtypes = [u64, i64, dbl, vp]
    lib.synth_uniform_int.argtypes = [u64, i64, i32, vp]
    lib.synth_uniform_f64.argtypes = [u64, i64, vp]
    lib.synth_q4_codes.argtypes = [u64, i64, vp]
    for f in ("synth_normal_bf16", "synth_normal_f32", "synth_normal_f64", "synth_uniform_int",
              "synth_uniform_f64", "synth_q4_codes"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def key_of(seed: int, tag: str) -> int:
    """Stream key: seed XOR FNV-1a-64 of the tag."""
    return (int(seed) ^ int(_load().synth_fnv1a64(tag.encode()))) & 0xFFFFFFFFFFFFFFFF


def splitmix64(key: int, ctr: int) -> int:
    return int(_load().synth_splitmix64(key, ctr))


def normal_bf16(key: int, shape, std: float, absval: bool = False) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    _load().synth_normal_bf16(key, out.size, std, int(absval), out.ctypes.data)
    return out


def normal_f32(key: int, shape, std: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(key, out.size, std, out.ctypes.data)
    return out


def normal_f64(key: int, shape, std: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.float64)
    _load().synth_normal_f64(key, out.size, std, out.ctypes.data)
    return out


def uniform_int(key: int, n: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_int(key, n, hi, out.ctypes.data)
    return out


def uniform_f64(key: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(key, n, out.ctypes.data)
    return out


def q4_codes(key: int, rows: int, cols: int) -> np.ndarray:
    assert cols % 8 == 0
    out = np.empty((rows, cols // 8), dtype=np.uint32)
    _load().synth_q4_codes(key, rows * cols, out.ctypes.data)
    return out


BF16_ONE = 0x3F80


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """Shape and format of a dense pre-norm decoder (Llama / Qwen3 style)."""

    family: str            # weight-stream namespace; truncated models share it
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    weight_format: str     # "f32" | "bf16" | "q4" | "i8" | "q8" | "q4_0"
    qk_norm: bool
    tied: bool
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    init_std: float = 0.02
    q4_scale_std: float = 0.003
    gain_std: float = 0.0  # 0 -> every norm gain is exactly 1.0
    kv_i8: bool = False    # KV cache held as int8 codes, one scale per position and KV head

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    def with_(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)

    def linear_shapes(self) -> Dict[str, tuple]:
        H, I = self.hidden, self.intermediate
        shapes = {}
        for i in range(self.n_layers):
            p = "layers.%d." % i
            shapes[p + "self_attn.q_proj"] = (self.q_dim, H)
            shapes[p + "self_attn.k_proj"] = (self.kv_dim, H)
            shapes[p + "self_attn.v_proj"] = (self.kv_dim, H)
            shapes[p + "self_attn.o_proj"] = (H, self.q_dim)
            shapes[p + "mlp.gate_proj"] = (I, H)
            shapes[p + "mlp.up_proj"] = (I, H)
            shapes[p + "mlp.down_proj"] = (H, I)
        return shapes

    def gain_shapes(self) -> Dict[str, tuple]:
        shapes = {"norm": (self.hidden,)}
        for i in range(self.n_layers):
            p = "layers.%d." % i
            shapes[p + "input_layernorm"] = (self.hidden,)
            shapes[p + "post_attention_layernorm"] = (self.hidden,)
            if self.qk_norm:
                shapes[p + "self_attn.q_norm"] = (self.head_dim,)
                shapes[p + "self_attn.k_norm"] = (self.head_dim,)
        return shapes

    def n_linear_params(self) -> int:
        return sum(a * b for a, b in self.linear_shapes().values())


# The five workload shapes.  Unstated values (eps, theta, gains) follow the
# plainest reading: 1e-6, 1e6 and 1.0 everywhere.
TINY = ModelConfig("tiny", 2, 256, 4, 2, 64, 768, 4096, "f32", qk_norm=False, tied=False)
Q06B = ModelConfig("q06b", 28, 1024, 16, 8, 128, 3072, 151936, "bf16", qk_norm=True, tied=True)
Q06B_Q4 = ModelConfig("q06b_q4", 28, 1024, 16, 8, 128, 3072, 151936, "q4", qk_norm=True, tied=True)
Q8B = ModelConfig("q8b", 36, 4096, 32, 8, 128, 12288, 151936, "bf16", qk_norm=True, tied=False)

# int8 per-channel variants of the same shapes (other weight formats on the
# same decode path)
Q06B_I8 = Q06B.with_(family="q06b_i8", weight_format="i8")
Q8B_I8 = Q8B.with_(family="q8b_i8", weight_format="i8")
# Q8 block variants (32 weights per float32 scale)
Q06B_Q8 = Q06B.with_(family="q06b_q8", weight_format="q8")
Q8B_Q8 = Q8B.with_(family="q8b_q8", weight_format="q8")
# GGUF-style Q4_0 variants (32 weights per fp16 scale, codes 0..15 around 8)
Q06B_Q40 = Q06B.with_(family="q06b_q40", weight_format="q4_0")
Q8B_Q40 = Q8B.with_(family="q8b_q40", weight_format="q4_0")

CONFIGS = {"tiny": TINY, "q06b": Q06B, "q06b_q4": Q06B_Q4, "q8b": Q8B, "q06b_i8": Q06B_I8, "q8b_i8": Q8B_I8,
           "q06b_q8": Q06B_Q8, "q8b_q8": Q8B_Q8, "q06b_q40": Q06B_Q40, "q8b_q40": Q8B_Q40}


def _gain(cfg: ModelConfig, seed: int, name: str, shape) -> np.ndarray:
    if cfg.gain_std == 0.0:
        g64 = np.ones(shape, dtype=np.float64)
    else:
        g64 = 1.0 + normal_f64(key_of(seed, cfg.family + "/" + name), shape, cfg.gain_std)
    if cfg.weight_format == "f32":
        return g64.astype(np.float32)
    return f32_to_bf16_bits(g64.astype(np.float32))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even) and return the bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _linear(cfg: ModelConfig, seed: int, name: str, shape) -> Dict[str, np.ndarray]:
    tag = cfg.family + "/" + name
    rows, cols = shape
    if cfg.weight_format == "f32":
        return {name: normal_f32(key_of(seed, tag), shape, cfg.init_std)}
    if cfg.weight_format == "bf16":
        return {name: normal_bf16(key_of(seed, tag), shape, cfg.init_std)}
    if cfg.weight_format == "i8":
        w = normal_f32(key_of(seed, tag), shape, cfg.init_std)
        sc = f32_to_bf16_bits((np.abs(w).max(axis=1, keepdims=True) / 127.0).astype(np.float32))
        q = np.clip(np.rint(w / bf16_bits_to_f32(sc)), -127, 127).astype(np.int8)
        return {name + ".q": q, name + ".scales": sc}
    if cfg.weight_format == "q8":
        assert cols % 32 == 0
        w = normal_f32(key_of(seed, tag), shape, cfg.init_std).reshape(rows, cols // 32, 32)
        sc = (np.abs(w).max(axis=2) / np.float32(127.0)).astype(np.float32)
        q = np.clip(np.rint(w / np.where(sc > 0, sc, np.float32(1.0))[..., None]), -127, 127)
        return {name + ".q": q.astype(np.int8).reshape(rows, cols), name + ".scales": sc}
    if cfg.weight_format == "q4_0":
        assert cols % 32 == 0
        w = normal_f32(key_of(seed, tag), shape, cfg.init_std).reshape(rows, cols // 32, 32)
        d = (np.abs(w).max(axis=2) / np.float32(7.0)).astype(np.float16)
        d32 = d.astype(np.float32)
        c = np.clip(np.rint(w / np.where(d32 > 0, d32, np.float32(1.0))[..., None]), -8, 7).astype(np.int32) + 8
        packed = (c[..., :16] | (c[..., 16:] << 4)).astype(np.uint8)  # byte j: elements j and j + 16
        return {name + ".q": packed.reshape(rows, cols // 2), name + ".scales": d}
    if cfg.weight_format == "q4":
        assert cols % 64 == 0
        return {
            name + ".codes": q4_codes(key_of(seed, tag + ".codes"), rows, cols),
            name + ".scales": normal_bf16(key_of(seed, tag + ".scales"), (rows, cols // 64),
                                          cfg.q4_scale_std, absval=True),
            name + ".biases": normal_bf16(key_of(seed, tag + ".biases"), (rows, cols // 64),
                                          cfg.init_std),
        }
    raise ValueError(cfg.weight_format)


def make_weights(cfg: ModelConfig, seed: int = 0, names: Optional[List[str]] = None
                 ) -> Dict[str, np.ndarray]:
    """All host weight arrays of a model (or only the listed logical tensors)."""
    out: Dict[str, np.ndarray] = {}
    want = None if names is None else set(names)
    V, H = cfg.vocab, cfg.hidden
    if want is None or "embed_tokens" in want:
        out.update(_linear(cfg, seed, "embed_tokens", (V, H)))
    if not cfg.tied and (want is None or "lm_head" in want):
        out.update(_linear(cfg, seed, "lm_head", (V, H)))
    for name, shape in cfg.gain_shapes().items():
        if want is None or name in want:
            out[name] = _gain(cfg, seed, name, shape)
    for name, shape in cfg.linear_shapes().items():
        if want is None or name in want:
            out.update(_linear(cfg, seed, name, shape))
    return out


def prompt_ids(cfg: ModelConfig, n: int, seed: int = 0, index: int = 0) -> np.ndarray:
    """n uniform token ids in [0, vocab) for prompt number ``index``."""
    return uniform_int(key_of(seed, "%s/prompt/%d" % (cfg.family, index)), n, cfg.vocab)


def corrupt_drafts(cfg: ModelConfig, greedy: np.ndarray, p: float, seed: int, round_: int
                   ) -> np.ndarray:
    """Replace each id independently with probability p by a uniform id."""
    n = len(greedy)
    u = uniform_f64(key_of(seed, "%s/draft/u/%d" % (cfg.family, round_)), n)
    r = uniform_int(key_of(seed, "%s/draft/id/%d" % (cfg.family, round_)), n, cfg.vocab)
    out = np.array(greedy, dtype=np.int32).copy()
    repl = u < p
    out[repl] = r[repl]
    return out
