"""CPU oracle for the dense decoder forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The GPU library never calls it, and it
shares no code with the GPU library: the only common dependency is the
``synth`` input generator, which holds no decoder arithmetic.

What it computes (plain, slow, obviously correct; float64 by default):

* The block is a pre-norm Llama/Qwen decoder layer: RMSNorm -> QKV -> RoPE ->
  grouped-query causal attention -> output projection + residual -> RMSNorm ->
  SwiGLU MLP + residual ("LLMs on the ANE" page, section "What's inside").
* Qwen3 specifics: head_dim independent of hidden/heads, and a per-head
  RMSNorm on Q and K applied before RoPE ("LLMs on the ANE", "Correctness").
* The decode order per token -- embedding gather, per layer norm / q,k,v GEMV /
  rope at the cache length / cache append / attention over the cache / o GEMV /
  add / norm / gate, up / silu-mul / down / add, then final norm and lm_head --
  follows the single-token decode diagram of the Butter architecture notes.
* The KV cache is resident state; a step writes one slot ("LLMs on the ANE",
  "Prefill and decode"; Butter notes, decode diagram).
* MLX 4-bit affine weights: w = scale * code + bias per group of 64 inputs
  (oxinfer 0.0.5 docs, "MLX checkpoints"); int8 weights with one scale per
  output row, w = scale * q ("LLMs on the ANE", "Quantized weights").
* Greedy speculative verify: accept while draft[i] equals the argmax of row i,
  then one bonus token; a KV cache rolls back by moving its length cursor
  (Butter notes, speculative decoding loop; oxinfer docs, "Speculative
  decoding": greedy verification reproduces plain greedy output).

Readings where the pages are silent (each one is listed in the design notes):
RMSNorm is x / sqrt(mean(x^2) + eps) * g; RoPE pairs element i with i + d/2
("rotate_half") and uses inv_freq_i = theta^(-2i/d); the attention scale is
1/sqrt(head_dim); query head h uses KV head floor(h / G); linear layers are
[out, in] without biases; argmax ties go to the lowest index.

The block path (``forward_block``, used for prefill and verify) and the step
path (``forward_step``, used for decode) are written separately -- matrix
products over all rows with an explicit masked score matrix versus matrix-
vector products over the cache -- so that their agreement is a real check.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import synth


# --------------------------------------------------------------------------
# element-wise pieces
# --------------------------------------------------------------------------

def rms_norm(x: torch.Tensor, g: torch.Tensor, eps: float) -> torch.Tensor:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    Named (rms_norm(x, weight, eps)) in the Butter decode diagram and as the
    block's norm in "LLMs on the ANE", "What's inside"; the formula is the
    standard RMSNorm definition (reading: no mean subtraction, gain g)."""
    ms = (x * x).mean(dim=-1, keepdim=True)
    return x / torch.sqrt(ms + eps) * g


def rope_angles(positions: torch.Tensor, head_dim: int, theta: float, dtype) -> torch.Tensor:
    """phi[p, i] = pos_p * theta^(-2i/d) for i < d/2."""
    i = torch.arange(head_dim // 2, dtype=torch.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return (positions.to(torch.float64)[:, None] * inv_freq[None, :]).to(dtype)


def apply_rope(x: torch.Tensor, positions: torch.Tensor, theta: float) -> torch.Tensor:
    """x * cos + rotate_half(x) * sin ("LLMs on the ANE", "What's inside").

    x: [M, heads, d]; positions: [M].  rotate_half(x) = (-x[d/2:], x[:d/2]), so
    the pair (x_i, x_{i+d/2}) is rotated by the angle phi_i."""
    d = x.shape[-1]
    phi = rope_angles(positions, d, theta, x.dtype)           # [M, d/2]
    cos = torch.cat([torch.cos(phi), torch.cos(phi)], dim=-1)[:, None, :]
    sin = torch.cat([torch.sin(phi), torch.sin(phi)], dim=-1)[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    rot = torch.cat([-x2, x1], dim=-1)
    return x * cos + rot * sin


def softmax(s: torch.Tensor) -> torch.Tensor:
    """Max-subtracted softmax over the last axis (masked entries are -inf)."""
    m = s.max(dim=-1, keepdim=True).values
    e = torch.exp(s - m)
    return e / e.sum(dim=-1, keepdim=True)


def silu(z: torch.Tensor) -> torch.Tensor:
    """silu(z) = z / (1 + exp(-z)) (the silu_mul step of the Butter diagram)."""
    return z / (1.0 + torch.exp(-z))


def argmax_lowest(x: torch.Tensor) -> int:
    """Index of the maximum; exact ties go to the lowest index."""
    m = x.max()
    return int(torch.nonzero(x == m)[0, 0])


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

def unpack_q4(codes: np.ndarray) -> np.ndarray:
    """uint32 [N, K/8] -> uint8 [N, K]; element 8w+j is bits 4j..4j+3 of word w."""
    n, kw = codes.shape
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    nib = (codes[:, :, None] >> shifts) & np.uint32(0xF)
    return nib.reshape(n, kw * 8).astype(np.uint8)


def dequant_q4(codes: np.ndarray, scales_bf16: np.ndarray, biases_bf16: np.ndarray,
               dtype=torch.float64) -> torch.Tensor:
    """w[n, k] = scale[n, k//64] * code[n, k] + bias[n, k//64]
    (oxinfer docs, "MLX checkpoints"), evaluated in float64."""
    c = torch.from_numpy(unpack_q4(codes)).to(torch.float64)
    s = torch.from_numpy(synth.bf16_bits_to_f32(scales_bf16)).to(torch.float64)
    b = torch.from_numpy(synth.bf16_bits_to_f32(biases_bf16)).to(torch.float64)
    s = torch.repeat_interleave(s, 64, dim=1)
    b = torch.repeat_interleave(b, 64, dim=1)
    return (c * s + b).to(dtype)


def dequant_i8(q: np.ndarray, scales_bf16: np.ndarray, dtype=torch.float64) -> torch.Tensor:
    """w[n, k] = scale[n] * q[n, k] (int8 with one scale per output row, the
    int8 weights of "LLMs on the ANE", "Quantized weights"), in float64."""
    s = torch.from_numpy(synth.bf16_bits_to_f32(scales_bf16)).to(torch.float64)
    return (torch.from_numpy(q.astype(np.float64)) * s).to(dtype)


def dequant_q8(q: np.ndarray, scales_f32: np.ndarray, dtype=torch.float64) -> torch.Tensor:
    """w[n, k] = scale[n, k // 32] * q[n, k], in float64: int8 codes in blocks of
    32 weights along the input dimension, one float32 scale per block (oxinfer
    docs page, "Build and run", the q8 quantization flag)."""
    s = torch.from_numpy(np.ascontiguousarray(scales_f32, dtype=np.float32).astype(np.float64))
    return (torch.from_numpy(q.astype(np.float64)) * torch.repeat_interleave(s, 32, dim=1)).to(dtype)


def dequant_q40(packed: np.ndarray, d_f16: np.ndarray, dtype=torch.float64) -> torch.Tensor:
    """w = d * (c - 8) for GGUF-style 4-bit blocks of 32 weights (oxinfer docs
    page, "Build and run", the q4 quantization flag: blocks of 32, 4-bit codes,
    an fp16 scale).  Byte j of a block's 16 holds code j in its low nibble and
    code j + 16 in its high nibble.  In float64."""
    rows, half = packed.shape
    b = packed.reshape(rows, half // 16, 16).astype(np.int64)
    codes = np.concatenate([b & 0xF, b >> 4], axis=2)  # [rows, blocks, 32]
    d = np.ascontiguousarray(d_f16, dtype=np.float16).astype(np.float64)
    w = d[..., None] * (codes.astype(np.float64) - 8.0)
    return torch.from_numpy(w.reshape(rows, half * 2)).to(dtype)


class OracleModel:
    """The decoder with weights taken exactly as stored (bf16 widen exactly)."""

    def __init__(self, cfg: synth.ModelConfig, weights: Dict[str, np.ndarray],
                 dtype=torch.float64, cache_weights: bool = True):
        self.cfg = cfg
        self.w = weights
        self.dtype = dtype
        self.cache_weights = cache_weights
        self._cache: Dict[str, torch.Tensor] = {}

    def _dense(self, name: str) -> torch.Tensor:
        cfg = self.cfg
        if cfg.weight_format == "q4" and name + ".codes" in self.w:
            return dequant_q4(self.w[name + ".codes"], self.w[name + ".scales"],
                              self.w[name + ".biases"], self.dtype)
        if cfg.weight_format == "i8" and name + ".q" in self.w:
            return dequant_i8(self.w[name + ".q"], self.w[name + ".scales"], self.dtype)
        if cfg.weight_format == "q8" and name + ".q" in self.w:
            return dequant_q8(self.w[name + ".q"], self.w[name + ".scales"], self.dtype)
        if cfg.weight_format == "q4_0" and name + ".q" in self.w:
            return dequant_q40(self.w[name + ".q"], self.w[name + ".scales"], self.dtype)
        a = self.w[name]
        if a.dtype == np.uint16:
            return torch.from_numpy(synth.bf16_bits_to_f32(a)).to(self.dtype)
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.dtype)

    def W(self, name: str) -> torch.Tensor:
        if name in self._cache:
            return self._cache[name]
        t = self._dense(name)
        if self.cache_weights:
            self._cache[name] = t
        return t

    def _kv(self, x: torch.Tensor) -> torch.Tensor:
        """What the cache holds for new keys / values x [..., d]."""
        return quantize_kv(x) if self.cfg.kv_i8 else x

    def head_name(self) -> str:
        return "embed_tokens" if self.cfg.tied else "lm_head"

    def embed_rows(self, ids: Sequence[int]) -> torch.Tensor:
        """h = E[id] (Butter decode diagram: gather).  A 4-bit table is
        dequantized one row at a time (oxinfer docs, "MLX checkpoints")."""
        cfg = self.cfg
        ids = [int(i) for i in ids]
        if cfg.weight_format == "q4":
            rows = [dequant_q4(self.w["embed_tokens.codes"][i:i + 1],
                               self.w["embed_tokens.scales"][i:i + 1],
                               self.w["embed_tokens.biases"][i:i + 1], self.dtype)[0]
                    for i in ids]
            return torch.stack(rows)
        if cfg.weight_format == "i8":
            sel = np.array(ids, dtype=np.int64)
            return dequant_i8(self.w["embed_tokens.q"][sel], self.w["embed_tokens.scales"][sel], self.dtype)
        if cfg.weight_format == "q8":
            sel = np.array(ids, dtype=np.int64)
            return dequant_q8(self.w["embed_tokens.q"][sel], self.w["embed_tokens.scales"][sel], self.dtype)
        if cfg.weight_format == "q4_0":
            sel = np.array(ids, dtype=np.int64)
            return dequant_q40(self.w["embed_tokens.q"][sel], self.w["embed_tokens.scales"][sel], self.dtype)
        E = self.w["embed_tokens"]
        rows = E[np.array(ids, dtype=np.int64)]
        if rows.dtype == np.uint16:
            rows = synth.bf16_bits_to_f32(rows)
        return torch.from_numpy(np.ascontiguousarray(rows)).to(self.dtype)

    def new_cache(self, max_seq: int) -> "KVCache":
        return KVCache(self.cfg, max_seq, self.dtype)

    # ----------------------------------------------------------------------
    # block path: M rows at positions start..start+M-1 (prefill, verify)
    # ----------------------------------------------------------------------
    def forward_block(self, cache: "KVCache", ids: Sequence[int], start: int,
                      all_rows: bool = False) -> torch.Tensor:
        cfg = self.cfg
        M = len(ids)
        assert start <= cache.length and start + M <= cache.max_seq
        d, Hq, Hkv, G = cfg.head_dim, cfg.n_heads, cfg.n_kv_heads, cfg.group
        pos = torch.arange(start, start + M)
        h = self.embed_rows(ids)                                   # [M, H]
        T = start + M
        # key j is visible to row i iff j <= start + i (causal within the block,
        # everything before the block is visible)
        visible = torch.arange(T)[None, :] <= pos[:, None]        # [M, T]
        for l in range(cfg.n_layers):
            p = "layers.%d." % l
            y = rms_norm(h, self.W(p + "input_layernorm"), cfg.rms_eps)
            q = (y @ self.W(p + "self_attn.q_proj").T).view(M, Hq, d)
            k = (y @ self.W(p + "self_attn.k_proj").T).view(M, Hkv, d)
            v = (y @ self.W(p + "self_attn.v_proj").T).view(M, Hkv, d)
            if cfg.qk_norm:
                q = rms_norm(q, self.W(p + "self_attn.q_norm"), cfg.rms_eps)
                k = rms_norm(k, self.W(p + "self_attn.k_norm"), cfg.rms_eps)
            q = apply_rope(q, pos, cfg.rope_theta)
            k = apply_rope(k, pos, cfg.rope_theta)
            cache.k[l][:, start:T, :] = self._kv(k.transpose(0, 1))
            cache.v[l][:, start:T, :] = self._kv(v.transpose(0, 1))
            o = torch.empty(M, Hq, d, dtype=self.dtype)
            for hh in range(Hq):
                g = hh // G
                K = cache.k[l][g, :T, :]                            # [T, d]
                V = cache.v[l][g, :T, :]
                s = (q[:, hh, :] @ K.T) / math.sqrt(d)              # [M, T]
                s = s.masked_fill(~visible, float("-inf"))
                o[:, hh, :] = softmax(s) @ V
            h = h + o.reshape(M, Hq * d) @ self.W(p + "self_attn.o_proj").T
            y = rms_norm(h, self.W(p + "post_attention_layernorm"), cfg.rms_eps)
            gate = y @ self.W(p + "mlp.gate_proj").T
            up = y @ self.W(p + "mlp.up_proj").T
            h = h + (silu(gate) * up) @ self.W(p + "mlp.down_proj").T
        cache.length = T
        rows = h if all_rows else h[-1:]
        hn = rms_norm(rows, self.W("norm"), cfg.rms_eps)
        return hn @ self.W(self.head_name()).T                      # [rows, V]

    # ----------------------------------------------------------------------
    # step path: one token at position pos against the cache (decode)
    # ----------------------------------------------------------------------
    def forward_step(self, cache: "KVCache", token: int, pos: int) -> torch.Tensor:
        cfg = self.cfg
        assert pos <= cache.length and pos < cache.max_seq
        d, Hq, Hkv, G = cfg.head_dim, cfg.n_heads, cfg.n_kv_heads, cfg.group
        x = self.embed_rows([token])[0]                             # [H]
        posv = torch.tensor([pos])
        for l in range(cfg.n_layers):
            p = "layers.%d." % l
            y = rms_norm(x, self.W(p + "input_layernorm"), cfg.rms_eps)
            q = torch.mv(self.W(p + "self_attn.q_proj"), y).view(1, Hq, d)
            k = torch.mv(self.W(p + "self_attn.k_proj"), y).view(1, Hkv, d)
            v = torch.mv(self.W(p + "self_attn.v_proj"), y).view(Hkv, d)
            if cfg.qk_norm:
                q = rms_norm(q, self.W(p + "self_attn.q_norm"), cfg.rms_eps)
                k = rms_norm(k, self.W(p + "self_attn.k_norm"), cfg.rms_eps)
            q = apply_rope(q, posv, cfg.rope_theta)[0]                # [Hq, d]
            k = apply_rope(k, posv, cfg.rope_theta)[0]                # [Hkv, d]
            cache.k[l][:, pos, :] = self._kv(k)
            cache.v[l][:, pos, :] = self._kv(v)
            o = torch.empty(Hq, d, dtype=self.dtype)
            for hh in range(Hq):
                g = hh // G
                K = cache.k[l][g, : pos + 1, :]
                V = cache.v[l][g, : pos + 1, :]
                s = torch.mv(K, q[hh]) / math.sqrt(d)                 # [pos+1]
                pr = softmax(s)
                o[hh] = torch.mv(V.T, pr)
            x = x + torch.mv(self.W(p + "self_attn.o_proj"), o.reshape(-1))
            y = rms_norm(x, self.W(p + "post_attention_layernorm"), cfg.rms_eps)
            gate = torch.mv(self.W(p + "mlp.gate_proj"), y)
            up = torch.mv(self.W(p + "mlp.up_proj"), y)
            x = x + torch.mv(self.W(p + "mlp.down_proj"), silu(gate) * up)
        cache.length = pos + 1
        xn = rms_norm(x, self.W("norm"), cfg.rms_eps)
        return torch.mv(self.W(self.head_name()), xn)               # [V]


def quantize_kv(x: torch.Tensor) -> torch.Tensor:
    """The value an int8 KV cache returns for x [..., d]: each position's
    head vector is held as int8 codes q = round(x / s) (clipped to +-127) with
    one float32 scale s = max |x| / 127 (Butter notes, architecture: the
    affine-quantized KV cache; here the affine map's offset is zero), and
    read back as s * q.  An all-zero vector has s = 0 and reads back zeros."""
    s = (x.abs().amax(dim=-1, keepdim=True).double() / 127.0).float().double()
    q = torch.clamp(torch.round(x.double() / torch.where(s > 0, s, torch.ones_like(s))), -127, 127)
    return (s * q).to(x.dtype)


class KVCache:
    """Per layer K and V of shape [n_kv_heads, max_seq, head_dim] and a length
    cursor; rolling back is setting the cursor (Butter notes, cache rollback)."""

    def __init__(self, cfg: synth.ModelConfig, max_seq: int, dtype):
        self.max_seq = max_seq
        self.length = 0
        shape = (cfg.n_kv_heads, max_seq, cfg.head_dim)
        self.k = [torch.zeros(shape, dtype=dtype) for _ in range(cfg.n_layers)]
        self.v = [torch.zeros(shape, dtype=dtype) for _ in range(cfg.n_layers)]


# --------------------------------------------------------------------------
# schedules
# --------------------------------------------------------------------------

def greedy_run(model: OracleModel, prompt: Sequence[int], n_steps: int,
               max_seq: Optional[int] = None, keep_logits: bool = True) -> dict:
    """Prefill the prompt (block path), then n_steps greedy decode steps (step
    path).  g_0 = argmax of the prefill logits; step s consumes g_s at position
    P + s and yields g_{s+1}."""
    P = len(prompt)
    cache = model.new_cache(max_seq or (P + n_steps))
    logits = [model.forward_block(cache, prompt, 0)[0]]
    ids = [argmax_lowest(logits[0])]
    for s in range(n_steps):
        lg = model.forward_step(cache, ids[-1], P + s)
        ids.append(argmax_lowest(lg))
        logits.append(lg if keep_logits else None)
    return {"logits": logits, "ids": ids, "cache": cache}


def accept_length(ids_in: Sequence[int], argmax_rows: Sequence[int]) -> int:
    """Greedy acceptance: ids_in = [t, d_1..d_K]; m = number of leading drafts
    with d_{i+1} == argmax of row i (Butter notes, accept/reject, greedy)."""
    K = len(ids_in) - 1
    m = 0
    while m < K and int(ids_in[m + 1]) == int(argmax_rows[m]):
        m += 1
    return m


def verify(model: OracleModel, cache: KVCache, ids_in: Sequence[int], pos: int) -> dict:
    """One verify pass of K+1 rows at positions pos..pos+K (block path), then
    the accepted prefix m, the bonus token argmax[m] and the cursor pos+m+1."""
    logits = model.forward_block(cache, ids_in, pos, all_rows=True)
    am = [argmax_lowest(logits[i]) for i in range(logits.shape[0])]
    m = accept_length(ids_in, am)
    cache.length = pos + m + 1
    return {"logits": logits, "argmax": am, "accepted": m, "bonus": am[m]}


def tie_exempt(logits: torch.Tensor, rel: float = 3e-3) -> bool:
    """True when the top-2 gap is below rel * max|logit| ("LLMs on the ANE",
    "lm_head on the ANE": the tie-margin rule)."""
    top2 = torch.topk(logits.to(torch.float64), 2).values
    return bool(top2[0] - top2[1] < rel * logits.abs().max())
