"""Python binding of the dpk C-ABI library (dense decoder prefill / KV-cache
decode on MI355X).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of ``_dpk.so``.  PyTorch provides device memory and streams.  The
functions below carry the C names without the ``dpk_`` prefix; ``Decoder``
bundles the usual create / allocate / bind / load sequence.

The library is required: importing this package raises if ``_dpk.so`` has not
been built (``python -m decoder_prefill_kv_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_dpk.so")

DPK_OK, DPK_EINVAL, DPK_ERANGE, DPK_ESTATE, DPK_ENOMEM, DPK_EHIP = 0, -1, -2, -3, -4, -5
FMT_F32, FMT_BF16, FMT_Q4G64, FMT_I8, FMT_Q8, FMT_Q40 = 0, 1, 2, 3, 4, 5
FLAG_PREFILL_STREAM = 1
FLAG_KV_I8 = 4
DT_F32, DT_BF16, DT_U32, DT_I8, DT_U8, DT_F16 = 0, 1, 2, 3, 4, 5
SYMBOLS = ["dpk_create", "dpk_workspace_size", "dpk_bind_workspace", "dpk_load_weights", "dpk_prefill",
           "dpk_prefill_at", "dpk_decode_step", "dpk_verify", "dpk_seq_length", "dpk_check_device_errors",
           "dpk_test_set_barrier_abort", "dpk_profile_begin", "dpk_profile_end", "dpk_spec_generate", "dpk_sample",
           "dpk_spec_accept_workspace_size", "dpk_spec_accept", "dpk_spec_accept_noalloc", "dpk_last_error",
           "dpk_destroy"]


class DpkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("dpk status %d: %s" % (status, msg))
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double),
                ("qk_norm", ctypes.c_int32), ("tied_embedding", ctypes.c_int32),
                ("weight_format", ctypes.c_int32), ("max_batch", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("max_rows", ctypes.c_int32), ("flags", ctypes.c_int32)]


class Tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class SpecConfig(ctypes.Structure):
    _fields_ = [("k_init", ctypes.c_int32), ("k_min", ctypes.c_int32), ("k_max", ctypes.c_int32)]


class SpecStats(ctypes.Structure):
    _fields_ = [("rounds", ctypes.c_int32), ("drafted", ctypes.c_int32), ("accepted", ctypes.c_int32),
                ("draft_steps", ctypes.c_int32)]


class Sampler(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float)]


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("bytes", ctypes.c_double), ("flops", ctypes.c_double)]


def library_path() -> str:
    return _SO


def _load():
    if not os.path.exists(_SO):
        raise ImportError("dpk native library not built: %s (run python -m decoder_prefill_kv_amd.build)" % _SO)
    lib = ctypes.CDLL(_SO)
    vp, i32, p32 = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
    sz = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "dpk_create": [ctypes.POINTER(Config), ctypes.POINTER(vp)],
        "dpk_workspace_size": [vp, sz, sz, sz],
        "dpk_bind_workspace": [vp, vp, vp, vp, vp],
        "dpk_load_weights": [vp, ctypes.POINTER(Tensor), i32, vp],
        "dpk_prefill": [vp, i32, p32, i32, vp, vp, vp],
        "dpk_prefill_at": [vp, i32, i32, p32, i32, vp, vp, vp],
        "dpk_decode_step": [vp, i32, p32, p32, vp, p32, vp, vp, vp],
        "dpk_verify": [vp, i32, p32, i32, i32, vp, vp, p32, vp],
        "dpk_seq_length": [vp, i32, p32],
        "dpk_check_device_errors": [vp, vp],
        "dpk_test_set_barrier_abort": [vp, vp],
        "dpk_profile_begin": [vp, i32],
        "dpk_profile_end": [vp, ctypes.POINTER(KernelStat), i32, p32],
        "dpk_spec_generate": [vp, vp, i32, i32, i32, i32, ctypes.POINTER(SpecConfig), p32,
                              ctypes.POINTER(SpecStats), vp],
        "dpk_sample": [vp, i32, i32, ctypes.c_int64, ctypes.POINTER(Sampler), vp, vp, vp],
        "dpk_spec_accept_workspace_size": [i32, sz],
        "dpk_spec_accept": [vp, vp, ctypes.c_int64, i32, i32, vp, ctypes.POINTER(Sampler), vp, vp, vp, vp,
                            ctypes.c_size_t, vp],
        "dpk_spec_accept_noalloc": [vp, vp, ctypes.c_int64, i32, i32, vp, ctypes.POINTER(Sampler), vp, vp, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.dpk_last_error.restype = ctypes.c_char_p
    lib.dpk_last_error.argtypes = []
    lib.dpk_destroy.restype = None
    lib.dpk_destroy.argtypes = [vp]
    return lib


_lib_handle = None


def lib():
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = _load()
    return _lib_handle


def last_error() -> str:
    return lib().dpk_last_error().decode()


def _check(st: int):
    if st != DPK_OK:
        raise DpkError(st, last_error())


def _i32(a: Sequence[int]):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ------------------------------------------------------------------ C names
def create(cfg: Config) -> int:
    h = ctypes.c_void_p()
    _check(lib().dpk_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h.value


def workspace_size(model: int):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().dpk_workspace_size(model, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def bind_workspace(model: int, kv: int, scratch: int, prep: Optional[int], stream=None):
    _check(lib().dpk_bind_workspace(model, kv, scratch, prep, _stream(stream)))


def load_weights(model: int, tensors: Sequence[Tensor], stream=None):
    arr = (Tensor * len(tensors))(*tensors)
    _check(lib().dpk_load_weights(model, arr, len(tensors), _stream(stream)))


def prefill(model: int, seq: int, ids: Sequence[int], logits_dev=None, argmax_dev=None, stream=None):
    a, p = _i32(ids)
    _check(lib().dpk_prefill(model, seq, p, len(a), _ptr(logits_dev), _ptr(argmax_dev), _stream(stream)))


def prefill_at(model: int, seq: int, start: int, ids: Sequence[int], logits_dev=None, argmax_dev=None,
               stream=None):
    a, p = _i32(ids)
    _check(lib().dpk_prefill_at(model, seq, start, p, len(a), _ptr(logits_dev), _ptr(argmax_dev),
                                _stream(stream)))


def decode_step(model: int, seqs: Sequence[int], ids: Optional[Sequence[int]], pos: Sequence[int], argmax_dev,
                logits_dev=None, ids_dev=None, stream=None):
    s, sp = _i32(seqs)
    q, qp = _i32(pos)
    if ids is not None:
        i, ip = _i32(ids)
    else:
        ip = None
    _check(lib().dpk_decode_step(model, len(s), sp, ip, _ptr(ids_dev), qp, _ptr(logits_dev), _ptr(argmax_dev),
                                _stream(stream)))


def verify(model: int, seq: int, ids: Sequence[int], pos: int, argmax_dev, logits_dev=None, stream=None) -> int:
    a, p = _i32(ids)
    acc = ctypes.c_int32()
    _check(lib().dpk_verify(model, seq, p, len(a), pos, _ptr(logits_dev), _ptr(argmax_dev), ctypes.byref(acc),
                           _stream(stream)))
    return acc.value


def seq_length(model: int, seq: int) -> int:
    v = ctypes.c_int32()
    _check(lib().dpk_seq_length(model, seq, ctypes.byref(v)))
    return v.value


def check_device_errors(model: int, stream=None):
    _check(lib().dpk_check_device_errors(model, _stream(stream)))


def test_set_barrier_abort(model: int, stream=None):
    _check(lib().dpk_test_set_barrier_abort(model, _stream(stream)))


def profile_begin(model: int, max_launches: int = 100000):
    _check(lib().dpk_profile_begin(model, max_launches))


def profile_end(model: int):
    """-> {class name: dict(launches, total_ms, bytes, flops)}"""
    arr = (KernelStat * 64)()
    n = ctypes.c_int32()
    st = lib().dpk_profile_end(model, arr, 64, ctypes.byref(n))
    out = {}
    for i in range(min(n.value, 64)):
        k = arr[i]
        out[k.name.decode()] = dict(launches=k.launches, total_ms=k.total_ms, bytes=k.bytes, flops=k.flops)
    _check(st)
    return out


def spec_generate(target: int, draft: int, seq: int, pos: int, token: int, n_new: int, k_init: int = 4,
                  k_min: int = 2, k_max: int = 6, stream=None):
    """-> (list of n_new token ids, stats dict)"""
    out = np.zeros(n_new, dtype=np.int32)
    sc = SpecConfig(k_init, k_min, k_max)
    st = SpecStats()
    _check(lib().dpk_spec_generate(target, draft, seq, pos, token, n_new, ctypes.byref(sc),
                                   out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(st),
                                   _stream(stream)))
    return [int(t) for t in out], dict(rounds=st.rounds, drafted=st.drafted, accepted=st.accepted,
                                        draft_steps=st.draft_steps)


def sample(logits_dev, u_dev, out_dev, temperature: float, top_k: int = 0, top_p: float = 1.0, stream=None):
    """One token per row of logits_dev (fp32 [rows, V] device tensor) with the
    rows' uniforms u_dev (fp32 [rows]) into out_dev (int32 [rows])."""
    rows, V = logits_dev.shape
    sp = Sampler(temperature, top_k, top_p)
    _check(lib().dpk_sample(_ptr(logits_dev), rows, V, logits_dev.stride(0), ctypes.byref(sp), _ptr(u_dev),
                            _ptr(out_dev), _stream(stream)))


def spec_accept_workspace_size(k: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().dpk_spec_accept_workspace_size(k, ctypes.byref(n)))
    return n.value


def spec_accept(target_logits, draft_logits, drafts_dev, r_dev, u_dev, out_dev, workspace, temperature: float,
                top_k: int = 0, top_p: float = 1.0, stream=None):
    """target_logits [k+1, V], draft_logits [k, V] (same row stride), drafts
    int32 [k], r fp32 [k], u fp32 [k+1], out int32 [2] (all device tensors);
    workspace: a device tensor of spec_accept_workspace_size(k) bytes."""
    k = draft_logits.shape[0]
    assert target_logits.stride(0) == draft_logits.stride(0)
    sp = Sampler(temperature, top_k, top_p)
    _check(lib().dpk_spec_accept(_ptr(target_logits), _ptr(draft_logits), target_logits.stride(0),
                                 target_logits.shape[1], k, _ptr(drafts_dev), ctypes.byref(sp), _ptr(r_dev),
                                 _ptr(u_dev), _ptr(out_dev), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def spec_accept_noalloc(target_logits, draft_logits, drafts_dev, r_dev, u_dev, out_dev, temperature: float,
                        top_k: int = 0, top_p: float = 1.0, stream=None):
    """spec_accept with the library's built-in workspace (no allocation)."""
    k = draft_logits.shape[0]
    assert target_logits.stride(0) == draft_logits.stride(0)
    sp = Sampler(temperature, top_k, top_p)
    _check(lib().dpk_spec_accept_noalloc(_ptr(target_logits), _ptr(draft_logits), target_logits.stride(0),
                                         target_logits.shape[1], k, _ptr(drafts_dev), ctypes.byref(sp),
                                         _ptr(r_dev), _ptr(u_dev), _ptr(out_dev), _stream(stream)))


def destroy(model: int):
    lib().dpk_destroy(model)


# ------------------------------------------------------------------ convenience
_FMT = {"f32": FMT_F32, "bf16": FMT_BF16, "q4": FMT_Q4G64, "i8": FMT_I8, "q8": FMT_Q8, "q4_0": FMT_Q40}


def make_config(mc, max_batch: int, max_seq: int, max_rows: int = 512, flags: int = 0) -> Config:
    """dpk_config from any object with the decoder shape attributes (an int8
    KV cache when the object's ``kv_i8`` is true)."""
    if getattr(mc, "kv_i8", False):
        flags |= FLAG_KV_I8
    return Config(mc.n_layers, mc.hidden, mc.n_heads, mc.n_kv_heads, mc.head_dim, mc.intermediate, mc.vocab,
                  float(mc.rms_eps), float(mc.rope_theta), int(bool(mc.qk_norm)), int(bool(mc.tied)),
                  _FMT[mc.weight_format], max_batch, max_seq, max_rows, flags)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.uint32:
        return DT_U32
    if a.dtype == np.int8:
        return DT_I8
    if a.dtype == np.uint8:
        return DT_U8
    if a.dtype == np.float16:
        return DT_F16
    raise TypeError(a.dtype)


class Decoder:
    """Owns the device buffers of one model: weights, KV cache, scratch and the
    fp16 prefill copy, all allocated through torch on ``device``."""

    def __init__(self, mc, weights: Dict[str, np.ndarray], max_batch: int, max_seq: int, max_rows: int = 512,
                 device: str = "cuda", stream=None, flags: int = 0):
        import torch
        self.torch = torch
        self.mc = mc
        self.device = torch.device(device)
        self.stream = stream
        self.cfg = make_config(mc, max_batch, max_seq, max_rows, flags)
        self.handle = create(self.cfg)
        kvb, scb, prb = workspace_size(self.handle)
        alloc = lambda n: torch.empty(max(int(n), 256), dtype=torch.uint8, device=self.device)
        self.kv, self.scratch = alloc(kvb), alloc(scb)
        self.prep = alloc(prb) if prb else None
        self.sizes = (kvb, scb, prb)
        bind_workspace(self.handle, self.kv.data_ptr(), self.scratch.data_ptr(),
                       self.prep.data_ptr() if self.prep is not None else None, stream)
        self.wdev = {}
        tensors = []
        self._names = []
        for name, arr in weights.items():
            arr = np.ascontiguousarray(arr)
            t = torch.from_numpy(arr.view(np.uint8).reshape(-1)).to(self.device)
            self.wdev[name] = t
            rows, cols = (1, arr.shape[0]) if arr.ndim == 1 else arr.shape
            nb = name.encode()
            self._names.append(nb)
            tensors.append(Tensor(nb, t.data_ptr(), _dtype_code(arr), rows, cols))
        load_weights(self.handle, tensors, stream)
        self.vocab = mc.vocab

    def logits_buffer(self, rows: int = 1):
        return self.torch.empty(rows, self.vocab, dtype=self.torch.float32, device=self.device)

    def argmax_buffer(self, rows: int = 1):
        return self.torch.empty(rows, dtype=self.torch.int32, device=self.device)

    def prefill(self, seq: int, ids, logits=None, argmax=None):
        prefill(self.handle, seq, ids, logits, argmax, self.stream)

    def prefill_at(self, seq: int, start: int, ids, logits=None, argmax=None):
        prefill_at(self.handle, seq, start, ids, logits, argmax, self.stream)

    def decode_step(self, seqs, ids, pos, argmax, logits=None, ids_dev=None):
        decode_step(self.handle, seqs, ids, pos, argmax, logits, ids_dev, self.stream)

    def verify(self, seq: int, ids, pos: int, argmax, logits=None) -> int:
        return verify(self.handle, seq, ids, pos, argmax, logits, self.stream)

    def seq_length(self, seq: int) -> int:
        return seq_length(self.handle, seq)

    def close(self):
        if self.handle:
            self.torch.cuda.synchronize(self.device)
            destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
