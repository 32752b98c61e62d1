"""CPU oracle of the dense decoder forward pass -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the GPU library (decoder_prefill_kv_amd).
"""
from .decoder import (KVCache, OracleModel, accept_length, apply_rope, argmax_lowest,  # noqa: F401
                      dequant_i8, dequant_q4, dequant_q8, dequant_q40, quantize_kv, greedy_run, rms_norm, rope_angles, silu, softmax, tie_exempt,
                      unpack_q4, verify)
