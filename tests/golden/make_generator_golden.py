"""Writes generator.txt: a fingerprint of the seeded input recipe (calls synth only)."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import synth  # noqa: E402

w = synth.make_weights(synth.TINY, 0, names=["layers.0.self_attn.q_proj"])
ids = synth.prompt_ids(synth.TINY, 16, 0)
out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "generator.txt")
with open(out, "w") as f:
    f.write("# fingerprint of the synth input recipe, written by make_generator_golden.py\n")
    f.write("tiny_prompt = %s\n" % " ".join(str(int(i)) for i in ids))
    f.write("tiny_q0_sum = %.17g\n" % float(w["layers.0.self_attn.q_proj"].astype(np.float64).sum()))
