"""CPU oracle for token sampling and speculative-sampling acceptance -- TEST
INFRASTRUCTURE ONLY (only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` may import it; the GPU library never does).

What it computes, in float64, from the plain definitions:

* The sampling distribution of one logit row ("Butter architecture notes",
  GPU sampling diagram: temperature, top-k and top-p applied to the logits in
  a final kernel; oxinfer 0.0.5 docs, "Speculative decoding", sampled
  generation):
    - temperature T: z = logits / T (T = 0 means greedy: all mass on the
      lowest index of the maximum);
    - top-k (k > 0): keep the tokens whose z is at least the k-th largest z
      (tokens tied with the k-th value are kept);
    - softmax over the kept tokens;
    - top-p (0 < p < 1): walk the kept tokens by decreasing probability; the
      probability v* of the token at which the running mass first reaches p
      is the cut, and every token with probability >= v* is kept (ties with
      the cut are kept, so the set does not depend on how ties are ordered);
    - renormalise over what is kept.
* Drawing a token from a distribution with a uniform u in [0, 1): the
  smallest index i whose cumulative probability (in index order) exceeds u.
* Speculative-sampling acceptance (oxinfer docs, "Speculative decoding": the
  standard speculative-sampling acceptance rule; Butter notes, speculative
  decoding loop): for drafts d_1..d_K drawn from the draft's distributions
  q_1..q_K and the target's distributions p_0..p_K from one verify pass,
  draft d_i is accepted when r_i < min(1, p_{i-1}(d_i) / q_i(d_i)); at the
  first rejection the next token is drawn from the residual
  max(0, p_{i-1} - q_i), renormalised, with the uniform u_i; if all K are
  accepted the bonus token is drawn from p_K with u_K.  The rule makes the
  emitted token follow the target's distribution exactly (checked by
  enumeration in the tests).
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np
import torch


def sampling_probs(logits: torch.Tensor, temperature: float, top_k: int = 0, top_p: float = 1.0) -> torch.Tensor:
    """float64 probabilities over the vocabulary after temperature, top-k and
    top-p (zeros outside the kept set)."""
    x = logits.to(torch.float64).reshape(-1)
    V = x.numel()
    if temperature == 0.0:
        out = torch.zeros(V, dtype=torch.float64)
        out[int(torch.nonzero(x == x.max())[0, 0])] = 1.0
        return out
    z = x / temperature
    keep = torch.ones(V, dtype=torch.bool)
    if 0 < top_k < V:
        kth = torch.sort(z, descending=True).values[top_k - 1]
        keep = z >= kth
    zk = torch.where(keep, z, torch.full_like(z, float("-inf")))
    w = torch.exp(zk - zk.max())
    p = w / w.sum()
    if top_p < 1.0:
        order = torch.sort(p, descending=True, stable=True).values
        run = torch.cumsum(order, 0)
        n = int(torch.nonzero(run >= top_p)[0, 0]) if bool((run >= top_p).any()) else V - 1
        cut = order[n]
        p = torch.where(p >= cut, p, torch.zeros_like(p))
        p = p / p.sum()
    return p


def draw(probs: torch.Tensor, u: float) -> int:
    """Smallest index whose cumulative probability (index order) exceeds u."""
    c = torch.cumsum(probs.to(torch.float64), 0)
    hit = torch.nonzero(c > u * c[-1])
    return int(hit[0, 0]) if hit.numel() else int(torch.nonzero(probs > 0)[-1, 0])


def sample(logits: torch.Tensor, u: float, temperature: float, top_k: int = 0, top_p: float = 1.0) -> int:
    return draw(sampling_probs(logits, temperature, top_k, top_p), u)


def residual(p: torch.Tensor, q: torch.Tensor) -> torch.Tensor:
    """max(0, p - q) renormalised (the distribution drawn from after a
    rejection); if p <= q everywhere the residual is p itself."""
    r = torch.clamp(p - q, min=0.0)
    s = r.sum()
    return r / s if s > 0 else p


def spec_accept(target_logits: torch.Tensor, draft_logits: torch.Tensor, drafts: Sequence[int],
                r: Sequence[float], u: Sequence[float], temperature: float, top_k: int = 0,
                top_p: float = 1.0) -> Dict[str, int]:
    """Speculative-sampling acceptance of K drafts.  target_logits [K+1, V]
    (rows 0..K of a verify pass), draft_logits [K, V] (the draft's row that
    drew d_i is row i-1), r [K] acceptance uniforms, u [K+1] uniforms for the
    residual / bonus draw.  Returns the accepted count m and the next token."""
    K = len(drafts)
    for i in range(K):
        p = sampling_probs(target_logits[i], temperature, top_k, top_p)
        q = sampling_probs(draft_logits[i], temperature, top_k, top_p)
        d = int(drafts[i])
        if not (float(r[i]) * float(q[d]) < float(p[d])):
            return {"accepted": i, "token": draw(residual(p, q), float(u[i]))}
    p = sampling_probs(target_logits[K], temperature, top_k, top_p)
    return {"accepted": K, "token": draw(p, float(u[K]))}


def emitted_distribution(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Exact distribution of the first emitted token under the acceptance
    rule, by enumeration: a draft d ~ q is kept with probability
    min(1, p(d)/q(d)), otherwise the token comes from the residual."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros_like(p)
    reject = 0.0
    for d in range(len(p)):
        if q[d] == 0.0:
            continue
        a = min(1.0, p[d] / q[d])
        out[d] += q[d] * a
        reject += q[d] * (1.0 - a)
    res = residual(torch.from_numpy(p), torch.from_numpy(q)).numpy()
    return out + reject * res
