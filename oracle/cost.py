"""The speedup model of speculative decoding (float64).

LLM Primer ch. 9, section 9.3: the speedup of a speculative step is the
expected number of accepted tokens divided by (T_draft / T_decode + 1 +
alpha * N), where alpha is the verification overhead per candidate position
(typically 0.05 to 0.15) and N the number of candidates. With N growing,
alpha * N eventually dominates, so there is a best N (the pages put it at
6 to 8 for an acceptance rate of 0.8 and 10 to 12 for 0.9), and as the
acceptance rate approaches 1 the speedup approaches 1 / alpha.

Readings: "expected accepted tokens" counts every token a step emits
(accepted candidates plus the one drawn at the stopping node), which for a
chain of N candidates accepted with probability p each is
sum_{i=0}^{N} p^i (jisaku.com glossary, linear-speculation closed form);
for a tree, with the draft's own estimate of acceptance (the product of q
along a node's path), it is 1 + the sum over candidate nodes of their path
products.
"""

from __future__ import annotations

import math

import numpy as np


def speedup(expected_emitted: float, draft_ratio: float, alpha: float, n: int) -> float:
    """E[emitted] / (T_draft/T_decode + 1 + alpha * N)."""
    return float(expected_emitted) / (float(draft_ratio) + 1.0 + float(alpha) * n)


def chain_expected_emitted(p: float, n: int) -> float:
    """sum_{i=0}^{n} p^i, term by term."""
    total, term = 0.0, 1.0
    for _ in range(n + 1):
        total += term
        term *= p
    return total


def best_chain_length(p: float, draft_ratio: float, alpha: float, n_max: int):
    """The N in [1, n_max] with the largest model speedup for a chain (the
    smallest such N on ties); returns (N, speedup)."""
    best_n, best_s = 0, -math.inf
    for n in range(1, n_max + 1):
        s = speedup(chain_expected_emitted(p, n), draft_ratio, alpha, n)
        if s > best_s:
            best_n, best_s = n, s
    return best_n, best_s


def tree_expected_emitted(parent, logq) -> float:
    """1 + sum over non-root nodes of exp(sum of log q along the path)."""
    par = np.asarray(parent)
    lq = np.asarray(logq, dtype=np.float64)
    total = 1.0
    for i in range(1, par.shape[0]):
        s, j = 0.0, i
        while j != 0:
            s += min(float(lq[j]), 0.0)
            j = int(par[j])
        total += math.exp(s)
    return total


def alpha_from_times(n_values, step_us) -> float:
    """Per-position overhead from verification times T(N): the least-squares
    slope of T(N) / T(1) - 1 against N - 1 (through the origin), with T(1)
    the time at the smallest N given, which must be 1."""
    n = np.asarray(n_values, dtype=np.float64)
    t = np.asarray(step_us, dtype=np.float64)
    if n[0] != 1:
        raise ValueError("the first N must be 1")
    x = n - 1.0
    y = t / t[0] - 1.0
    return float((x * y).sum() / (x * x).sum())


def linear_us(params: float, tokens: int, hbm_gbs: float, mfma_tflops: float) -> float:
    """Roofline time of a bf16 weight matrix product: its weights read once
    (2 bytes each) or 2 FLOP per weight per token, whichever takes longer."""
    return max(2.0 * params / (hbm_gbs * 1e3), 2.0 * params * tokens / (mfma_tflops * 1e6))


def verify_speedup(expected_emitted: float, draft_ratio: float, layers: int,
                   layer_params: float, head_params: float, batch: int, n: int,
                   attn_verify_us: float, sampler_verify_us: float, attn_decode_us: float,
                   sampler_decode_us: float, hbm_gbs: float, mfma_tflops: float):
    """The speedup model of LLM Primer ch. 9 section 9.3 with a whole decode
    step as the baseline, at batch B (the yuuk.io wiki notes the speedup
    falls as the batch grows; this is why):

      T_decode = layers (lin(B) + attn_decode) + head(B) + sampler_decode
      T_verify = layers (lin(B n) + attn_verify) + head(B n) + sampler_verify
      alpha    = (T_verify / T_decode - 1) / n
      speedup  = E / (T_draft/T_decode + 1 + alpha n)

    lin and head are ``linear_us`` of a layer's projections and of the
    vocabulary head; attn and sampler are measured times of one layer's
    attention and of the walk. Returns (speedup, alpha, T_decode, T_verify),
    times in us."""
    t_dec = layers * (linear_us(layer_params, batch, hbm_gbs, mfma_tflops) + attn_decode_us) \
        + linear_us(head_params, batch, hbm_gbs, mfma_tflops) + sampler_decode_us
    t_ver = layers * (linear_us(layer_params, batch * n, hbm_gbs, mfma_tflops) + attn_verify_us) \
        + linear_us(head_params, batch * n, hbm_gbs, mfma_tflops) + sampler_verify_us
    alpha = (t_ver / t_dec - 1.0) / n
    return speedup(expected_emitted, draft_ratio, alpha, n), alpha, t_dec, t_ver
