"""CPU oracle for the KVzap scoring variant (test infrastructure only).

TEST INFRASTRUCTURE ONLY, like ``dms_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may import it;
it shares no code with the HIP library.  float64 throughout.

Pages followed:

* "动态内存稀疏化（DMS）策略：KVzap-linear-Llama-3.1-8B-Instruct的核心创新点"
  (below: *KVzap-linear page*), sections 什么是动态内存稀疏化（DMS）？ (score
  every KV pair, prune the ones below a threshold), KVzap-linear的技术架构
  (one linear layer from the hidden size 4096 to the 8 KV heads, float32;
  workflow: hidden states (T x D_h) -> scores (T x H) -> threshold plus a
  sliding window that keeps the last 128 tokens) and 快速集成指南
  (threshold -4).
* "革命性LLM加速技术：NVIDIA KVzap-mlp-Qwen3-8B如何实现高效KV缓存修剪？"
  (below: *KVzap-mlp page*), sections 模型架构 (two layers with a GELU
  between them, 4096 in, 8 out, 36 modules, about 76M parameters), 工作流程
  (the same three steps) and 高级配置 (threshold -4 by default; a lower
  threshold keeps more pairs).

Readings (listed in the design notes as well):

* K1 — the MLP's inner width is 512: with biases, 36 x (4096*512 + 512 +
  512*8 + 8) = 75.7M parameters, the stated "about 76M".
* K2 — both layers carry a bias (the linear default); the parameter counts
  fit with or without one.
* K3 — GELU is the exact erf form 0.5 x (1 + erf(x / sqrt 2)).
* K4 — the score of token t comes from the layer's hidden state at t as it
  is (the pages name no normalisation).
* K5 — a token is pruned when its score is below the threshold (strict: a
  tie keeps it), and only once it has left the window of the last 128
  tokens: for query position i, key j is visible iff j <= i and
  (score_j >= threshold or i - j < 128).  This is the delayed-eviction cache
  of the DMS path with the decision e_j = [score_j < threshold] and window
  128, so the paged store, the slot rule and the attention are shared.
* K6 — weights in float32 for both variants (the linear page states it; the
  MLP page gives no dtype).

Pins: ``tests/test_kvzap_oracle_pins.py``.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

THRESHOLD = -4.0        # both pages' default
WINDOW = 128            # the sliding window of the last tokens


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU (K3): x * Phi(x) with Phi the standard normal CDF."""
    x = np.asarray(x, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def scores_linear(h: np.ndarray, W: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """KVzap-linear page, 轻量级网络设计 / 工作流程: s[..., k] = W[k] . h + b[k].

    h [..., H], W [Hkv, H], b [Hkv] or None -> scores [..., Hkv]."""
    s = np.asarray(h, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
    if b is not None:
        s = s + np.asarray(b, dtype=np.float64)
    return s


def scores_mlp(h: np.ndarray, W1: np.ndarray, b1: Optional[np.ndarray], W2: np.ndarray,
               b2: Optional[np.ndarray]) -> np.ndarray:
    """KVzap-mlp page, 模型架构: s = W2 . gelu(W1 . h + b1) + b2.

    h [..., H], W1 [Hm, H], b1 [Hm], W2 [Hkv, Hm], b2 [Hkv] -> [..., Hkv]."""
    z = scores_linear(h, W1, b1)
    return scores_linear(gelu(z), W2, b2)


def decisions(scores: np.ndarray, threshold: float = THRESHOLD) -> np.ndarray:
    """Both pages' threshold step (K5): prune (1) when the score is below the
    threshold, keep (0) otherwise."""
    return (np.asarray(scores, dtype=np.float64) < threshold).astype(np.uint8)


def visible(scores_row: np.ndarray, i: int, threshold: float = THRESHOLD, w: int = WINDOW) -> np.ndarray:
    """Keys j <= i a query at position i attends to (K5): the last w tokens and
    every earlier token whose score reached the threshold."""
    s = np.asarray(scores_row, dtype=np.float64)[: i + 1]
    j = np.arange(i + 1)
    return j[(s >= threshold) | (i - j < w)]
