"""CPU oracle for the training-mode forward of DMS (test infrastructure only).

TEST INFRASTRUCTURE ONLY, like ``dms_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may import it;
it shares no code with the HIP library.  float64 throughout.

Follows the DMS walkthrough ("基于 DMS 的 KV Cache 压缩实战：为 Qwen3-8B 训练驱逐适配器"),
sections Gumbel 噪声与可微门控 (the noisy, tempered sigmoid gate and its
straight-through decision) and 注意力 / 训练模式 (the score_mod of the soft
eviction: within the sliding window a score is kept, beyond it the key's
log(1 - alpha) = logsigmoid(-logit) is added; non-causal pairs get the mask
value -50000).

Readings (listed in the design notes as well):

* T1 — the logit fed to logsigmoid is the gate's tempered noisy logit
  y = (logit + noise) / tau, so that exp(penalty) = 1 - sigmoid(y) = 1 - the
  gate's soft probability.  The pages' "shift the decision logits by one"
  is a re-indexing of y along the key axis done by the caller (R2: training
  only, its direction is garbled on the page); these functions take y
  already aligned to the keys.
* T2 — the straight-through decision's forward value is [sigmoid(y) > 1/2],
  taken as [y > 0] (the same set, without a rounding of the sigmoid deciding).
* T3 — the window test is q_idx - k_idx < w, as at inference (R1).

Backward: ``train_attention_backward`` (the gradients of the forward for an
upstream output gradient; pinned by central finite differences of
``train_attention`` and by torch autograd of a torch restatement).

Pins: ``tests/test_train_oracle_pins.py``.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

MASK_VALUE = -50000.0     # the walkthrough's causal mask value


def logsigmoid(x: np.ndarray) -> np.ndarray:
    """log(sigmoid(x)) = -log(1 + exp(-x)), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0.0, -np.log1p(np.exp(-np.abs(x))), x - np.log1p(np.exp(-np.abs(x))))


def train_gate(logits: np.ndarray, noise: Optional[np.ndarray], tau: float):
    """Walkthrough, Gumbel 噪声与可微门控: y = (logits + noise) / tau;
    probs = sigmoid(y); the straight-through decision's forward value (T2).

    Returns (y, probs, hard), float64."""
    lg = np.asarray(logits, dtype=np.float64)
    y = (lg + (0.0 if noise is None else np.asarray(noise, dtype=np.float64))) / float(tau)
    probs = 1.0 / (1.0 + np.exp(-y))
    hard = (y > 0.0).astype(np.float64)
    return y, probs, hard


def train_gate_backward(logits: np.ndarray, noise: Optional[np.ndarray], tau: float,
                        dy: Optional[np.ndarray] = None, dhard: Optional[np.ndarray] = None,
                        dprobs: Optional[np.ndarray] = None) -> np.ndarray:
    """Gradient to the decision logits of train_gate (walkthrough, Gumbel
    噪声与可微门控).  y = (logits + noise) / tau reaches the loss directly (the
    training attention's penalty, gradient dy), through probs = sigmoid(y)
    (gradient dprobs) and through the straight-through decision, whose forward
    value is the hard threshold and whose gradient is that of probs (reading
    T4; gradient dhard).  So
        dlogits = (dy + (dhard + dprobs) * probs * (1 - probs)) / tau.
    A missing gradient is zero.  float64."""
    y, probs, _ = train_gate(logits, noise, tau)
    g = np.zeros_like(y)
    if dy is not None:
        g = g + np.asarray(dy, dtype=np.float64)
    via_probs = np.zeros_like(y)
    if dhard is not None:
        via_probs = via_probs + np.asarray(dhard, dtype=np.float64)
    if dprobs is not None:
        via_probs = via_probs + np.asarray(dprobs, dtype=np.float64)
    return (g + via_probs * probs * (1.0 - probs)) / float(tau)


def _scored(q_rows: np.ndarray, kk: np.ndarray, pen: np.ndarray, rows: np.ndarray, w: int, scale: float) -> np.ndarray:
    """score_mod of the walkthrough's training mode for query positions `rows`
    against all T keys of one (sequence, head): [R, T] float64."""
    T = kk.shape[0]
    score = scale * (q_rows @ kk.T)                                   # [R, T]
    q_idx = rows[:, None]
    k_idx = np.arange(T)[None, :]
    causal = (q_idx >= k_idx).astype(np.float64)
    within = (q_idx - k_idx < w).astype(np.float64)
    modified = within * score + (1.0 - within) * (pen[None, :] + score)
    return (1.0 - causal) * MASK_VALUE + causal * modified


def train_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, y: np.ndarray, w: int,
                    scale: Optional[float] = None, rows: Optional[Sequence[int]] = None
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """Training-mode soft-eviction attention (walkthrough, 训练模式).

    q [B, T, Hq, D], k and v [B, T, Hkv, D], y [B, Hkv, T] (gate logits of the
    keys, T1); query head h uses KV head h // (Hq // Hkv).  Each score is
    score_mod(scale * <q_i, k_j>) with the key's penalty logsigmoid(-y_j);
    softmax over all keys (the -50000 entries carry zero weight).

    Returns (out [B, R, Hq, D], lse [B, Hq, R]) for the query positions `rows`
    (default: all T); lse is the natural log of the softmax normaliser."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    out = np.zeros((B, R, Hq, D))
    lse = np.zeros((B, Hq, R))
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            pen = logsigmoid(-y[b, kv])
            s = _scored(q[b, rows, h], k[b, :, kv], pen, rows, w, scale)
            mx = s.max(axis=1, keepdims=True)
            e = np.exp(s - mx)
            den = e.sum(axis=1, keepdims=True)
            out[b, :, h] = (e @ v[b, :, kv]) / den
            lse[b, h] = (mx + np.log(den))[:, 0]
    return out, lse


def train_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, y: np.ndarray, w: int,
                             dout: np.ndarray, scale: Optional[float] = None):
    """Gradients of the training-mode attention (walkthrough, 训练模式) for an
    upstream gradient dout of its output.

    With s_ij the modified score and P = softmax_j(s): dP = dO V^T,
    dS = P * (dP - rowsum(dO * O)), dq_i = scale * sum_j dS_ij k_j,
    dk_j = scale * sum_i dS_ij q_i, dv_j = sum_i P_ij dO_i (the last two summed
    over the query heads that share the KV head), and, as key j's penalty
    logsigmoid(-y_j) enters every score with i - j >= w (i >= j),
    dy_j = -sigmoid(y_j) * sum over those (i, head) of dS_ij.  The -50000
    entries are constants.

    Shapes as in train_attention; dout like q.  Returns (dq, dk, dv, dy),
    float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(T)
    q_idx = rows[:, None]
    k_idx = rows[None, :]
    penalised = ((q_idx >= k_idx) & (q_idx - k_idx >= w)).astype(np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dy = np.zeros_like(y)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            pen = logsigmoid(-y[b, kv])
            s = _scored(q[b, :, h], k[b, :, kv], pen, rows, w, scale)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            o = p @ v[b, :, kv]
            dp = dout[b, :, h] @ v[b, :, kv].T
            delta = (dout[b, :, h] * o).sum(axis=1, keepdims=True)
            ds = p * (dp - delta)
            dq[b, :, h] = scale * (ds @ k[b, :, kv])
            dk[b, :, kv] += scale * (ds.T @ q[b, :, h])
            dv[b, :, kv] += p.T @ dout[b, :, h]
            dy[b, kv] += (ds * penalised).sum(axis=0)
    dy *= -1.0 / (1.0 + np.exp(-y))
    return dq, dk, dv, dy
