"""Pins of the training-mode oracle against things other than itself (CPU only).

* logsigmoid     -> the direct formula log(1 / (1 + e^-x)) where it is exact
                    enough, log(0.5) at 0, and the two asymptotes
* train_gate     -> torch.sigmoid; the forward decision is [logit + noise > 0]
* train_gate_backward -> central differences of train_gate's y and probs
                    (the dy and dprobs paths); torch autograd through the
                    straight-through construct hard - probs.detach() + probs
                    built with torch ops (the dhard path)
* train_attention:
    - every key kept (gate logits -> -inf: penalty 0)       -> torch SDPA causal
    - every key evicted (gate logits -> +inf: no weight past the window)
                                                            -> SDPA with a band mask
    - a hand-worked two-token case                          -> closed form
    - hard gates (penalty 0 or -inf per key)                -> the inference oracle's
      masked attention with the same decisions (pinned separately)
    - lse                                                    -> torch.logsumexp over a
      score matrix built with torch ops from the definition
  A dropped penalty, a penalty on the wrong side of the window, a wrong sign
  of y, an off-by-one window or a transposed q/k fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import dms_train_oracle as tor

RNG = np.random.default_rng(24680)


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    """torch SDPA in float64 with GQA expansion; q [T,Hq,D], k/v [T,Hkv,D]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    g = Hq // Hkv
    tq = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)[None]
    tk = torch.from_numpy(np.asarray(k, np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    tv = torch.from_numpy(np.asarray(v, np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    am = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, is_causal=causal, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_logsigmoid_values():
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(tor.logsigmoid(x), np.log(1.0 / (1.0 + np.exp(-x))), rtol=1e-12, atol=1e-13)
    assert tor.logsigmoid(np.array(0.0)) == pytest.approx(-math.log(2.0), abs=1e-15)
    # asymptotes: log sigmoid(x) ~ -e^-x for large x, ~ x for very negative x
    assert tor.logsigmoid(np.array(60.0)) == pytest.approx(-math.exp(-60.0), rel=1e-12)
    assert tor.logsigmoid(np.array(-800.0)) == pytest.approx(-800.0, rel=1e-15)
    assert np.isfinite(tor.logsigmoid(np.array([-1e6, 1e6]))).all()


def test_train_gate_matches_torch_sigmoid_and_threshold():
    logits = RNG.normal(0, 3, 1000)
    noise = RNG.logistic(0, 1, 1000)
    for tau in (0.1, 1.0):
        y, probs, hard = tor.train_gate(logits, noise, tau)
        np.testing.assert_allclose(y, (logits + noise) / tau, rtol=1e-15)
        np.testing.assert_allclose(probs, torch.sigmoid(torch.from_numpy(y)).numpy(), rtol=1e-14, atol=1e-300)
        assert np.array_equal(hard, (logits + noise > 0).astype(np.float64))
    y0, _, h0 = tor.train_gate(logits, None, 0.5)
    assert np.array_equal(h0, (logits > 0).astype(np.float64))


def test_gate_backward_matches_central_differences():
    n = 400
    logits = RNG.normal(0, 2, n)
    noise = RNG.logistic(0, 1, n)
    dy = RNG.standard_normal(n)
    dprobs = RNG.standard_normal(n)
    for tau in (0.25, 1.0, 3.0):
        got = tor.train_gate_backward(logits, noise, tau, dy=dy, dprobs=dprobs)
        # L(logits) = sum(dy * y + dprobs * probs), elementwise in the logits
        h = 1e-6

        def loss_terms(lg):
            y, p, _ = tor.train_gate(lg, noise, tau)
            return dy * y + dprobs * p
        fd = (loss_terms(logits + h) - loss_terms(logits - h)) / (2 * h)
        np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8)
    assert np.array_equal(tor.train_gate_backward(logits, noise, 1.0), np.zeros(n))


def test_gate_backward_straight_through_matches_torch_autograd():
    n = 300
    logits = RNG.normal(0, 2, n)
    noise = RNG.logistic(0, 1, n)
    dhard = RNG.standard_normal(n)
    dy = RNG.standard_normal(n)
    for tau in (0.5, 2.0):
        t = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
        y = (t + torch.from_numpy(noise)) / tau
        probs = torch.sigmoid(y)
        hard = (probs > 0.5).to(probs.dtype) - probs.detach() + probs
        (torch.from_numpy(dhard) * hard + torch.from_numpy(dy) * y).sum().backward()
        got = tor.train_gate_backward(logits, noise, tau, dy=dy, dhard=dhard)
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-12, atol=1e-15)
        # the construct's forward value is the hard decision
        assert np.array_equal(hard.detach().numpy(), tor.train_gate(logits, noise, tau)[2])


def _inputs(B, T, Hq, Hkv, D):
    q = RNG.standard_normal((B, T, Hq, D))
    k = RNG.standard_normal((B, T, Hkv, D))
    v = RNG.standard_normal((B, T, Hkv, D))
    return q, k, v


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (3, 3)])
def test_all_kept_is_causal_attention(Hq, Hkv):
    B, T, D, w = 2, 23, 8, 5
    q, k, v = _inputs(B, T, Hq, Hkv, D)
    y = np.full((B, Hkv, T), -1e6)                      # logsigmoid(1e6) = 0: no penalty
    out, _ = tor.train_attention(q, k, v, y, w)
    for b in range(B):
        np.testing.assert_allclose(out[b], _sdpa(q[b], k[b], v[b], causal=True), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("w", [1, 4, 30])
def test_all_evicted_is_sliding_window_attention(w):
    B, T, Hq, Hkv, D = 1, 19, 4, 2, 8
    q, k, v = _inputs(B, T, Hq, Hkv, D)
    y = np.full((B, Hkv, T), 1e6)                       # penalty -1e6: no weight beyond the window
    out, _ = tor.train_attention(q, k, v, y, w)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    band = (j <= i) & (i - j < w)
    np.testing.assert_allclose(out[0], _sdpa(q[0], k[0], v[0], mask=band), rtol=1e-10, atol=1e-12)


def test_two_token_closed_form():
    # one head, D = 1, w = 1: query 1 sees key 1 in the window and key 0 beyond it
    q = np.array([0.7, -1.3]).reshape(1, 2, 1, 1)
    k = np.array([1.1, 0.4]).reshape(1, 2, 1, 1)
    v = np.array([2.0, -5.0]).reshape(1, 2, 1, 1)
    y0, y1 = 0.8, -2.0
    y = np.array([y0, y1]).reshape(1, 1, 2)
    out, lse = tor.train_attention(q, k, v, y, w=1, scale=1.0)
    pen0 = -math.log(1.0 + math.exp(y0))               # log(1 - sigmoid(y0))
    s10 = -1.3 * 1.1 + pen0
    s11 = -1.3 * 0.4
    o1 = (math.exp(s10) * 2.0 + math.exp(s11) * -5.0) / (math.exp(s10) + math.exp(s11))
    assert out[0, 0, 0, 0] == pytest.approx(2.0, abs=1e-15)          # query 0: key 0 only
    assert out[0, 1, 0, 0] == pytest.approx(o1, rel=1e-13)
    assert lse[0, 0, 0] == pytest.approx(0.7 * 1.1, rel=1e-13)
    assert lse[0, 0, 1] == pytest.approx(math.log(math.exp(s10) + math.exp(s11)), rel=1e-13)


def test_hard_gates_match_inference_visibility():
    B, T, Hq, Hkv, D, w = 1, 40, 4, 2, 16, 6
    q, k, v = _inputs(B, T, Hq, Hkv, D)
    e = (RNG.random((B, Hkv, T)) < 0.5).astype(np.uint8)
    y = np.where(e == 1, 1e6, -1e6)
    out, _ = tor.train_attention(q, k, v, y, w)
    rows = np.arange(T)
    ref = oracle.attention_rows(q[0], k[0], v[0], e[0], w, rows, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(out[0], ref, rtol=1e-10, atol=1e-12)


def test_lse_matches_torch_logsumexp():
    B, T, Hq, Hkv, D, w = 1, 31, 2, 1, 8, 7
    q, k, v = _inputs(B, T, Hq, Hkv, D)
    y = RNG.normal(0, 2, (B, Hkv, T))
    _, lse = tor.train_attention(q, k, v, y, w)
    scale = 1.0 / math.sqrt(D)
    tq = torch.from_numpy(q[0]).permute(1, 0, 2)                          # [Hq, T, D]
    tk = torch.from_numpy(k[0]).permute(1, 0, 2).expand(Hq, T, D)
    s = scale * torch.matmul(tq, tk.transpose(1, 2))                      # [Hq, T, T]
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    pen = F.logsigmoid(-torch.from_numpy(y[0, 0]))[None, :].expand(T, T)
    s = torch.where(i - j >= w, s + pen, s)
    s = s.masked_fill(j > i, float("-inf"))
    np.testing.assert_allclose(lse[0], torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_rows_subset_equals_full():
    B, T, Hq, Hkv, D, w = 2, 17, 4, 2, 8, 3
    q, k, v = _inputs(B, T, Hq, Hkv, D)
    y = RNG.normal(0, 2, (B, Hkv, T))
    out, lse = tor.train_attention(q, k, v, y, w)
    rows = [0, 5, 16]
    o2, l2 = tor.train_attention(q, k, v, y, w, rows=rows)
    np.testing.assert_array_equal(o2, out[:, rows])
    np.testing.assert_array_equal(l2, lse[:, :, rows])


def _loss(q, k, v, y, w, dout, scale=None):
    out, _ = tor.train_attention(q, k, v, y, w, scale=scale)
    return float((out * dout).sum())


def test_backward_matches_central_differences():
    B, T, Hq, Hkv, D, w = 1, 9, 4, 2, 4, 3
    q, k, v = _inputs(B, T, Hq, Hkv, D)
    y = RNG.normal(0, 1.5, (B, Hkv, T))
    dout = RNG.standard_normal((B, T, Hq, D))
    dq, dk, dv, dy = tor.train_attention_backward(q, k, v, y, w, dout)
    eps = 1e-6
    for name, x, gr in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("y", y, dy)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v, "y": y}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], args["y"], w, dout)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], args["y"], w, dout)
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(gr, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_matches_torch_autograd():
    B, T, Hq, Hkv, D, w = 2, 21, 4, 2, 8, 5
    q, k, v = _inputs(B, T, Hq, Hkv, D)
    y = RNG.normal(0, 2, (B, Hkv, T))
    dout = RNG.standard_normal((B, T, Hq, D))
    scale = 1.0 / math.sqrt(D)
    tq, tk, tv, ty = (torch.tensor(x, requires_grad=True) for x in (q, k, v, y))
    g = Hq // Hkv
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    outs = []
    for b in range(B):
        per_head = []
        for h in range(Hq):
            kv = h // g
            s = scale * tq[b, :, h] @ tk[b, :, kv].T
            pen = F.logsigmoid(-ty[b, kv])[None, :].expand(T, T)
            s = torch.where(i - j >= w, s + pen, s)
            s = torch.where(j > i, torch.full_like(s, -50000.0), s)
            per_head.append(torch.softmax(s, dim=-1) @ tv[b, :, kv])
        outs.append(torch.stack(per_head, dim=1))
    out = torch.stack(outs)
    (out * torch.from_numpy(dout)).sum().backward()
    dq, dk, dv, dy = tor.train_attention_backward(q, k, v, y, w, dout)
    for name, got, ref in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad), ("y", dy, ty.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_backward_no_penalty_region_gives_zero_gate_gradient():
    B, T, Hq, Hkv, D = 1, 12, 2, 1, 4
    q, k, v = _inputs(B, T, Hq, Hkv, D)
    y = RNG.normal(0, 2, (B, Hkv, T))
    dout = RNG.standard_normal((B, T, Hq, D))
    _, _, _, dy = tor.train_attention_backward(q, k, v, y, T, dout)     # window covers every pair
    assert np.array_equal(dy, np.zeros_like(dy))
