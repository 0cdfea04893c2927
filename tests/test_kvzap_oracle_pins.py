"""Pins of the KVzap oracle against things other than itself (CPU only).

* gelu            -> values of x * Phi(x) at 0 and +-1 from the normal CDF
                     written with math.erfc, the identity gelu(x) - gelu(-x) = x,
                     the asymptotes, and torch's exact GELU (approximate='none');
                     the tanh approximation differs by ~1e-4 and fails
* scores_linear   -> one-hot hidden states pick a column of W plus the bias;
                     torch.nn.functional.linear in float64
* scores_mlp      -> torch Linear -> GELU -> Linear in float64; a hand-worked
                     case with H = 2, Hm = 2, Hkv = 1
* decisions       -> the threshold's direction: lowering it keeps more
                     (KVzap-mlp page, 高级配置); a tie keeps
* visible         -> the DMS cache model fed e = decisions(scores) with window
                     128 holds exactly the keys `visible` lists (brute force
                     over every position), and the window keeps the last 128
A dropped bias, a transposed weight, the tanh GELU, a flipped comparison or an
off-by-one window fails at least one of them.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle import kvzap_oracle as kz

RNG = np.random.default_rng(97531)


def _phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def test_gelu_values_identity_asymptotes():
    assert kz.gelu(np.array(0.0)) == 0.0
    assert abs(float(kz.gelu(np.array(1.0))) - _phi(1.0)) < 1e-15
    assert abs(float(kz.gelu(np.array(-1.0))) + _phi(-1.0)) < 1e-15
    assert abs(float(kz.gelu(np.array(1.0))) - 0.8413447460685429) < 1e-15
    x = RNG.normal(0, 3, 200)
    np.testing.assert_allclose(kz.gelu(x) - kz.gelu(-x), x, rtol=0, atol=1e-13)
    assert float(kz.gelu(np.array(40.0))) == 40.0
    assert float(kz.gelu(np.array(-40.0))) == 0.0 or abs(float(kz.gelu(np.array(-40.0)))) < 1e-300
    t = torch.from_numpy(x)
    np.testing.assert_allclose(kz.gelu(x), F.gelu(t, approximate="none").numpy(), rtol=1e-14, atol=1e-15)
    tanh = F.gelu(t, approximate="tanh").numpy()
    assert np.abs(kz.gelu(x) - tanh).max() > 1e-5          # the two forms are told apart


def test_scores_linear_one_hot_and_torch():
    H, Hkv = 16, 3
    W = RNG.normal(0, 1, (Hkv, H))
    b = RNG.normal(0, 1, Hkv)
    eye = np.eye(H)
    s = kz.scores_linear(eye, W, b)
    np.testing.assert_array_equal(s, W.T + b)
    np.testing.assert_array_equal(kz.scores_linear(eye, W, None), W.T)
    h = RNG.normal(0, 1, (5, 7, H))
    ref = F.linear(torch.from_numpy(h), torch.from_numpy(W), torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(kz.scores_linear(h, W, b), ref, rtol=1e-13, atol=1e-13)


def test_scores_mlp_torch_and_hand_case():
    H, Hm, Hkv = 24, 16, 4
    W1, b1 = RNG.normal(0, 0.3, (Hm, H)), RNG.normal(0, 0.3, Hm)
    W2, b2 = RNG.normal(0, 0.3, (Hkv, Hm)), RNG.normal(0, 0.3, Hkv)
    h = RNG.normal(0, 1, (3, 9, H))
    net = torch.nn.Sequential(torch.nn.Linear(H, Hm), torch.nn.GELU(), torch.nn.Linear(Hm, Hkv)).double()
    with torch.no_grad():
        net[0].weight.copy_(torch.from_numpy(W1))
        net[0].bias.copy_(torch.from_numpy(b1))
        net[2].weight.copy_(torch.from_numpy(W2))
        net[2].bias.copy_(torch.from_numpy(b2))
        ref = net(torch.from_numpy(h)).numpy()
    np.testing.assert_allclose(kz.scores_mlp(h, W1, b1, W2, b2), ref, rtol=1e-12, atol=1e-13)
    # H = Hm = 2, Hkv = 1: z = (1*1 + 2*0 + 0.5, 1*(-1) + 2*3 - 1) = (1.5, 4)
    s = kz.scores_mlp(np.array([1.0, 2.0]), np.array([[1.0, 0.0], [-1.0, 3.0]]), np.array([0.5, -1.0]),
                      np.array([[2.0, -1.0]]), np.array([0.25]))
    want = 2.0 * 1.5 * _phi(1.5) - 4.0 * _phi(4.0) + 0.25
    assert abs(float(s[0]) - want) < 1e-14


def test_decisions_direction_and_tie():
    s = np.array([-5.0, -4.0, -3.9, -4.0000001, 10.0])
    assert list(kz.decisions(s)) == [1, 0, 0, 1, 0]
    x = RNG.normal(-4, 2, 1000)
    assert kz.decisions(x, -6.0).sum() < kz.decisions(x, -4.0).sum() < kz.decisions(x, -2.0).sum()


def test_visible_equals_cache_model_with_window_128():
    T, Hkv = 400, 2
    s = RNG.normal(-4.0, 1.5, (Hkv, T))
    e = kz.decisions(s)
    sim = oracle.CacheSim(1, Hkv, kz.WINDOW, 32, T, 64)
    for t in range(T):
        sim.append([0], e[None, :, t:t + 1])
        for kh in range(Hkv):
            held = np.sort(sim.resident_positions(0, kh))
            want = kz.visible(s[kh], t)
            assert np.array_equal(held, want), (t, kh)
    # the window keeps the last 128 whatever the scores
    low = np.full(300, -100.0)
    assert np.array_equal(kz.visible(low, 299), np.arange(172, 300))
    assert np.array_equal(kz.visible(low, 50), np.arange(51))
