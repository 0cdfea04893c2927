"""Training-mode forward (dms_train_gate, dms_train_attn_fwd) against the CPU
oracle (needs an MI355X).

Seeded bf16 Q/K/V (N(0, 1) rounded to bf16, the bits both sides use) and
float32 gate logits; the backward also takes a bf16 output gradient and is
checked against the oracle's float64 gradients (dq, dk, dv and the gate
logits') relative to each tensor's largest entry.  Attention outputs within 2e-2 max / 2e-3 mean absolute
error (bf16 inputs, bf16-rounded probabilities in P.V, fp32 accumulation);
the log-sum-exp within 4e-3 absolute (its sum runs over the same bf16-rounded
probabilities: at most 2^-9 relative).  Shapes: GQA 1/2/4, head_dim 64/128,
ragged lengths (not multiples of the 32-key block or the token tiles),
windows shorter than, equal to and longer than a block, penalties of both
signs and the two extremes (nothing evicted, everything evicted).
"""
import math

import numpy as np
import pytest

from oracle import dms_train_oracle as tor
from tests.harness import from_dev, log, to_dev

pytestmark = pytest.mark.gpu

OUT_TOL = (2e-2, 2e-3)
LSE_TOL = 4e-3


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _bf16(gen, shape):
    from learned_kv_cache_amd import synth
    return synth.as_dtype(gen.standard_normal(shape, dtype=np.float32), "bf16")


def _run(torch, q, k, v, y, w):
    from learned_kv_cache_amd import dms
    B, T, Hq, D = q.shape
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    yd = to_dev(y, "f32")
    out = torch.empty_like(qd)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device="cuda")
    dms.dms_train_attn_fwd(qd, kd, vd, yd, out, lse, window=w)
    torch.cuda.synchronize()
    return from_dev(out), from_dev(lse)


def _check(got_o, got_l, ref_o, ref_l, what):
    err = np.abs(got_o - ref_o)
    lerr = np.abs(got_l - ref_l)
    log(f"{what}: out err max {err.max():.2e} mean {err.mean():.2e}; lse err max {lerr.max():.2e}")
    assert err.max() <= OUT_TOL[0] and err.mean() <= OUT_TOL[1], (what, err.max(), err.mean())
    assert lerr.max() <= LSE_TOL, (what, lerr.max())


# (Hq, Hkv, D, T, window)
SHAPES = [
    (8, 2, 128, 333, 48),
    (8, 4, 64, 1000, 200),
    (4, 4, 128, 700, 32),
    (8, 2, 64, 97, 512),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"hq{s[0]}_hkv{s[1]}_d{s[2]}_t{s[3]}_w{s[4]}" for s in SHAPES])
def test_train_attn_fwd_shapes(shape):
    torch = _torch()
    Hq, Hkv, D, T, w = shape
    gen = np.random.default_rng(SHAPES.index(shape) + 700)
    B = 2
    q, k, v = _bf16(gen, (B, T, Hq, D)), _bf16(gen, (B, T, Hkv, D)), _bf16(gen, (B, T, Hkv, D))
    y = gen.normal(0.0, 3.0, (B, Hkv, T)).astype(np.float32)
    got_o, got_l = _run(torch, q, k, v, y, w)
    ref_o, ref_l = tor.train_attention(q, k, v, y, w)
    _check(got_o, got_l, ref_o, ref_l, f"shape {shape}")


@pytest.mark.parametrize("gate", [-40.0, 40.0])
def test_train_attn_fwd_extremes(gate):
    torch = _torch()
    Hq, Hkv, D, T, w = 8, 2, 128, 300, 64
    gen = np.random.default_rng(800)
    B = 1
    q, k, v = _bf16(gen, (B, T, Hq, D)), _bf16(gen, (B, T, Hkv, D)), _bf16(gen, (B, T, Hkv, D))
    y = np.full((B, Hkv, T), gate, dtype=np.float32)
    got_o, got_l = _run(torch, q, k, v, y, w)
    ref_o, ref_l = tor.train_attention(q, k, v, y, w)
    _check(got_o, got_l, ref_o, ref_l, f"gate {gate}")


def test_train_attn_fwd_qwen8b_4k_sampled_rows():
    """Qwen3-8B layer shape, T 4096, window 512: 48 sampled query rows per
    sequence (the last 16 among them) against the oracle."""
    torch = _torch()
    Hq, Hkv, D, T, w = 32, 8, 128, 4096, 512
    gen = np.random.default_rng(801)
    B = 2
    q, k, v = _bf16(gen, (B, T, Hq, D)), _bf16(gen, (B, T, Hkv, D)), _bf16(gen, (B, T, Hkv, D))
    y = gen.normal(0.0, 3.0, (B, Hkv, T)).astype(np.float32)
    got_o, got_l = _run(torch, q, k, v, y, w)
    rows = np.unique(np.concatenate([gen.choice(T - 16, 32, replace=False), np.arange(T - 16, T)]))
    ref_o, ref_l = tor.train_attention(q, k, v, y, w, rows=rows)
    _check(got_o[:, rows], got_l[:, :, rows], ref_o, ref_l, "qwen8b T4096")


def test_train_gate():
    torch = _torch()
    from learned_kv_cache_amd import dms
    gen = np.random.default_rng(802)
    n = 100_003
    logits = gen.normal(0.0, 3.0, n).astype(np.float32)
    noise = gen.logistic(0.0, 1.0, n).astype(np.float32)
    tau = 0.1
    ld, nd = to_dev(logits, "f32"), to_dev(noise, "f32")
    y, p, h = (torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3))
    dms.dms_train_gate(ld, nd, tau, y, p, h)
    ry, rp, rh = tor.train_gate(logits.astype(np.float64), noise.astype(np.float64), tau)
    gy, gp, gh = from_dev(y), from_dev(p), from_dev(h)
    np.testing.assert_allclose(gy, ry, rtol=2e-6, atol=1e-6)
    np.testing.assert_allclose(gp, rp, rtol=0, atol=2e-6)
    clear = np.abs(ry) > 1e-4                      # the decision is not a rounding question
    assert clear.mean() > 0.999
    assert np.array_equal(gh[clear], rh[clear])
    # no noise, tau 1: y equals the logits bit for bit
    dms.dms_train_gate(ld, None, 1.0, y, None, None)
    assert np.array_equal(from_dev(y), logits.astype(np.float64))


def test_train_gate_bwd():
    """dms_train_gate_bwd against the oracle's chain rule (pinned on the CPU by
    central differences and by torch autograd through the straight-through
    construct), every combination of present and missing gradients."""
    torch = _torch()
    from learned_kv_cache_amd import dms
    gen = np.random.default_rng(803)
    n = 100_003
    logits = gen.normal(0.0, 3.0, n).astype(np.float32)
    noise = gen.logistic(0.0, 1.0, n).astype(np.float32)
    grads = {k: gen.standard_normal(n).astype(np.float32) for k in ("dy", "dhard", "dprobs")}
    ld, nd = to_dev(logits, "f32"), to_dev(noise, "f32")
    gd = {k: to_dev(v, "f32") for k, v in grads.items()}
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    for tau in (0.1, 1.0):
        for mask in range(8):
            use = {k: bool(mask >> i & 1) for i, k in enumerate(("dy", "dhard", "dprobs"))}
            for with_noise in (True, False):
                dms.dms_train_gate_bwd(ld, nd if with_noise else None, tau, out,
                                       **{k: (gd[k] if use[k] else None) for k in use})
                ref = tor.train_gate_backward(logits.astype(np.float64),
                                              noise.astype(np.float64) if with_noise else None, tau,
                                              **{k: (grads[k].astype(np.float64) if use[k] else None) for k in use})
                got = from_dev(out)
                scale = max(1.0, float(np.abs(ref).max()))
                np.testing.assert_allclose(got, ref, rtol=1e-5, atol=2e-6 * scale)


# ---------------------------------------------------------------------------
# backward

def _bwd(torch, q, k, v, y, w, dout, scale=0.0):
    from learned_kv_cache_amd import dms
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, dout))
    yd = to_dev(y, "f32")
    out = torch.empty_like(qd)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device="cuda")
    dms.dms_train_attn_fwd(qd, kd, vd, yd, out, lse, window=w, softmax_scale=scale)
    dq = torch.empty(B, T, Hq, D, dtype=torch.float32, device="cuda")
    dk = torch.empty(B, T, Hkv, D, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    dy = torch.empty(B, Hkv, T, dtype=torch.float32, device="cuda")
    dms.dms_train_attn_bwd(qd, kd, vd, out, dod, yd, lse, dq, dk, dv, dy, window=w, softmax_scale=scale)
    torch.cuda.synchronize()
    return [from_dev(x) for x in (dq, dk, dv, dy)]


# Gradient tolerance, relative to the largest reference entry of each tensor:
# the products take bf16 operands (P, dS, and the bf16 forward output in
# delta = rowsum(dO * O)), each rounded to 2^-9 relative, so an entry's error
# is a few 2^-9 of the magnitudes summed into it: 2e-2 of the tensor's
# largest entry at most, 2e-3 on average.
GRAD_TOL = (2e-2, 2e-3)
# The largest reference entry is taken as at least GRAD_FLOOR: where every
# exact gradient vanishes (one token: P = 1 so dS = dP - delta = 0; a window
# covering every pair: no gate gradient), what is left is fp32 rounding of
# dP and delta (magnitudes below 16, so about 1e-6), far below 2e-2 * 5e-3.
GRAD_FLOOR = 5e-3


def _grad_check(what, name, got, ref, floor=GRAD_FLOOR):
    scale = max(float(np.abs(ref).max()), floor)
    err = np.abs(got - ref)
    log(f"{what} {name}: max |ref| {float(np.abs(ref).max()):.3g}, err max {err.max():.2e} mean {err.mean():.2e}")
    assert err.max() <= GRAD_TOL[0] * scale and err.mean() <= GRAD_TOL[1] * scale, (what, name)

BWD_SHAPES = [
    (8, 2, 128, 333, 48),
    (8, 4, 64, 200, 16),
    (4, 4, 128, 130, 32),
    (8, 2, 64, 97, 512),
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=[f"hq{s[0]}_hkv{s[1]}_d{s[2]}_t{s[3]}_w{s[4]}" for s in BWD_SHAPES])
def test_train_attn_bwd_shapes(shape):
    torch = _torch()
    Hq, Hkv, D, T, w = shape
    gen = np.random.default_rng(BWD_SHAPES.index(shape) + 900)
    B = 2
    q, k, v = _bf16(gen, (B, T, Hq, D)), _bf16(gen, (B, T, Hkv, D)), _bf16(gen, (B, T, Hkv, D))
    y = gen.normal(0.0, 3.0, (B, Hkv, T)).astype(np.float32)
    dout = _bf16(gen, (B, T, Hq, D))
    got = _bwd(torch, q, k, v, y, w, dout)
    ref = tor.train_attention_backward(q, k, v, y, w, dout)
    for name, g_, r_ in zip(("dq", "dk", "dv", "dgate"), got, ref):
        _grad_check(f"bwd {shape}", name, g_, r_)


# degenerate and small cases: one token; a window of one (every pair off the
# diagonal penalised); fewer tokens than one 16-row block; a non-default
# softmax scale; penalties at both extremes (nothing and everything evicted)
BWD_EDGE = [
    # (Hq, Hkv, D, T, w, scale, y mean)
    (2, 2, 64, 1, 1, 0.0, 0.0),
    (4, 1, 128, 17, 1, 0.0, 0.0),
    (1, 1, 64, 5, 3, 0.0, 0.0),
    (4, 2, 128, 70, 8, 0.05, 0.0),
    (4, 2, 64, 90, 8, 0.0, -30.0),
    (4, 2, 64, 90, 8, 0.0, 30.0),
]


@pytest.mark.parametrize("case", BWD_EDGE, ids=[f"hq{c[0]}_hkv{c[1]}_d{c[2]}_t{c[3]}_w{c[4]}_s{c[5]}_y{c[6]}"
                                               for c in BWD_EDGE])
def test_train_attn_bwd_edge_cases(case):
    torch = _torch()
    Hq, Hkv, D, T, w, scale, ym = case
    gen = np.random.default_rng(BWD_EDGE.index(case) + 950)
    B = 2
    q, k, v = _bf16(gen, (B, T, Hq, D)), _bf16(gen, (B, T, Hkv, D)), _bf16(gen, (B, T, Hkv, D))
    y = (ym + gen.normal(0.0, 3.0, (B, Hkv, T))).astype(np.float32)
    dout = _bf16(gen, (B, T, Hq, D))
    got = _bwd(torch, q, k, v, y, w, dout, scale)
    ref = tor.train_attention_backward(q, k, v, y, w, dout, scale=scale if scale > 0 else None)
    for name, g_, r_ in zip(("dq", "dk", "dv", "dgate"), got, ref):
        # at the extreme penalties the gate gradient is ~1e-9 (sigmoid(-30),
        # or P ~ e^-30): checked against its own scale, with no floor
        _grad_check(f"bwd edge {case}", name, g_, r_, 0.0 if name == "dgate" and ym != 0.0 else GRAD_FLOOR)


def test_train_attn_bwd_qwen3_8b_shape_groups():
    """The benchmarked shape (Qwen3-8B layer: B 2, T 4096, 32 query and 8 KV
    heads, D 128, window 512) in the launch configuration the benchmark times;
    every entry of two KV groups (the first sequence's first group and the
    second sequence's last) against the oracle run on those groups alone."""
    torch = _torch()
    B, T, Hq, Hkv, D, w = 2, 4096, 32, 8, 128, 512
    G = Hq // Hkv
    gen = np.random.default_rng(4096)
    q, k, v = _bf16(gen, (B, T, Hq, D)), _bf16(gen, (B, T, Hkv, D)), _bf16(gen, (B, T, Hkv, D))
    y = gen.normal(0.0, 3.0, (B, Hkv, T)).astype(np.float32)
    dout = _bf16(gen, (B, T, Hq, D))
    got = _bwd(torch, q, k, v, y, w, dout)
    for b, kv in ((0, 0), (1, Hkv - 1)):
        hs, ks = slice(kv * G, (kv + 1) * G), slice(kv, kv + 1)
        ref = tor.train_attention_backward(q[b:b + 1, :, hs], k[b:b + 1, :, ks], v[b:b + 1, :, ks],
                                           y[b:b + 1, ks], w, dout[b:b + 1, :, hs])
        mine = (got[0][b:b + 1, :, hs], got[1][b:b + 1, :, ks], got[2][b:b + 1, :, ks], got[3][b:b + 1, ks])
        for name, g_, r_ in zip(("dq", "dk", "dv", "dgate"), mine, ref):
            _grad_check(f"bwd full shape (b {b}, kv {kv})", name, g_, r_)
