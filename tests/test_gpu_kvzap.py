"""dms_kvzap_score (the KVzap scorers) against the CPU oracle, and KVzap
decisions driving the paged cache (needs an MI355X).

Hidden states N(0, 1) rounded to bf16 (or kept in f32), weights N(0, 1/fan_in)
in f32, inner biases N(0, 0.1^2); the last bias is set per head from the
oracle's pre-bias scores so that about half of the tokens fall below the
threshold -4 (the median of the head's scores moves to the threshold).
Scores within 2e-4 absolute of the float64 oracle (fp32 accumulation over
H = 4096 terms of unit-scale products: ~1e-5); every token whose oracle score
lies within 1e-3 of the threshold for some head has its hidden row redrawn
first, so every decision compares bit for bit.
Shapes: linear with 3, 8 and 16 heads, bf16 and f32 hidden states, 1 to 2100
tokens (both workgroup shapes, ragged tails), hidden sizes 4096, 2080 (a
partial last slab of 1024 elements) and 5120 (past the slabs whose rows load
before the first product); the MLP 2080 -> 192 -> 8 at 4, 70 and 300 tokens
(ragged 32-column stages, three 64-unit groups) and the MLP 4096 -> 512 -> 8 of the
KVzap-mlp page at 1, 8, 16 tokens (the decode-size path), 17 and 600 tokens
and a 4096-token prefill chunk (the matrix-core path, ragged token tiles);
MLP scores are bit-identical from one call to the next.
End to end: a window-128 cache fed the MLP's decisions over a chunked prompt
and decode steps, attention checked against the oracle's masked attention.
"""
import math

import numpy as np
import pytest

from learned_kv_cache_amd import synth
from oracle import dms_oracle as dor
from oracle import kvzap_oracle as kz
from tests.harness import from_dev, log, to_dev

pytestmark = pytest.mark.gpu

THR = kz.THRESHOLD
SCORE_TOL = 2e-4
MARGIN = 1e-3


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _hidden(gen, shape, dtype):
    x = gen.standard_normal(shape, dtype=np.float32)
    return synth.as_dtype(x, dtype) if dtype == "bf16" else x


def _weights(gen, H, Hkv, Hm):
    if Hm == 0:
        return gen.normal(0, 1 / math.sqrt(H), (Hkv, H)).astype(np.float32), None, None, None
    W1 = gen.normal(0, 1 / math.sqrt(H), (Hm, H)).astype(np.float32)
    b1 = gen.normal(0, 0.1, Hm).astype(np.float32)
    W2 = gen.normal(0, 1 / math.sqrt(Hm), (Hkv, Hm)).astype(np.float32)
    return W1, b1, W2, None


def _oracle_scores(h, W1, b1, W2, b2):
    if W2 is None:
        return kz.scores_linear(h, W1, b1)
    return kz.scores_mlp(h, W1, b1, W2, b2)


def _calibrated_bias(h, W1, b1, W2):
    """Per-head last bias that puts the median score of these tokens at the threshold."""
    s0 = _oracle_scores(h.reshape(-1, h.shape[-1]), W1, b1 if W2 is not None else None, W2, None)
    return (THR - np.median(s0, axis=0)).astype(np.float32)


def _run(torch, h, W1, b1, W2, b2, dtype):
    from learned_kv_cache_amd import dms
    B, T, H = h.shape
    Hkv = W2.shape[0] if W2 is not None else W1.shape[0]
    hd = to_dev(h, dtype)
    ev = torch.empty(B * Hkv * T, dtype=torch.uint8, device="cuda")
    sc = torch.empty(B * Hkv * T, dtype=torch.float32, device="cuda")
    dev = lambda x: None if x is None else to_dev(x, "f32")
    dms.dms_kvzap_score(hd, dev(W1), dev(b1), ev, W2=dev(W2), b2=dev(b2), threshold=THR, scores_out=sc)
    torch.cuda.synchronize()
    return from_dev(sc).reshape(B, Hkv, T), ev.cpu().numpy().reshape(B, Hkv, T)


def _clear_of_threshold(gen, h, score, dtype):
    """Redraws (in place) the hidden row of every token whose oracle score is
    within MARGIN of the threshold for some head, until none is; returns the
    oracle scores [B, T, Hkv] of the final rows."""
    s = score(h)
    for _ in range(50):
        bad = np.abs(s - THR).min(axis=-1) < MARGIN
        if not bad.any():
            return s
        h[bad] = _hidden(gen, (int(bad.sum()), h.shape[-1]), dtype)
        s[bad] = score(h[bad][None])[0]
    raise AssertionError("margin redraw did not converge")


def _check(got_s, got_e, ref, what):
    """ref: oracle scores [B, T, Hkv], every one at least MARGIN from the threshold."""
    ref = np.transpose(ref, (0, 2, 1))
    assert np.abs(ref - THR).min() >= MARGIN
    err = np.abs(got_s - ref)
    want_e = kz.decisions(ref)
    frac = float(want_e.mean())
    log(f"{what}: score err max {err.max():.2e}; evicted {frac:.2f}")
    assert err.max() <= SCORE_TOL, (what, err.max())
    assert np.array_equal(got_e, want_e), what
    if want_e.size >= 64:
        assert 0.2 < frac < 0.8


# (B, T, Hkv, dtype, H): H 4096 as on the pages; 2080 ends in a partial
# 1024-element slab; 5120 is past the four slabs whose rows are loaded
# before the first product (the per-slab kernel)
LINEAR = [(1, 1, 8, "bf16", 4096), (2, 37, 8, "bf16", 4096), (3, 700, 8, "bf16", 4096), (1, 2100, 16, "bf16", 4096),
          (2, 45, 3, "f32", 4096), (1, 333, 16, "f32", 4096), (2, 300, 8, "bf16", 2080), (1, 200, 16, "f32", 2080),
          (2, 150, 8, "bf16", 5120), (1, 90, 16, "f32", 5120), (1, 5, 8, "bf16", 2080)]


@pytest.mark.parametrize("case", LINEAR, ids=[f"b{c[0]}_t{c[1]}_hkv{c[2]}_{c[3]}_h{c[4]}" for c in LINEAR])
def test_kvzap_linear(case):
    torch = _torch()
    B, T, Hkv, dtype, H = case
    gen = np.random.default_rng(900 + LINEAR.index(case))
    h = _hidden(gen, (B, T, H), dtype)
    W1, _, _, _ = _weights(gen, H, Hkv, 0)
    cal = _hidden(gen, (256, H), dtype)
    b1 = _calibrated_bias(cal, W1, None, None)
    ref = _clear_of_threshold(gen, h, lambda x: kz.scores_linear(x, W1, b1), dtype)
    got_s, got_e = _run(torch, h, W1, b1, None, None, dtype)
    _check(got_s, got_e, ref, f"linear {case}")


# (B, T, dtype, H, Hm): the KVzap-mlp page's 4096 -> 512 -> 8, and a hidden
# size of 2080 with an inner width of 192 (neither a power of two: ragged
# 32-column stages of h, three 64-unit groups)
MLP = [(1, 1, "bf16", 4096, 512), (8, 1, "bf16", 4096, 512), (2, 8, "bf16", 4096, 512),
       (1, 17, "bf16", 4096, 512), (2, 300, "bf16", 4096, 512), (1, 4096, "bf16", 4096, 512),
       (3, 5, "f32", 4096, 512), (1, 100, "f32", 4096, 512), (2, 4, "bf16", 2080, 192),
       (2, 150, "bf16", 2080, 192), (1, 70, "f32", 2080, 192)]


@pytest.mark.parametrize("case", MLP, ids=[f"b{c[0]}_t{c[1]}_{c[2]}_h{c[3]}_m{c[4]}" for c in MLP])
def test_kvzap_mlp(case):
    torch = _torch()
    B, T, dtype, H, Hm = case
    Hkv = 8
    gen = np.random.default_rng(950 + MLP.index(case))
    h = _hidden(gen, (B, T, H), dtype)
    W1, b1, W2, _ = _weights(gen, H, Hkv, Hm)
    cal = _hidden(gen, (256, H), dtype)
    b2 = _calibrated_bias(cal, W1, b1, W2)
    ref = _clear_of_threshold(gen, h, lambda x: kz.scores_mlp(x, W1, b1, W2, b2), dtype)
    got_s, got_e = _run(torch, h, W1, b1, W2, b2, dtype)
    _check(got_s, got_e, ref, f"mlp {case}")
    again_s, again_e = _run(torch, h, W1, b1, W2, b2, dtype)            # the shares add in a fixed order
    assert np.array_equal(again_s, got_s) and np.array_equal(again_e, got_e)


def test_kvzap_arguments():
    torch = _torch()
    from learned_kv_cache_amd import dms
    h = torch.zeros(1, 4, 100, dtype=torch.bfloat16, device="cuda")          # H not a multiple of 32
    W = torch.zeros(8, 100, device="cuda")
    ev = torch.empty(32, dtype=torch.uint8, device="cuda")
    with pytest.raises(dms.DmsError):
        dms.dms_kvzap_score(h, W, None, ev)
    h = torch.zeros(1, 4, 128, dtype=torch.bfloat16, device="cuda")
    W1 = torch.zeros(64, 128, device="cuda")
    W2 = torch.zeros(8, 64, device="cuda")
    short = torch.empty(16, dtype=torch.uint8, device="cuda")                   # the MLP's workspace is too small
    assert dms.dms_kvzap_workspace_bytes(1, 4, 8, 64) == 16 * 4 * 8 * 4
    with pytest.raises(dms.DmsError):
        dms.dms_kvzap_score(h, W1, None, ev, W2=W2, workspace=short)
    # zero tokens: nothing to do
    dms.dms_kvzap_score(torch.zeros(0, 4, 128, dtype=torch.bfloat16, device="cuda"), torch.zeros(8, 128, device="cuda"),
                        None, torch.empty(0, dtype=torch.uint8, device="cuda"))


def test_kvzap_mlp_decisions_drive_the_cache():
    """KVzap-mlp decisions into a window-128 cache: chunked prompt (prefill
    attention per chunk) then decode steps; every output row against the
    oracle's masked attention with the oracle's decisions, which the GPU's
    equal exactly (hidden rows within 1e-3 of the threshold are redrawn)."""
    torch = _torch()
    from learned_kv_cache_amd import dms
    B, T0, S, H, Hm, Hq, Hkv, D, P, C = 2, 300, 24, 256, 64, 8, 2, 128, 64, 64
    T = T0 + S
    gen = np.random.default_rng(990)
    W1 = gen.normal(0, 1 / math.sqrt(H), (Hm, H)).astype(np.float32)
    b1 = gen.normal(0, 0.1, Hm).astype(np.float32)
    W2 = gen.normal(0, 1 / math.sqrt(Hm), (Hkv, Hm)).astype(np.float32)
    b2 = _calibrated_bias(_hidden(gen, (256, H), "bf16"), W1, b1, W2)
    h = _hidden(gen, (B, T, H), "bf16")
    for _ in range(50):                                   # margin redraws (the offsets stay)
        s = kz.scores_mlp(h, W1, b1, W2, b2)
        bad = np.abs(s - THR).min(axis=-1) < MARGIN
        if not bad.any():
            break
        h[bad] = _hidden(gen, (int(bad.sum()), H), "bf16")
    assert not bad.any()
    e = np.transpose(kz.decisions(s), (0, 2, 1)).copy()          # [B, Hkv, T]
    q = _hidden(gen, (B, T, Hq, D), "bf16")
    k = _hidden(gen, (B, T, Hkv, D), "bf16")
    v = _hidden(gen, (B, T, Hkv, D), "bf16")
    cfg = dms.make_config(max_batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, hidden=H, window=kz.WINDOW,
                          block_size=P, max_tokens_per_seq=T, pool_pages=B * Hkv * math.ceil(T / P), max_chunk=C)
    cache = dms.DmsCache(cfg)
    seq = to_dev(np.arange(B, dtype=np.int32), "i32")
    W1d, b1d, W2d, b2d = (to_dev(x, "f32") for x in (W1, b1, W2, b2))
    scale = 1.0 / math.sqrt(D)
    worst = 0.0

    def score(hh):
        Bn, Tn, _ = hh.shape
        ev = torch.empty(Bn * Hkv * Tn, dtype=torch.uint8, device="cuda")
        sc = torch.empty(Bn * Hkv * Tn, dtype=torch.float32, device="cuda")
        dms.dms_kvzap_score(to_dev(hh, "bf16"), W1d, b1d, ev, W2=W2d, b2=b2d, threshold=THR, scores_out=sc)
        return ev

    def check(got, b, rows):
        nonlocal worst
        ref = dor.attention_rows(q[b, rows], k[b, : rows[-1] + 1], v[b, : rows[-1] + 1], e[b, :, : rows[-1] + 1],
                                 kz.WINDOW, rows, scale)
        err = np.abs(got - ref)
        worst = max(worst, float(err.max()))
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (b, rows[0], err.max(), err.mean())

    for s0 in range(0, T0, C):
        c = min(C, T0 - s0)
        ev = score(np.ascontiguousarray(h[:, s0:s0 + c]))
        assert np.array_equal(ev.cpu().numpy().reshape(B, Hkv, c), e[:, :, s0:s0 + c])
        qd, kd, vd = (to_dev(np.ascontiguousarray(x[:, s0:s0 + c]), "bf16") for x in (q, k, v))
        out = torch.empty_like(qd)
        dms.dms_prefill_attn(cache, seq, qd, kd, vd, ev, out, B, c)
        dms.dms_append_evict(cache, seq, kd, vd, ev, B, c)
        got = from_dev(out).reshape(B, c, Hq, D)
        for b in range(B):
            check(got[b], b, np.arange(s0, s0 + c))
    for t in range(T0, T):
        ev = score(np.ascontiguousarray(h[:, t:t + 1]))
        assert np.array_equal(ev.cpu().numpy().reshape(B, Hkv), e[:, :, t])
        kd, vd = (to_dev(np.ascontiguousarray(x[:, t:t + 1]), "bf16") for x in (k, v))
        dms.dms_append_evict(cache, seq, kd, vd, ev, B, 1)
        qd = to_dev(np.ascontiguousarray(q[:, t]), "bf16").reshape(-1)
        out = torch.empty_like(qd)
        dms.dms_decode_attn(cache, seq, qd, out, B)
        got = from_dev(out).reshape(B, Hq, D)
        for b in range(B):
            check(got[b][None], b, np.array([t]))
    assert dms.dms_cache_status(cache) == 0
    dump = dms.dms_cache_dump(cache)
    for b in range(B):
        for kh in range(Hkv):
            assert int(dump["lengths"][b, kh]) == dor.length_closed_form(e[b, kh], T - 1, kz.WINDOW)
    log(f"kvzap cache: worst attention err {worst:.2e}, lengths {dump['lengths'].tolist()} of {T}")
