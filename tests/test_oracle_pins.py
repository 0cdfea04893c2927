"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it pins and why a plausible mistake in the oracle (a
dropped term, a wrong sign or index, a transposed operand, an off-by-one in
the window) would fail it:

* decide_linear  -> torch rms_norm + linear (library routines, float64)
* decide_qneuron -> closed form e = [q > o / a] and the zeroed neuron
* attention_rows -> torch SDPA (causal, when nothing is evicted / window >= T;
                    banded sliding window, when everything is evicted)
* CacheSim       -> closed-form lengths; brute force over every decision
                    vector of tiny cases (occupants == visible set, no holes,
                    pages == ceil(L / P)); attention over the simulated slots
                    equals the masked definition; chunk-size invariance
* e4m3           -> all 256 codes, ties, saturation vs torch.float8_e4m3fn
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from learned_kv_cache_amd import synth

RNG = np.random.default_rng(12345)


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


# ---------------------------------------------------------------------------
# decisions

@pytest.mark.parametrize("B,T,H,Hkv", [(2, 5, 256, 2), (1, 3, 4096, 8)])
def test_decide_linear_matches_torch_rmsnorm_linear(B, T, H, Hkv):
    h = RNG.standard_normal((B, T, H))
    gamma = RNG.uniform(0.5, 1.5, H)
    W = RNG.normal(0, 1 / math.sqrt(H), (Hkv, H))
    off = RNG.uniform(-3, 3, Hkv)
    logits, evict = oracle.decide_linear(h, gamma, W, off, alpha_scale=100.0, eps=1e-6)
    x = F.rms_norm(torch.from_numpy(h), (H,), weight=torch.from_numpy(gamma), eps=1e-6)
    ref = (F.linear(x, torch.from_numpy(W)) * 100.0 - torch.from_numpy(off)).permute(0, 2, 1).numpy()
    np.testing.assert_allclose(logits, ref, rtol=1e-12, atol=1e-10)
    assert np.array_equal(evict, (ref > 0).astype(np.uint8))


def test_decide_linear_layer_mode_and_disable():
    h = RNG.standard_normal((2, 7, 64))
    W = RNG.normal(0, 0.2, (4, 64))
    off = np.array([0.3, -1.0, 2.0, 0.0])
    lh, eh = oracle.decide_linear(h, np.ones(64), W, off, alpha_scale=100.0, eps=1e-6)
    ll, el = oracle.decide_linear(h, np.ones(64), W, off, alpha_scale=100.0, eps=1e-6, alpha_per="layer")
    for k in range(4):   # every head takes head 0's decision
        assert np.array_equal(el[:, k], eh[:, 0])
        np.testing.assert_array_equal(ll[:, k], lh[:, 0])
    _, ed = oracle.decide_linear(h, np.ones(64), W, off, alpha_scale=100.0, eps=1e-6, disable_eviction=True)
    assert ed.sum() == 0
    with pytest.raises(ValueError):
        oracle.decide_linear(h, np.ones(64), W, off, alpha_scale=100.0, eps=1e-6, alpha_per="token")


def test_decide_linear_zero_adapter_keeps_everything():
    # Zeroed adapter weights (the training start state) with a positive offset: logit = -offset < 0.
    h = RNG.standard_normal((1, 9, 32))
    _, e = oracle.decide_linear(h, np.ones(32), np.zeros((2, 32)), np.array([5.0, 5.0]),
                                alpha_scale=100.0, eps=1e-6)
    assert e.sum() == 0


def test_decide_qneuron_closed_form():
    B, T, Hq, Hkv, D = 2, 11, 8, 2, 16
    q = synth.round_bf16(RNG.standard_normal((B, T, Hq, D)).astype(np.float32))
    off = np.array([5.0, 2.0])
    logits, e, qz = oracle.decide_qneuron(q, off, num_kv_heads=Hkv, alpha_scale=100.0)
    g = Hq // Hkv
    for b, t, k in itertools.product(range(B), range(T), range(Hkv)):
        val = float(q[b, t, k * g, D - 1])
        assert e[b, k, t] == (1 if val > off[k] / 100.0 else 0)
        assert logits[b, k, t] == pytest.approx(100.0 * val - off[k], abs=1e-9)
    # only the first query head of each group loses its last element
    changed = (qz != q.astype(np.float64))
    assert not changed[..., :-1].any()
    for h in range(Hq):
        if h % g:
            assert not changed[:, :, h, -1].any()
        else:
            assert (qz[:, :, h, -1] == 0).all()
    _, el, _ = oracle.decide_qneuron(q, off, num_kv_heads=Hkv, alpha_scale=100.0, alpha_per="layer")
    assert np.array_equal(el[:, 1], e[:, 0])


# ---------------------------------------------------------------------------
# attention

@pytest.mark.parametrize("Hq,Hkv,D,T", [(4, 2, 32, 40), (8, 8, 16, 23), (6, 1, 8, 17)])
def test_no_eviction_is_causal_attention(Hq, Hkv, D, T):
    q = RNG.standard_normal((T, Hq, D))
    k = RNG.standard_normal((T, Hkv, D))
    v = RNG.standard_normal((T, Hkv, D))
    scale = 1 / math.sqrt(D)
    ref = _sdpa(q, k, v, causal=True, scale=scale)
    e0 = np.zeros((Hkv, T), np.uint8)
    out = oracle.attention_rows(q, k, v, e0, w=4, rows=np.arange(T), scale=scale)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    # any decisions at all are irrelevant when the window covers the sequence
    er = (RNG.random((Hkv, T)) < 0.7).astype(np.uint8)
    out = oracle.attention_rows(q, k, v, er, w=T, rows=np.arange(T), scale=scale)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("w,T", [(1, 12), (3, 20), (8, 33)])
def test_all_evicted_is_sliding_window_attention(w, T):
    Hq, Hkv, D = 4, 2, 8
    q = RNG.standard_normal((T, Hq, D))
    k = RNG.standard_normal((T, Hkv, D))
    v = RNG.standard_normal((T, Hkv, D))
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    band = (j <= i) & (j > i - w)
    ref = _sdpa(q, k, v, mask=band, scale=0.3)
    out = oracle.attention_rows(q, k, v, np.ones((Hkv, T), np.uint8), w=w, rows=np.arange(T), scale=0.3)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_qneuron_attention_uses_zeroed_query():
    T, Hq, Hkv, D = 30, 4, 2, 16
    q = RNG.standard_normal((1, T, Hq, D))
    k = RNG.standard_normal((T, Hkv, D))
    v = RNG.standard_normal((T, Hkv, D))
    _, e, qz = oracle.decide_qneuron(q, np.array([0.0, 0.0]), num_kv_heads=Hkv, alpha_scale=100.0,
                                     disable_eviction=True)
    ref = _sdpa(qz[0], k, v, causal=True, scale=0.25)
    out = oracle.attention_rows(qz[0], k, v, e[0], w=4, rows=np.arange(T), scale=0.25)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# paged store

def _run_tokenwise(sim, e_bkt, seq_ids):
    B, Hkv, T = e_bkt.shape
    for t in range(T):
        sim.append(seq_ids, e_bkt[:, :, t:t + 1])


@pytest.mark.parametrize("w,P", [(2, 1), (3, 1), (3, 2), (4, 1), (4, 2), (4, 3)])
def test_brute_force_every_decision_vector(w, P):
    T = 10
    D = 3
    kv = RNG.standard_normal((T, 2, D))
    qv = RNG.standard_normal(D)
    for bits in range(1 << T):
        e = np.array([(bits >> t) & 1 for t in range(T)], dtype=np.uint8)
        sim = oracle.CacheSim(1, 1, w, P, max_tokens=T, pool_pages=T)
        for t in range(T):
            sim.append([0], e[None, None, t:t + 1])
            resident = sim.resident_positions(0, 0)
            vis = np.flatnonzero(oracle.visible(e[: t + 1], t, w))
            assert np.array_equal(resident, vis), (bits, t)
            L = sim.L[0][0]
            assert L == len(vis) == oracle.length_closed_form(e, t, w)
            occ = sim.slot_table(0, 0)
            assert len(set(occ.tolist())) == L            # no hole, no double occupancy
            assert len(sim.pages[0][0]) == -(-L // P)
        if bits % 97 == 0:
            # attention over whatever order the slots hold == masked definition
            occ = sim.slot_table(0, 0)
            got = oracle.attention_over_keys(qv, kv[occ, 0], kv[occ, 1], 0.7)
            ref = oracle.attention_rows(qv[None, None], kv[:, :1], kv[:, 1:], e[None], w,
                                        rows=[T - 1], scale=0.7)[0, 0]
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_lengths_match_closed_form_and_compression():
    B, Hkv, T, w, P = 3, 4, 300, 16, 8
    e = (RNG.random((B, Hkv, T)) < np.array([0.2, 0.5, 0.8, 0.95])[None, :, None]).astype(np.uint8)
    sim = oracle.CacheSim(B, Hkv, w, P, max_tokens=T, pool_pages=B * Hkv * (T // P + 1))
    for t in range(T):
        sim.append([0, 1, 2], e[:, :, t:t + 1])
        for b, k in itertools.product(range(B), range(Hkv)):
            assert sim.L[b][k] == oracle.length_closed_form(e[b, k], t, w)
    st = sim.stats()
    assert st["tokens"] == B * Hkv * T
    assert st["live_slots"] == sum(oracle.length_closed_form(e[b, k], T - 1, w)
                                   for b in range(B) for k in range(Hkv))
    closed = e.sum()
    assert st["token_cr"] == pytest.approx(1.0 / (1.0 - closed / (B * Hkv * T)))
    assert st["cache_cr"] == pytest.approx(B * Hkv * T / st["live_slots"])


def test_chunk_size_invariance_of_slot_tables():
    B, Hkv, T, w, P = 2, 3, 200, 16, 8
    e = (RNG.random((B, Hkv, T)) < 0.6).astype(np.uint8)
    ref = oracle.CacheSim(B, Hkv, w, P, max_tokens=T, pool_pages=400)
    _run_tokenwise(ref, e, [0, 1])
    for C in (7, 16, 64, 200):
        sim = oracle.CacheSim(B, Hkv, w, P, max_tokens=T, pool_pages=400)
        for s in range(0, T, C):
            sim.append([0, 1], e[:, :, s:s + C])
        for b, k in itertools.product(range(B), range(Hkv)):
            assert np.array_equal(sim.slot_table(b, k), ref.slot_table(b, k))
            assert sim.slot_of[b][k] == ref.slot_of[b][k]
            assert len(sim.pages[b][k]) == len(ref.pages[b][k])


def test_layer_mode_tables_identical_across_heads():
    h = RNG.standard_normal((1, 120, 32))
    W = RNG.normal(0, 0.2, (4, 32))
    _, e = oracle.decide_linear(h, np.ones(32), W, np.zeros(4), alpha_scale=100.0, eps=1e-6,
                                alpha_per="layer")
    sim = oracle.CacheSim(1, 4, 8, 4, max_tokens=120, pool_pages=200)
    sim.append([0], e[:, :, :50])
    sim.append([0], e[:, :, 50:])
    for k in range(1, 4):
        assert np.array_equal(sim.slot_table(0, k), sim.slot_table(0, 0))


def test_pool_order_reset_and_exhaustion():
    sim = oracle.CacheSim(2, 2, 4, 2, max_tokens=64, pool_pages=6)
    e = np.zeros((2, 2, 1), np.uint8)
    sim.append([0, 1], e)                      # four pairs each open a page: 0,1,2,3 in row-major order
    assert [sim.pages[b][k] for b in range(2) for k in range(2)] == [[0], [1], [2], [3]]
    sim.append([0, 1], e)
    sim.append([1], e[:1])                     # seq 1 needs pages for both heads: 4, 5
    assert sim.pages[1] == [[2, 4], [3, 5]]
    sim.reset([1])
    assert sim.free[-4:] == [5, 3, 4, 2]       # next pops: 2, 4, 3, 5
    sim.append([1], np.zeros((1, 2, 3), np.uint8))
    assert sim.pages[1] == [[2, 4], [3, 5]]
    with pytest.raises(oracle.PoolExhausted):
        sim.append([0, 1], np.zeros((2, 2, 8), np.uint8))
    with pytest.raises(oracle.CapacityExceeded):
        sim.append([0], np.zeros((1, 2, 64), np.uint8))


def test_window_must_exceed_block():
    with pytest.raises(ValueError):
        oracle.CacheSim(1, 1, 4, 4, 10, 10)
    with pytest.raises(ValueError):
        oracle.CacheSim(1, 1, 4, 0, 10, 10)


# ---------------------------------------------------------------------------
# fp8 e4m3

def test_e4m3_codes_roundtrip_and_match_torch():
    vals = np.array([oracle.e4m3_value(c) for c in range(256)])
    finite = ~np.isnan(vals)
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and finite.sum() == 254
    assert vals[0x7E] == 448.0 and vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6
    codes = np.arange(256)[finite]
    enc = oracle.e4m3_encode(vals[finite])
    # every finite code decodes and re-encodes to itself (except -0 -> +0)
    assert np.array_equal(np.where(codes == 0x80, 0, codes), enc)
    # torch's own e4m3fn bit patterns decode to the same values
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(t), np.isnan(vals))
    np.testing.assert_array_equal(t[finite], vals[finite])


def test_e4m3_rounding_ties_and_saturation_match_torch():
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = 0.5 * (pos[:-1] + pos[1:])                      # exact ties
    x = np.concatenate([mids, -mids, RNG.standard_normal(20000) * 50,
                        RNG.standard_normal(2000) * 1e-3, [448.0, 460.0, 1e4, -1e4, 0.0]])
    x = x.astype(np.float32).astype(np.float64)
    clamped = np.clip(x, -448.0, 448.0)
    ref = torch.from_numpy(clamped.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x)
    ref = np.where(ref == 0x80, 0, ref)                    # torch keeps -0; this store writes +0
    np.testing.assert_array_equal(got, ref)
    # ties go to the even code
    tie_codes = oracle.e4m3_encode(mids)
    assert (tie_codes % 2 == 0).all()


def test_page_scale_is_tight_power_of_two_with_headroom():
    for amax in np.concatenate([RNG.uniform(1e-3, 1e3, 500), [448.0, 447.99, 448.01, 1.0, 3.5, 3.5001]]):
        s = oracle.page_scale(float(amax))
        e = math.log2(s)
        assert e == int(e)
        base = s / 2 ** oracle.SCALE_HEADROOM_BINADES
        assert amax <= 448.0 * base and amax > 448.0 * base / 2


def test_fp8_page_scales_in_sim():
    B, Hkv, T, D, w, P = 1, 2, 40, 8, 4, 2
    k = RNG.standard_normal((B, T, Hkv, D))
    v = RNG.standard_normal((B, T, Hkv, D)) * 3
    e = (RNG.random((B, Hkv, T)) < 0.5).astype(np.uint8)
    sim = oracle.CacheSim(B, Hkv, w, P, max_tokens=T, pool_pages=64, fp8=True)
    sim.append([0], e[:, :, :30], k[:, :30], v[:, :30])
    for t in range(30, T):
        sim.append([0], e[:, :, t:t + 1], k[:, t:t + 1], v[:, t:t + 1])
    for kh in range(Hkv):
        for page_idx, page in enumerate(sim.pages[0][kh]):
            sk, sv = sim.page_scale[page]
            assert math.log2(sk) == int(math.log2(sk))
        # every resident token is stored with its page's scale and is exactly representable
        for t in sim.resident_positions(0, kh):
            sk, sv = sim.tok_scale[0][kh][t]
            slot = sim.slot_of[0][kh][t]
            page = sim.pages[0][kh][slot // P]
            assert (sk, sv) == sim.page_scale[page]
            kk = oracle.effective_kv(sim, 0, kh, k[0, :, kh], 0)[t]
            assert np.array_equal(oracle.fp8_roundtrip(kk, sk), kk)


# ---------------------------------------------------------------------------
# serving accounting: worst-case pages of a continuation

def _random_sim(seed, w=6, P=4, Hkv=2, T=37, p=0.5):
    rng = np.random.default_rng(seed)
    sim = oracle.CacheSim(2, Hkv, w, P, 200, 400)
    for b in range(2):
        e = (rng.random((1, Hkv, T + 5 * b)) < p).astype(np.uint8)
        sim.append([b], e)
    return sim, rng


@pytest.mark.parametrize("seed", range(6))
def test_pages_needed_worst_bounds_every_decision_and_is_reached(seed):
    import copy
    sim, rng = _random_sim(seed)
    for b in range(2):
        for n in (0, 1, 3, 6, 7, 13, 40):
            worst = oracle.pages_needed_worst(sim, b, n)
            for trial in range(8):
                e = (rng.random((1, sim.Hkv, n)) < rng.random()).astype(np.uint8) if trial else \
                    np.zeros((1, sim.Hkv, n), np.uint8)
                s2 = copy.deepcopy(sim)
                before = len(s2.free)
                if n:
                    s2.append([b], e)
                taken = before - len(s2.free)
                assert taken <= worst
                if trial == 0:
                    assert taken == worst            # all kept reaches the bound


def test_pages_needed_worst_closed_form_without_marks():
    sim = oracle.CacheSim(1, 3, 5, 4, 100, 100)
    sim.append([0], np.zeros((1, 3, 11), np.uint8))     # nothing marked: no overwrite to come
    for n in (0, 1, 5, 9, 30):
        assert oracle.pages_needed_worst(sim, 0, n) == 3 * (math.ceil((11 + n) / 4) - math.ceil(11 / 4))


def test_pages_needed_worst_hand_case():
    # w = 4, P = 2, one head: positions 0..5 with marks 1,0,1,1,0,0 (t=4, 5 overwrite 0's slot... ):
    # t=4 overwrites slot(0) (marked), t=5 takes a new slot (1 not marked) -> L = 5 after 6 tokens.
    sim = oracle.CacheSim(1, 1, 4, 2, 100, 100)
    sim.append([0], np.array([[[1, 0, 1, 1, 0, 0]]], np.uint8))
    assert sim.L[0][0] == 5
    # next tokens t = 6, 7, 8, 9 look at 2, 3, 4, 5: marked, marked, kept, kept -> 2 new slots for n = 4
    # L 5 -> 7 slots: pages ceil(7/2) - ceil(5/2) = 4 - 3 = 1
    assert oracle.pages_needed_worst(sim, 0, 4) == 1
    # n = 2: both overwrite -> no new slot
    assert oracle.pages_needed_worst(sim, 0, 2) == 0
    # n = 6: t = 10, 11 look at the new tokens 6, 7 (worst case kept) -> 4 new slots: ceil(9/2) - 3 = 2
    assert oracle.pages_needed_worst(sim, 0, 6) == 2
    # capacity
    assert oracle.pages_needed_worst(sim, 0, 95) == -1


def _rows(mags, D=4):
    """[T, D] rows whose largest magnitude is mags[t] (held by one element, the
    others smaller), alternating signs so the amax is taken over |x|."""
    out = np.zeros((len(mags), D))
    for t, m in enumerate(mags):
        out[t] = [m * 0.25, -m * 0.5, (-1) ** t * m, m * 0.125]
    return out


def test_fp8_page_scale_rule_hand_worked():
    _check_fp8_page_scale_rule(oracle.CacheSim)


def _check_fp8_page_scale_rule(sim_cls):
    """Which values set a fresh page's K and V scale (reading R19; the pages only say
    FP8 storage follows eviction — FastDMS post, FP8 compact KV).

    Window 3, block 2, one sequence, two heads.  First call, six tokens; head 0
    marks token 0 only:
      t0 -> slot 0 (opens page 0), t1 -> slot 1, t2 -> slot 2 (opens page 1),
      t3 overwrites slot 0 in place (token 0 was marked), t4 -> slot 3,
      t5 -> slot 4 (opens page 2).
    Final occupants: page 0 = {t3, t1}, page 1 = {t2, t4}, page 2 = {t5}.
    Token 0 was written and overwritten inside the call, so its huge K (1000)
    must not set page 0's scale.  Head 1 keeps everything: pages 3, 4, 5.
    Scale = 4 * (smallest power of two s with amax <= 448 s):
      page 0: K amax max(3, 10) = 10   -> s 2^-5 -> 2^-3;  V amax max(200, 1) = 200 -> 2^-1 -> 2
              (with token 0 counted K would be 16; with K and V swapped K would be 2)
      page 1: K amax 0.7 -> 2^-9 -> 2^-7;                 V amax 50 -> 2^-3 -> 2^-1
      page 2: K amax 448 -> 1 -> 4 (exactly at the bound); V amax 448.01 -> 2 -> 8
      head 1: K amax 1 -> 2^-8 -> 2^-6;                   V amax 2 -> 2^-7 -> 2^-5
    Second call (one token, t6, head 0): token 3 (w back) is kept, so t6 takes
    slot 5 of page 2 and reuses page 2's scales (4, 8) although its K is 5000
    (saturates); head 1 opens page 6 in that call.  Third call (t7): head 0's
    slot 6 opens page 7, with scales from t7 alone.
    """
    w, P, Hkv, D = 3, 2, 2, 4
    sim = sim_cls(1, Hkv, w, P, max_tokens=16, pool_pages=32, fp8=True)
    k = np.zeros((1, 6, Hkv, D))
    v = np.zeros((1, 6, Hkv, D))
    k[0, :, 0] = _rows([1000.0, 3.0, 0.3, 10.0, 0.7, 448.0])
    v[0, :, 0] = _rows([0.5, 200.0, 50.0, 1.0, 5.0, 448.01])
    k[0, :, 1] = _rows([1.0] * 6)
    v[0, :, 1] = _rows([2.0] * 6)
    e = np.zeros((1, Hkv, 6), np.uint8)
    e[0, 0, 0] = 1
    sim.append([0], e, k, v)
    assert sim.pages[0][0] == [0, 1, 2] and sim.pages[0][1] == [3, 4, 5]
    assert sim.slot_table(0, 0).tolist() == [3, 1, 2, 4, 5]
    assert sim.page_scale[0] == (2.0 ** -3, 2.0)
    assert sim.page_scale[1] == (2.0 ** -7, 0.5)
    assert sim.page_scale[2] == (4.0, 8.0)
    for pg in (3, 4, 5):
        assert sim.page_scale[pg] == (2.0 ** -6, 2.0 ** -5)
    # what attention reads: K through the K scale, V through the V scale
    kk = oracle.effective_kv(sim, 0, 0, k[0, :, 0], 0)
    vv = oracle.effective_kv(sim, 0, 0, v[0, :, 0], 1)
    # t1's V element -200 / 2 = -100 lies halfway between the e4m3 values 96 and 104:
    # ties go to the even code (96), so the stored value is -192; with the K scale
    # (1/8) it would saturate at -448 / 8 = -56.
    assert vv[1, 2] == -192.0
    # t3's K element 10 / 2^-3 = 80 is exact in e4m3
    assert kk[3, 2] == -10.0
    # t2's K element 0.3 through 2^-7: 38.4 -> nearest e4m3 value 40 -> 0.3125
    # (through page 1's V scale 1/2 it would be 0.3 / 0.5 = 0.6 -> 0.625 * 0.5 = 0.3125 too,
    # which is why the V check above carries the swap test)
    assert kk[2, 2] == 0.3125
    # second call: t6 into slot 5 of page 2 with page 2's scales, K saturates at 448 * 4
    k6 = np.zeros((1, 1, Hkv, D))
    v6 = np.zeros((1, 1, Hkv, D))
    k6[0, 0, 0] = _rows([5000.0])[0]
    v6[0, 0, 0] = _rows([1.0])[0]
    k6[0, 0, 1] = _rows([1.0])[0]
    v6[0, 0, 1] = _rows([2.0])[0]
    sim.append([0], np.zeros((1, Hkv, 1), np.uint8), k6, v6)
    assert sim.slot_of[0][0][6] == 5 and sim.pages[0][0] == [0, 1, 2]
    assert sim.page_scale[2] == (4.0, 8.0)
    assert sim.tok_scale[0][0][6] == (4.0, 8.0)
    # head 1 opened page 6 (slot 6 of a kept-everything head) from its own values
    assert sim.pages[0][1] == [3, 4, 5, 6] and sim.page_scale[6] == (2.0 ** -6, 2.0 ** -5)
    full_k = np.concatenate([k[0, :, 0], k6[0, :, 0]])
    assert oracle.effective_kv(sim, 0, 0, full_k, 0)[6, 2] == 1792.0
    # third call: t7 takes slot 6 of head 0, opening page 7, scales from t7 alone
    k7 = np.zeros((1, 1, Hkv, D))
    v7 = np.zeros((1, 1, Hkv, D))
    k7[0, 0, 0] = _rows([0.05])[0]
    v7[0, 0, 0] = _rows([9.0])[0]
    k7[0, 0, 1] = _rows([1.0])[0]
    v7[0, 0, 1] = _rows([2.0])[0]
    sim.append([0], np.zeros((1, Hkv, 1), np.uint8), k7, v7)
    assert sim.pages[0][0] == [0, 1, 2, 7]
    # 0.05 / 448 -> s 2^-13 -> 2^-11;  9 / 448 -> 2^-5 -> 2^-3
    assert sim.page_scale[7] == (2.0 ** -11, 2.0 ** -3)


class _AllWrittenAmax(oracle.CacheSim):
    """Planted mistake: a fresh page's amax over every token the call placed in
    it, including those overwritten later in the same call."""

    def _set_scales(self, seq_ids, new_pages, written, k, v):
        T = k.shape[1]
        every = []
        for row, b in enumerate(seq_ids):
            s0 = self.pos[b] - T
            for kh in range(self.Hkv):
                for t in range(s0, s0 + T):
                    every.append((row, b, kh, t, self.slot_of[b][kh][t]))
        super()._set_scales(seq_ids, new_pages, every, k, v)


class _SwappedKV(oracle.CacheSim):
    """Planted mistake: K and V amax exchanged."""

    def _set_scales(self, seq_ids, new_pages, written, k, v):
        super()._set_scales(seq_ids, new_pages, written, v, k)


@pytest.mark.parametrize("mutant", [_AllWrittenAmax, _SwappedKV])
def test_fp8_page_scale_pin_rejects_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _check_fp8_page_scale_rule(mutant)
