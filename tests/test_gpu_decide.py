"""dms_decide with the linear adapter on prefill chunks against the CPU
oracle (needs an MI355X): the matrix-core kernel (bf16 hidden states, H a
multiple of 2048, tokens in groups of 16 with a ragged last group) and the
vector-ALU one it replaces when DMS_DECIDE_MFMA=0 or H is not a multiple of
2048.  Decisions bit for bit (hidden rows whose logit lies within 1e-2 of the
threshold for some head are redrawn, so that rounding cannot flip one),
logits within 5e-3.  Shapes: head and layer mode, with and without bias,
4 and 8 KV heads, up to the 4096 x 4096 chunk of the 32K prefill.
"""
import numpy as np
import pytest

import oracle
from learned_kv_cache_amd import synth

pytestmark = pytest.mark.gpu

# name: (B, T, H, Hkv, alpha_per, bias)
CASES = {
    "h2048_kv8_ragged": (2, 999, 2048, 8, "head", False),
    "h2048_kv4_layer_bias": (1, 777, 2048, 4, "layer", True),
    "h4096_kv8_chunk4096": (1, 4096, 4096, 8, "head", False),
    "h3072_kv8_vector_only": (1, 600, 3072, 8, "head", True),
    "h1024_kv2_vector_only": (3, 300, 1024, 2, "head", False),
}


def _draw(case, seed):
    B, T, H, Hkv, per, use_bias = CASES[case]
    rng = np.random.default_rng(seed)
    h = synth.as_dtype(rng.standard_normal((B, T, H), dtype=np.float32), "bf16").astype(np.float64)
    gamma = (1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    W = (rng.standard_normal((Hkv, H)) / np.sqrt(H)).astype(np.float32)
    bias = (0.05 * rng.standard_normal(Hkv)).astype(np.float32) if use_bias else None
    offsets = (5.0 + rng.uniform(-20, 20, Hkv)).astype(np.float32)
    kw = dict(alpha_scale=100.0, eps=1e-6, bias=bias, alpha_per=per)
    for _ in range(20):
        lg, _ = oracle.decide_linear(h, gamma, W, offsets, **kw)
        near = np.abs(lg) < 1e-2                       # [B, Hkv, T]
        bad = np.argwhere(near.any(axis=1))            # (b, t)
        if len(bad) == 0:
            break
        for b, t in bad:
            h[b, t] = synth.as_dtype(rng.standard_normal(H, dtype=np.float32), "bf16")
    else:
        raise AssertionError("could not clear the threshold margin")
    lg, ev = oracle.decide_linear(h, gamma, W, offsets, **kw)
    return h, gamma, W, bias, offsets, lg, ev


@pytest.mark.parametrize("mfma", ["1", "0"])
@pytest.mark.parametrize("case", list(CASES))
def test_decide_linear_chunk(case, mfma, monkeypatch):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from learned_kv_cache_amd import dms
    monkeypatch.setenv("DMS_DECIDE_MFMA", mfma)
    B, T, H, Hkv, per, use_bias = CASES[case]
    h, gamma, W, bias, offsets, ref_l, ref_e = _draw(case, 7 + list(CASES).index(case))
    cfg = dms.make_config(max_batch=B, num_q_heads=Hkv * 2, num_kv_heads=Hkv, head_dim=64, hidden=H, window=16,
                          block_size=8, max_tokens_per_seq=T, pool_pages=64, max_chunk=min(T, 8192),
                          kv_dtype="bf16", decide_mode="linear", alpha_per=per)
    cache = dms.DmsCache(cfg)
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    logits = torch.empty(B * Hkv * T, dtype=torch.float32, device="cuda")
    evict = torch.empty(B * Hkv * T, dtype=torch.uint8, device="cuda")
    dms.dms_decide(cache, dev(h, torch.bfloat16), dev(gamma, torch.float32), dev(W, torch.float32),
                   None if bias is None else dev(bias, torch.float32), dev(offsets, torch.float32), None, B, T,
                   logits, evict)
    got_e = evict.cpu().numpy().reshape(B, Hkv, T)
    got_l = logits.cpu().numpy().reshape(B, Hkv, T)
    assert np.array_equal(got_e, ref_e), f"decisions differ at {np.argwhere(got_e != ref_e)[:5]}"
    np.testing.assert_allclose(got_l, ref_l, atol=5e-3, rtol=0)
