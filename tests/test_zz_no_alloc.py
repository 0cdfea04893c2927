"""dms_decode_attn_noalloc (decode attention with the library's static
per-device scratch instead of a caller workspace) against dms_decode_attn with
a workspace, through the C ABI (needs an MI355X).

Two calls in a row on one cache, the second over fewer rows: each output must
equal dms_decode_attn's bit for bit (the same kernels, the same record order)
and the oracle's within 2e-2 max / 2e-3 mean absolute error.  The units are
split over several workgroups, so the partial records are used.  A call that
needs more than the 8 MiB of scratch is refused before any launch.
"""
import numpy as np
import pytest

import oracle
from learned_kv_cache_amd import synth
from tests.harness import Runner, from_dev, log, prepare, to_dev

pytestmark = pytest.mark.gpu


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _oracle_out(r, seqs, q_np):
    """The oracle's attention over each listed sequence's cache as it stands
    (the visible set of a query at its last appended position)."""
    wl = r.wl
    out = []
    for i, b in enumerate(seqs):
        t = r.sim.pos[b] - 1
        K, V = r.kv_view(b, t + 1)
        out.append(oracle.attention_rows(q_np[i][None], K, V, r.prep.evict[b][:, : t + 1], wl.window, [t],
                                         r.scale)[0])
    return np.stack(out)


def test_decode_attn_noalloc_matches_workspace_entry():
    torch = _cuda()
    from learned_kv_cache_amd import dms
    wl = synth.Workload(name="noalloc_g4_d128", cfg_id=70, B=3, hidden=256, Hq=8, Hkv=2, D=128, act_dtype="bf16",
                        kv_dtype="bf16", window=24, block=16, prefill=0, decode_steps=6, chunk=64,
                        p_range=(0.40, 0.70), ctx_range=(60, 400), decide="linear", alpha_per="head")
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    ctx = prep.draw.ctx
    for b in range(wl.B):
        s = 0
        while s < int(ctx[b]):
            n = min(64, int(ctx[b]) - s)
            r.prefill_chunk([b], s, n, attend=False)
            s += n
    for i in range(3):
        r.decode_step([0, 1, 2], [int(ctx[b]) + i for b in range(3)])
    r.check_tables()
    log(f"noalloc: lengths {[r.sim.L[b] for b in range(3)]}")
    gen = np.random.default_rng(71)
    mx, mn = 2e-2, 2e-3
    for seqs in ([2, 0, 1], [1]):                       # the second call over fewer rows
        B = len(seqs)
        q_np = synth.as_dtype(gen.standard_normal((B, wl.Hq, wl.D), dtype=np.float32), "bf16")
        q = to_dev(q_np, "bf16").reshape(-1)
        ids = to_dev(np.asarray(seqs, np.int32), "i32")
        ws = torch.empty(dms.dms_decode_workspace_bytes(r.cfg, B), dtype=torch.uint8, device="cuda")
        ref = torch.empty_like(q)
        dms.dms_decode_attn(r.cache, ids, q, ref, B, workspace=ws)
        got = torch.full_like(q, 7.0)
        dms.dms_decode_attn_noalloc(r.cache, ids, q, got, B)
        torch.cuda.synchronize()
        assert dms.dms_cache_status(r.cache) == 0
        g = from_dev(got).reshape(B, wl.Hq, wl.D)
        assert np.array_equal(g, from_dev(ref).reshape(B, wl.Hq, wl.D)), "noalloc differs from the workspace call"
        err = np.abs(g - _oracle_out(r, seqs, q_np.astype(np.float64)))
        log(f"noalloc B={B}: err max {err.max():.2e} mean {err.mean():.2e}")
        assert err.max() <= mx and err.mean() <= mn


def test_decode_attn_noalloc_refuses_more_than_its_scratch():
    torch = _cuda()
    from learned_kv_cache_amd import dms
    cfg = dms.make_config(max_batch=256, num_q_heads=64, num_kv_heads=8, head_dim=128, hidden=256, window=24,
                          block_size=16, max_tokens_per_seq=32, pool_pages=64, max_chunk=64)
    cache = dms.DmsCache(cfg)
    assert dms.dms_decode_workspace_bytes(cfg, 256) > 8 << 20
    q = torch.zeros(256 * 64 * 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(dms.DmsError) as ei:
        dms.dms_decode_attn_noalloc(cache, None, q, out, 256)
    assert ei.value.status == dms.DMS_ERR_CAPACITY and "8 MiB" in str(ei.value)
    # a call that fits runs (every head is empty: zeros)
    dms.dms_decode_attn_noalloc(cache, None, q[: 64 * 128], out[: 64 * 128], 1)
    assert float(out[: 64 * 128].float().abs().max()) == 0.0
    assert dms.dms_cache_status(cache) == 0
