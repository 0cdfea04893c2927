"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Decisions, slot tables, page tables, lengths, ring, positions and the free
stack are compared bit for bit; stored K/V page bytes bit for bit on the small
workloads; attention outputs within (2e-2 max, 2e-3 mean) abs error for bf16
and fp8 (fp32: 1e-4 / 1e-5) against the float64 oracle, with fp8 rounding
applied on the oracle side.
"""
import numpy as np
import pytest

from learned_kv_cache_amd import synth
from tests.harness import Runner, log, prepare, to_dev

pytestmark = pytest.mark.gpu


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("path", ["unfused", "prepare", "step"])
@pytest.mark.parametrize("mode", ["head", "layer", "disabled"])
def test_tiny_prefill_then_decode_every_step(mode, path):
    _cuda()
    wl = synth.TINY
    if mode == "layer":
        wl = wl.replace(alpha_per="layer")
    if mode == "disabled":
        wl = wl.replace(disable_eviction=True)
    log(f"tiny {mode}: prepare")
    prep = prepare(wl)
    r = Runner(prep)
    log(f"tiny {mode}: prefill 64")
    st = r.prefill_chunk([0], 0, 64, check_rows=64)
    log(f"tiny {mode}: prefill err {st}")
    r.check_tables(pages=True)
    for t in range(64, 128):
        r.decode_step([0], [t], fused=path == "prepare", step=path == "step")
        r.check_tables(pages=True)
    log(f"tiny {mode}: decode ok, stats {r.sim.stats()}")
    if mode == "disabled":
        assert r.sim.stats()["live_slots"] == 2 * 128
    if mode == "layer":
        assert r.sim.L[0][0] == r.sim.L[0][1]


@pytest.mark.parametrize("C", [1, 5, 16, 33])
def test_tiny_chunk_sizes_give_same_tables(C):
    _cuda()
    prep = prepare(synth.TINY)
    r = Runner(prep, max_chunk=64)
    log(f"tiny chunks C={C}")
    for s in range(0, 128, C):
        n = min(C, 128 - s)
        r.prefill_chunk([0], s, n, check_rows=n)
    r.check_tables(pages=True)


def test_tiny_reset_and_reuse():
    torch = _cuda()
    wl = synth.TINY.replace(B=3)
    prep = prepare(wl)
    r = Runner(prep, pool_pages=64)
    for s in (0, 40):
        r.prefill_chunk([0, 1, 2], s, 40, check_rows=8)
    r.check_tables()
    ids = to_dev(np.array([2, 0], np.int32), "i32")
    r.dms.dms_seq_reset(r.cache, ids, 2)
    r.sim.reset([2, 0])
    r.check_tables()
    # sequences 2 and 0 start over (reusing the same inputs from position 0)
    r.prefill_chunk([2, 0], 0, 40, check_rows=8)
    r.check_tables(pages=True)
    for t in range(40, 50):
        r.decode_step([2, 0], [t, t], fused=t % 2 == 0)
    r.decode_step([1], [80], step=True)
    r.check_tables(pages=True)
    assert r.dms.dms_cache_status(r.cache) == 0


def test_device_errors_are_sticky_and_guarded():
    torch = _cuda()
    from learned_kv_cache_amd import dms
    wl = synth.TINY
    prep = prepare(wl)
    # pool of 3 pages: the 64-token prefill needs more, so the append must stop and flag it
    r = Runner(prep, pool_pages=3)
    r.prefill_chunk([0], 0, 8, check_rows=8)        # opens one page per head (2 of 3)
    assert dms.dms_cache_status(r.cache) == 0
    k = torch.zeros(1 * 64 * wl.Hkv * wl.D, dtype=torch.float32, device="cuda")
    ev = torch.zeros(wl.Hkv * 64, dtype=torch.uint8, device="cuda")
    dms.dms_append_evict(r.cache, None, k, k, ev, 1, 64)
    st = dms.dms_cache_status(r.cache)
    assert st & dms.DMS_DEV_POOL_EXHAUSTED
    dms.dms_cache_clear_status(r.cache)
    assert dms.dms_cache_status(r.cache) == 0
    # a sequence past its preallocated capacity
    r2 = Runner(prep)
    big = torch.zeros(64 * wl.Hkv * wl.D, dtype=torch.float32, device="cuda")
    ev = torch.zeros(wl.Hkv * 64, dtype=torch.uint8, device="cuda")
    dms.dms_append_evict(r2.cache, None, big, big, ev, 1, 64)
    dms.dms_append_evict(r2.cache, None, big, big, ev, 1, 64)
    assert dms.dms_cache_status(r2.cache) == 0
    one = torch.zeros(wl.Hkv * wl.D, dtype=torch.float32, device="cuda")
    dms.dms_append_evict(r2.cache, None, one, one, ev[: wl.Hkv], 1, 1)
    assert dms.dms_cache_status(r2.cache) & dms.DMS_DEV_CAPACITY
    # an out-of-range sequence id
    r3 = Runner(prep)
    bad = to_dev(np.array([5], np.int32), "i32")
    dms.dms_append_evict(r3.cache, bad, one, one, ev[: wl.Hkv], 1, 1)
    assert dms.dms_cache_status(r3.cache) & dms.DMS_DEV_BAD_SEQ
    out = torch.empty(wl.Hq * wl.D, dtype=torch.float32, device="cuda")
    q = torch.zeros(wl.Hq * wl.D, dtype=torch.float32, device="cuda")
    dms.dms_decode_attn(r3.cache, None, q, out, 1)      # empty heads give zeros
    assert float(out.abs().max()) == 0.0
    two = torch.zeros(2 * wl.Hkv * wl.D, dtype=torch.float32, device="cuda")
    with pytest.raises(dms.DmsError) as ei:
        dms.dms_append_evict(r3.cache, None, two, two, ev[: 2 * wl.Hkv], 2, 1)   # B above max_batch
    assert ei.value.status == dms.DMS_ERR_CAPACITY


@pytest.mark.timeout(600)
def test_llama1b_prefill_8k_then_decode():
    _cuda()
    wl = synth.LLAMA1B_DECODE
    log("llama1b: prepare")
    prep = prepare(wl)
    r = Runner(prep)
    for s in (0, 4096):
        st = r.prefill_chunk([0], s, 4096, check_rows=128)
        log(f"llama1b: chunk {s} err {st}")
    r.check_tables(pages=True)
    worst = (0.0, 0.0)
    for i in range(wl.decode_steps):
        # the three paths in turn; the second of two one-launch steps runs on the
        # plan the first left
        st = r.decode_step([0], [8192 + i], fused=i % 4 == 1, step=i % 4 >= 2)
        worst = (max(worst[0], st[0]), max(worst[1], st[1]))
    r.check_tables()
    stats = r.dms.dms_cache_stats(r.cache)
    ref = r.sim.stats()
    assert stats["live_slots"] == ref["live_slots"] and stats["tokens"] == ref["tokens"]
    log(f"llama1b: decode worst err {worst}, cache cr {stats['cache_cr']:.2f}")


@pytest.mark.timeout(600)
def test_qwen8b_ctx8k_b8_decode():
    _cuda()
    wl = synth.QWEN8B_DECODE
    log("qwen8b decode: prepare")
    prep = prepare(wl)
    r = Runner(prep)
    seqs = list(range(wl.B))
    for s in (0, 4096):
        st = r.prefill_chunk(seqs, s, 4096, check_rows=16)
        log(f"qwen8b decode: prefill chunk {s} err {st}")
    r.check_tables()
    worst = (0.0, 0.0)
    for i in range(wl.decode_steps):
        # runs of three one-launch steps (the second and third on the plan the one
        # before left), then decide + append in one call and the attention
        st = r.decode_step(seqs, [8192 + i] * wl.B, fused=i % 4 == 3, step=i % 4 != 3)
        worst = (max(worst[0], st[0]), max(worst[1], st[1]))
        if i % 32 == 31:
            r.check_tables()
    log(f"qwen8b decode: worst err {worst}, stats {r.dms.dms_cache_stats(r.cache)}")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("variant", ["qneuron", "linear"])
def test_qwen8b_prefill_32k_chunked(variant):
    """Every row of the last 4096-token chunk and 1024 seeded rows (the last 8
    among them) of each earlier chunk against the oracle; decisions, slot
    tables and lengths in full; then 256 decode steps, every fourth checked."""
    _cuda()
    wl = synth.QWEN8B_PREFILL32K if variant == "qneuron" else synth.QWEN8B_PREFILL32K_LINEAR
    log(f"prefill32k {variant}: prepare")
    prep = prepare(wl)
    r = Runner(prep)
    frac = float(np.mean(prep.evict[0]))
    log(f"prefill32k {variant}: eviction fraction {frac:.3f}")
    for s in range(0, 32768, 4096):
        st = r.prefill_chunk([0], s, 4096, check_rows=1024 if s < 28672 else 4096)
        log(f"prefill32k {variant}: chunk {s} err {st}")
    r.check_tables()
    for i in range(wl.decode_steps):
        r.decode_step([0], [32768 + i], check=(i % 4 == 0), fused=i % 3 == 0, step=i % 3 == 1)
    r.check_tables()


@pytest.mark.timeout(1200)
def test_qwen8b_fp8_serving_b64():
    """Prompts of 64 sequences through fp8 pages (prefill attention checked on
    every fourth sequence, 32 seeded rows of each chunk plus its last 8), then
    256 decode steps of all 64 rows, every eighth checked row by row."""
    _cuda()
    wl = synth.QWEN8B_FP8_SERVING
    log("fp8 serving: prepare")
    prep = prepare(wl)
    r = Runner(prep)
    ctx = prep.draw.ctx
    for b in range(wl.B):
        for s in range(0, int(ctx[b]), wl.chunk):
            n = min(wl.chunk, int(ctx[b]) - s)
            check = 40 if b % 4 == 0 else None
            r.prefill_chunk([b], s, n, check_rows=check, attend=check is not None)
    log("fp8 serving: populated")
    r.check_tables()
    seqs = list(range(wl.B))
    for i in range(wl.decode_steps):
        st = r.decode_step(seqs, [int(ctx[b]) + i for b in seqs], check=(i % 8 == 0), fused=i % 2 == 1,
                           step=i % 2 == 0)
        if st:
            log(f"fp8 serving: step {i} err {st}")
    r.check_tables()
    stats = r.dms.dms_cache_stats(r.cache)
    log(f"fp8 serving: {stats}")
