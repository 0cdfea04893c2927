"""dms_decode_step (decision, append and attention of a decode token in one
call) against the CPU oracle (needs an MI355X).

Small bf16 layers with a short window (24) and small pages (16) so that, in a
few dozen steps, tokens overwrite the slots of marked tokens in place, heads
open pages from the shared pool, and sequences sit at different positions
(log-uniform prompt lengths, rows given in a shuffled order).  Every step
checks the decisions and logits, the attention output of every query head,
and, bit for bit, the slot tables, page tables, ring, positions, free stack
and page bytes (fp8 pages: codes and per-page scales, the current token's
row quantised by the attention exactly as the append stores it, in place,
into the current page or as the first row of a new page).  Shapes cover GQA
groups 1, 2, 4 and 8, head_dim 64 and 128, bf16 and fp8 pages, both decision
sources, layer mode, and more than 64 (row, KV head) units; bf16 pages run
the matrix-core decode, and, for two shapes, the lane-per-row-piece one; the
decisions and placements run one workgroup per (row, KV head) pair or, for
three shapes, one per batch row.
"""
import copy

import numpy as np
import pytest

import oracle
from learned_kv_cache_amd import synth
from tests.harness import Runner, from_dev, log, prepare, to_dev

pytestmark = pytest.mark.gpu

# name: (B, Hq, Hkv, D, decide, alpha_per, kv_dtype)
SHAPES = {
    "g4_d128_linear": (3, 8, 2, 128, "linear", "head", "bf16"),
    "g2_d64_qneuron": (3, 8, 4, 64, "qneuron", "head", "bf16"),
    "g8_d64_linear_layer": (2, 16, 2, 64, "linear", "layer", "bf16"),
    "g1_d128_qneuron_80_units": (20, 4, 4, 128, "qneuron", "head", "bf16"),
    "g4_d128_linear_fp8": (3, 8, 2, 128, "linear", "head", "fp8"),
    "g2_d64_qneuron_fp8": (3, 8, 4, 64, "qneuron", "head", "fp8"),
    # bf16 pages through the lane-per-row-piece kernel (the matrix-core one off)
    "g4_d128_linear_vector": (3, 8, 2, 128, "linear", "head", "bf16"),
    "g2_d64_qneuron_vector": (3, 8, 4, 64, "qneuron", "head", "bf16"),
    # one prepare workgroup per batch row (the layout of large batches)
    "g4_d128_linear_fp8_rows": (3, 8, 2, 128, "linear", "head", "fp8"),
    "g2_d64_qneuron_rows": (3, 8, 4, 64, "qneuron", "head", "bf16"),
    "g8_d64_linear_layer_rows": (2, 16, 2, 64, "linear", "layer", "bf16"),
}


@pytest.fixture(autouse=True)
def _one_launch(monkeypatch):
    """Every step=True call here runs the one-launch kernel, also where the
    default would take the two calls (a step too large for one resident
    launch); the caches read the setting when they are created."""
    monkeypatch.setenv("DMS_DECODE_STEP_FUSE", "1")


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _workload(name, idx, **kw):
    B, Hq, Hkv, D, decide, per, kv = SHAPES[name]
    args = dict(name=f"step_{name}", cfg_id=40 + idx, B=B, hidden=256, Hq=Hq, Hkv=Hkv, D=D, act_dtype="bf16",
                kv_dtype=kv, window=24, block=16, prefill=0, decode_steps=40, chunk=64,
                p_range=(0.40, 0.70), ctx_range=(20, 150), decide=decide, alpha_per=per)
    args.update(kw)
    return synth.Workload(**args)


def _fill(r, seqs):
    """Each sequence's prompt, in chunks of up to 64, one sequence at a time."""
    ctx = r.prep.draw.ctx
    for b in seqs:
        s = 0
        while s < int(ctx[b]):
            n = min(64, int(ctx[b]) - s)
            r.prefill_chunk([b], s, n, attend=False)
            s += n


@pytest.mark.parametrize("name", list(SHAPES))
def test_step_ragged_positions(name, monkeypatch):
    _cuda()
    if name.endswith("_vector"):
        monkeypatch.setenv("DMS_DECODE_MFMA", "0")
    if name.endswith("_rows"):
        monkeypatch.setenv("DMS_DECODE_STEP_ROWS", "1")
    wl = _workload(name, list(SHAPES).index(name))
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    ctx = prep.draw.ctx
    seqs = list(np.random.default_rng(wl.cfg_id).permutation(wl.B))
    _fill(r, seqs)
    r.check_tables(pages=True)
    log(f"{name}: prompts {[int(ctx[b]) for b in seqs]}")
    worst = (0.0, 0.0)
    for i in range(wl.decode_steps):
        # every third step through the two-call path: both leave the same state
        st = r.decode_step(seqs, [int(ctx[b]) + i for b in seqs], step=i % 3 != 2, fused=i % 3 == 2)
        worst = (max(worst[0], st[0]), max(worst[1], st[1]))
        r.check_tables(pages=True)
    assert r.dms.dms_cache_status(r.cache) == 0
    log(f"{name}: worst err {worst}, stats {r.sim.stats()}")


def test_step_from_empty_cache():
    """Decode from position 0: heads whose only key is the current token, a page
    opened every 16 steps, in-place reuse from step 24 on."""
    _cuda()
    wl = _workload("g4_d128_linear", 0, ctx_range=None, prefill=0, decode_steps=70, cfg_id=50)
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    seqs = [2, 0, 1]
    for t in range(wl.decode_steps):
        r.decode_step(seqs, [t] * 3, step=True)
        r.check_tables(pages=True)
    log(f"empty start: stats {r.sim.stats()}")


def test_step_plan_reuse_and_invalidation():
    """A step leaves the next step a plan of its split (rows, page ids and the
    next token's placement per attention workgroup).  Steps in a row use it;
    every other call that changes the cache (an append through dms_decide +
    dms_append_evict, dms_decode_prepare, a chunk append, a reset) leaves the
    next step to plan afresh, and so do another row order and fewer rows.
    Every step is checked against the oracle, the tables after each phase."""
    _cuda()
    from learned_kv_cache_amd import dms
    wl = _workload("g4_d128_linear", 0, cfg_id=52, decode_steps=48)
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    ctx = prep.draw.ctx
    seqs = [2, 0, 1]
    _fill(r, seqs)
    pos = {b: int(ctx[b]) for b in seqs}

    def step(rows, n=1, **kw):
        for _ in range(n):
            r.decode_step(rows, [pos[b] for b in rows], **kw)
            for b in rows:
                pos[b] += 1

    step(seqs, 3, step=True)
    step(seqs, step=False)                      # decide + append + attention
    step(seqs, 2, step=True)
    step(seqs, fused=True)                      # dms_decode_prepare + attention
    step(seqs, 2, step=True)
    r.check_tables(pages=True)
    step([0, 1, 2], 2, step=True)               # another row order, same batch
    step([1, 2], 2, step=True)                  # fewer rows
    step([0, 1, 2], step=True)
    r.prefill_chunk([1], pos[1], 5, attend=False)
    pos[1] += 5
    step([0, 1, 2], 2, step=True)
    r.check_tables(pages=True)
    # a reset right after a step over the same rows: sequence 0 starts again
    # from position 0
    dms.dms_seq_reset(r.cache, to_dev(np.array([0], np.int32), "i32"), 1)
    r.sim.reset([0])
    pos[0] = 0
    step([0, 1, 2], 3, step=True)
    r.check_tables(pages=True)
    assert r.dms.dms_cache_status(r.cache) == 0


def test_step_subset_of_rows_and_capacity():
    """A call over some rows leaves the others alone; a row at its capacity is
    flagged and not appended while the other rows proceed."""
    torch = _cuda()
    from learned_kv_cache_amd import dms
    wl = _workload("g2_d64_qneuron", 1, ctx_range=None, prefill=0, decode_steps=12, cfg_id=51)
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    for t in range(4):
        r.decode_step([1], [t], step=True)
    for t in range(4):
        r.decode_step([0, 2], [t, t], step=True)
    r.check_tables(pages=True)
    # row 1 runs to its capacity (12 tokens), then one more step over rows 1 and 0
    for t in range(4, 12):
        r.decode_step([1], [t], step=True)
    r.check_tables(pages=True)
    before = r.dms.dms_cache_dump(r.cache)
    B = 2
    ids = to_dev(np.array([1, 0], np.int32), "i32")
    q = torch.randn(B * wl.Hq * wl.D, device="cuda").to(torch.bfloat16)
    k = torch.randn(B * wl.Hkv * wl.D, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    ev = torch.empty(B * wl.Hkv, dtype=torch.uint8, device="cuda")
    dms.dms_decode_step(r.cache, ids, None, None, None, None, r.off, q.clone(), k, k, out, B, None, ev)
    assert dms.dms_cache_status(r.cache) & dms.DMS_DEV_CAPACITY
    after = r.dms.dms_cache_dump(r.cache)
    assert int(after["positions"][1]) == 12 and int(after["positions"][0]) == 5
    assert np.array_equal(after["lengths"][1], before["lengths"][1])
    # against the oracle: row 1 attends over its 12-token cache as it stands
    # (positions 0..11, the visible set of a query at position 11); row 0
    # appended its token at position 4, so it attends over positions 0..4
    # (all inside the window), the last with this call's k (= v) row
    q_np = from_dev(q).reshape(B, wl.Hq, wl.D)
    q_np[:, :: wl.g, -1] = 0.0                       # the decision neuron plays no part
    k_np = from_dev(k).reshape(B, wl.Hkv, wl.D)
    got = from_dev(out).reshape(B, wl.Hq, wl.D)
    mx, mn = 2e-2, 2e-3
    K1, V1 = r.kv_view(1, 12)
    ref1 = oracle.attention_rows(q_np[0][None], K1, V1, prep.evict[1][:, :12], wl.window, [11], r.scale)[0]
    K0, V0 = r.kv_view(0, 4)
    K0 = np.concatenate([K0, k_np[1][None]])
    V0 = np.concatenate([V0, k_np[1][None]])
    ref0 = oracle.attention_rows(q_np[1][None], K0, V0, np.zeros((wl.Hkv, 5), np.uint8), wl.window, [4],
                                 r.scale)[0]
    for g_, ref in ((got[0], ref1), (got[1], ref0)):
        err = np.abs(g_ - ref)
        assert err.max() <= mx and err.mean() <= mn, (err.max(), err.mean())


def test_step_bad_sequence_id():
    torch = _cuda()
    from learned_kv_cache_amd import dms
    wl = _workload("g4_d128_linear", 0, ctx_range=None, prefill=0, decode_steps=4, cfg_id=52)
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    r.decode_step([0, 1], [0, 0], step=True)
    ids = to_dev(np.array([0, 7], np.int32), "i32")
    B = 2
    h = torch.randn(B * wl.hidden, device="cuda").to(torch.bfloat16)
    q = torch.randn(B * wl.Hq * wl.D, device="cuda").to(torch.bfloat16)
    k = torch.randn(B * wl.Hkv * wl.D, device="cuda").to(torch.bfloat16)
    out = torch.full_like(q, 3.0)
    ev = torch.empty(B * wl.Hkv, dtype=torch.uint8, device="cuda")
    dms.dms_decode_step(r.cache, ids, h, r.gamma, r.W, None, r.off, q, k, k, out, B, None, ev)
    assert dms.dms_cache_status(r.cache) & dms.DMS_DEV_BAD_SEQ
    assert float(out[wl.Hq * wl.D:].float().abs().max()) == 0.0     # the bad row's heads have no keys
    dump = r.dms.dms_cache_dump(r.cache)
    assert int(dump["positions"][0]) == 2 and int(dump["positions"][1]) == 1


def test_step_max_units():
    """2048 (row, KV head) units, the most one call takes: 256 rows x 8 KV
    heads, prompts of two lengths; the three decode paths in turn (the fused
    step's commit then runs over eight batches of pairs, the attention's
    prologue scans eight units per thread and splits the concatenated slots)."""
    _cuda()
    wl = synth.Workload(name="step_max_units", cfg_id=53, B=256, hidden=256, Hq=8, Hkv=8, D=64, act_dtype="bf16",
                        kv_dtype="bf16", window=24, block=16, prefill=0, decode_steps=6, chunk=64,
                        p_range=(0.40, 0.70), ctx_range=(20, 150), decide="linear", alpha_per="head")
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    ctx = prep.draw.ctx
    seqs = list(range(wl.B))
    # prompts through one chunk call per (start, length) group of rows
    groups = {}
    for b in seqs:
        groups.setdefault(int(ctx[b]), []).append(b)
    for n, rows in sorted(groups.items()):
        s = 0
        while s < n:
            c = min(64, n - s)
            r.prefill_chunk(rows, s, c, attend=False)
            s += c
    r.check_tables(pages=False)
    for i in range(wl.decode_steps):
        r.decode_step(seqs, [int(ctx[b]) + i for b in seqs], step=i % 3 == 0, fused=i % 3 == 1)
    r.check_tables(pages=True)
    assert r.dms.dms_cache_status(r.cache) == 0
    log(f"max units: stats {r.sim.stats()}")


def test_step_fp8_concatenated_split():
    """fp8 pages, 320 (row, KV head) units: the attention cuts the
    concatenated slots into equal ranges, so some workgroups' ranges start at
    the current token's row — also when that token opens a new page (pages of
    16).  Regression case: such a range has no stored row to stand in for its
    masked lanes."""
    _cuda()
    wl = synth.Workload(name="step_fp8_concat", cfg_id=54, B=40, hidden=256, Hq=8, Hkv=8, D=128, act_dtype="bf16",
                        kv_dtype="fp8", window=24, block=16, prefill=0, decode_steps=24, chunk=64,
                        p_range=(0.40, 0.70), ctx_range=(20, 80), decide="linear", alpha_per="head")
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    ctx = prep.draw.ctx
    seqs = list(range(wl.B))
    _fill(r, seqs)
    r.check_tables(pages=True)
    for i in range(wl.decode_steps):
        r.decode_step(seqs, [int(ctx[b]) + i for b in seqs], step=True)
    r.check_tables(pages=True)
    assert r.dms.dms_cache_status(r.cache) == 0


def test_step_gives_up_and_recovers(monkeypatch):
    """The commit's bounded wait made to give up from the host
    (DMS_STEP_SPIN_LIMIT=0, every kernel still exits normally): the status
    bit is set and no table changes; after dms_cache_clear_status the same
    step, repeated, commits and the cache equals the oracle's (which saw the
    step once), and later steps go on normally."""
    _cuda()
    from learned_kv_cache_amd import dms
    wl = _workload("g4_d128_linear", 0, ctx_range=None, prefill=0, decode_steps=34, cfg_id=56)
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    seqs = [0, 2, 1]
    for t in range(30):                               # past the window of 24: in-place reuse happens
        r.decode_step(seqs, [t] * 3, step=True)
    r.check_tables(pages=True)
    saved = copy.deepcopy(r.sim)
    monkeypatch.setenv("DMS_STEP_SPIN_LIMIT", "0")
    r.decode_step(seqs, [30] * 3, step=True, check=False)     # decisions still checked
    assert dms.dms_cache_status(r.cache) == dms.DMS_DEV_STEP_SYNC
    r.sim = saved                                     # the step did not commit
    # positions, lengths, page tables, ring and pool as before the call (slot
    # metadata and rows of the slots it would have taken may be written)
    dump = dms.dms_cache_dump(r.cache)
    assert np.array_equal(dump["positions"], np.asarray(saved.pos, np.int32))
    assert np.array_equal(dump["lengths"], np.asarray(saved.L, np.int32))
    assert int(dump["free_count"][0]) == len(saved.free)
    for b in seqs:
        for kh in range(wl.Hkv):
            assert list(dump["page_table"][b, kh][: len(saved.pages[b][kh])]) == saved.pages[b][kh]
            for t, (slot, e) in saved.ring(b, kh).items():
                assert int(dump["ring"][b, kh, t % wl.window]) & 0xFFFFFFFF == slot | (e << 31)
    monkeypatch.delenv("DMS_STEP_SPIN_LIMIT")
    dms.dms_cache_clear_status(r.cache)
    assert dms.dms_cache_status(r.cache) == 0
    for t in range(30, 34):
        r.decode_step(seqs, [t] * 3, step=True)
        r.check_tables(pages=True)
    assert dms.dms_cache_status(r.cache) == 0


def test_decode_workspace_is_checked():
    """dms_decode_workspace_bytes gives two partial records per attention
    workgroup plus one per (row, KV head) unit; a missing or short workspace
    is refused before any launch, and an exact one works."""
    torch = _cuda()
    from learned_kv_cache_amd import dms
    wl = _workload("g4_d128_linear", 0, ctx_range=None, prefill=0, decode_steps=4, cfg_id=57)
    prep = prepare(wl)
    r = Runner(prep, max_chunk=64)
    B = 3
    n = dms.dms_decode_workspace_bytes(r.cfg, B)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rec = wl.g * (wl.D + 2) * 4
    want = (2 * 2 * cus + B * wl.Hkv) * rec
    assert want <= n < want + 256
    with pytest.raises(dms.DmsError):
        dms.dms_decode_workspace_bytes(r.cfg, 0)
    r.decode_step([0, 1, 2], [0] * 3, step=True)
    q = torch.zeros(B * wl.Hq * wl.D, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    short = torch.empty(n - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(dms.DmsError) as ei:
        dms.dms_decode_attn(r.cache, None, q, out, B, workspace=short)
    assert ei.value.status == dms.DMS_ERR_CAPACITY
    k = torch.zeros(B * wl.Hkv * wl.D, dtype=torch.bfloat16, device="cuda")
    ev = torch.empty(B * wl.Hkv, dtype=torch.uint8, device="cuda")
    h = torch.zeros(B * wl.hidden, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dms.DmsError) as ei:
        dms.dms_decode_step(r.cache, None, h, r.gamma, r.W, None, r.off, q, k, k, out, B, None, ev, workspace=short)
    assert ei.value.status == dms.DMS_ERR_CAPACITY
    r.check_tables(pages=True)                        # neither call touched the cache
    exact = torch.empty(n, dtype=torch.uint8, device="cuda")
    dms.dms_decode_attn(r.cache, None, q, out, B, workspace=exact)
    assert dms.dms_cache_status(r.cache) == 0
