"""dms_step_layers (the decode step of every layer of a model in one launch)
against the CPU oracle, layer by layer (needs an MI355X).

Each layer is one of the small caches of the one-call step tests (window 24,
pages of 16, ragged prompt lengths, rows in a shuffled order), with draws of
its own.  Every step checks, in every layer, the decisions and logits, the
attention output of every query head, and, bit for bit, the slot tables,
page tables, ring, positions, free stack and page bytes.  The one-launch
kernel is required where the shape allows it (bf16 pages, head groups of up
to 4), and the call's own fallback (one dms_decode_step per layer) is
exercised by fp8 pages; steps of a subset of the rows, steps interleaved with
per-layer dms_decode_step calls on the same caches, and the barrier and
commit waits made to give up from the host are covered too.
"""
import copy

import numpy as np
import pytest

from tests.harness import Runner, log, prepare
from tests.test_gpu_decode_step import SHAPES, _fill, _workload

pytestmark = pytest.mark.gpu

# shape -> whether the layers must run as one launch
LAYER_SHAPES = {
    "g4_d128_linear": True,
    "g2_d64_qneuron": True,
    "g8_d64_linear_layer": None,      # either (the group of 8 may not fit two workgroups per CU)
    "g4_d128_linear_fp8": None,
}


@pytest.fixture(autouse=True)
def _one_launch(monkeypatch):
    monkeypatch.setenv("DMS_DECODE_STEP_FUSE", "1")


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _runners(name, n_layers, **kw):
    idx = list(SHAPES).index(name)
    out = []
    for l in range(n_layers):
        wl = _workload(name, idx, cfg_id=200 + 10 * idx + l, **kw)
        out.append(Runner(prepare(wl), max_chunk=64))
    return out


def _bind(runners):
    """Static per-layer buffers of max_batch rows, bound to a StepLayers."""
    torch = _cuda()
    from learned_kv_cache_amd import dms
    io = []
    for r in runners:
        wl = r.wl
        bf = torch.bfloat16
        d = dict(q_inout=torch.zeros(wl.B * wl.Hq * wl.D, dtype=bf, device="cuda"),
                 k=torch.zeros(wl.B * wl.Hkv * wl.D, dtype=bf, device="cuda"),
                 v=torch.zeros(wl.B * wl.Hkv * wl.D, dtype=bf, device="cuda"),
                 out=torch.zeros(wl.B * wl.Hq * wl.D, dtype=bf, device="cuda"),
                 logits_out=torch.zeros(wl.B * wl.Hkv, dtype=torch.float32, device="cuda"),
                 evict_out=torch.zeros(wl.B * wl.Hkv, dtype=torch.uint8, device="cuda"),
                 offsets=r.off)
        if wl.decide == "linear":
            d.update(hidden=torch.zeros(wl.B * wl.hidden, dtype=bf, device="cuda"), rms_gamma=r.gamma, W=r.W)
        io.append(d)
    return dms.StepLayers([r.cache for r in runners], io), io


def _layers_step(L, io, runners, seqs, positions, check=True):
    """One token per row in every layer through dms_step_layers_run, then each
    layer's results against the oracle (positions[l]: the rows' positions in
    layer l's cache)."""
    xs = []
    for r, d, pos in zip(runners, io, positions):
        x = r.step_inputs(seqs, pos)
        B, wl = x["B"], r.wl
        d["q_inout"][: B * wl.Hq * wl.D].copy_(x["q_dev"].view(-1))
        d["k"][: B * wl.Hkv * wl.D].copy_(x["k_dev"].view(-1))
        d["v"][: B * wl.Hkv * wl.D].copy_(x["v_dev"].view(-1))
        if x["h_dev"] is not None:
            d["hidden"][: B * wl.hidden].copy_(x["h_dev"].view(-1))
        xs.append(x)
    L.run(xs[0]["seq_dev"], len(seqs))
    worst = (0.0, 0.0)
    for r, d, x, pos in zip(runners, io, xs, positions):
        B, wl = x["B"], r.wl
        x["q_dev"].view(-1).copy_(d["q_inout"][: B * wl.Hq * wl.D])
        x["out"].copy_(d["out"][: B * wl.Hq * wl.D])
        x["logits"].copy_(d["logits_out"][: B * wl.Hkv])
        x["evict"].copy_(d["evict_out"][: B * wl.Hkv])
        st = r.decode_step(seqs, pos, launched=x, check=check)
        if st is not None:
            worst = (max(worst[0], st[0]), max(worst[1], st[1]))
    return worst


@pytest.mark.parametrize("name", list(LAYER_SHAPES))
def test_layers_ragged_positions(name):
    """Three layers, 30 steps of all rows; every fourth step, every layer's
    cache takes the step through its own dms_decode_step instead (the plans
    the two leave are the same)."""
    _cuda()
    runners = _runners(name, 3)
    L, io = _bind(runners)
    B = runners[0].wl.B
    want = LAYER_SHAPES[name]
    if want is not None:
        assert L.one_launch(B) == want
    log(f"{name}: one launch {L.one_launch(B)}")
    seqs = list(np.random.default_rng(7).permutation(B))
    for r in runners:
        _fill(r, seqs)
        r.check_tables(pages=True)
    worst = (0.0, 0.0)
    for i in range(30):
        pos = [[int(r.prep.draw.ctx[b]) + i for b in seqs] for r in runners]
        if i % 4 == 3:
            for r, p in zip(runners, pos):
                r.decode_step(seqs, p, step=True)
        else:
            st = _layers_step(L, io, runners, seqs, pos)
            worst = (max(worst[0], st[0]), max(worst[1], st[1]))
        for r in runners:
            r.check_tables(pages=True)
    for r in runners:
        assert r.dms.dms_cache_status(r.cache) == 0
    log(f"{name}: worst err {worst}")


def test_layers_subset_of_rows():
    """Steps of two of the three rows, then of the third alone: the absent rows'
    tables do not move (four layers)."""
    _cuda()
    runners = _runners("g2_d64_qneuron", 4)
    L, io = _bind(runners)
    assert L.one_launch(2) and L.one_launch(1)
    for r in runners:
        _fill(r, [0, 1, 2])
    for i in range(12):
        seqs = [2, 0] if i < 8 else [1]
        pos = [[int(r.sim.pos[b]) for b in seqs] for r in runners]
        _layers_step(L, io, runners, seqs, pos)
        for r in runners:
            r.check_tables(pages=True)


def test_layers_give_up_and_recover(monkeypatch):
    """The commit's and the layer barrier's bounded waits made to give up from
    the host (DMS_STEP_SPIN_LIMIT=0; every kernel exits normally): the status
    bit is set in the layers' caches and no table changes; after
    dms_cache_clear_status the same step, repeated, commits in every layer and
    the caches equal the oracle's, and later steps go on normally."""
    _cuda()
    from learned_kv_cache_amd import dms
    runners = _runners("g4_d128_linear", 2, ctx_range=None, prefill=0, decode_steps=34)
    L, io = _bind(runners)
    assert L.one_launch(3)
    seqs = [0, 2, 1]
    for t in range(26):
        _layers_step(L, io, runners, seqs, [[t] * 3] * 2)
    for r in runners:
        r.check_tables(pages=True)
    saved = [copy.deepcopy(r.sim) for r in runners]
    monkeypatch.setenv("DMS_STEP_SPIN_LIMIT", "0")
    _layers_step(L, io, runners, seqs, [[26] * 3] * 2, check=False)
    for r, sv in zip(runners, saved):
        assert dms.dms_cache_status(r.cache) & dms.DMS_DEV_STEP_SYNC
        r.sim = sv                                    # the step did not commit
        dump = dms.dms_cache_dump(r.cache)
        assert np.array_equal(dump["positions"], np.asarray(sv.pos, np.int32))
        assert np.array_equal(dump["lengths"], np.asarray(sv.L, np.int32))
        assert int(dump["free_count"][0]) == len(sv.free)
    monkeypatch.delenv("DMS_STEP_SPIN_LIMIT")
    for r in runners:
        dms.dms_cache_clear_status(r.cache)
        assert dms.dms_cache_status(r.cache) == 0
    for t in range(26, 32):
        _layers_step(L, io, runners, seqs, [[t] * 3] * 2)
        for r in runners:
            r.check_tables(pages=True)
    for r in runners:
        assert dms.dms_cache_status(r.cache) == 0


def test_layers_arguments():
    """Binding errors: mismatched shapes, a cache twice, a missing buffer."""
    _cuda()
    from learned_kv_cache_amd import dms
    a = _runners("g4_d128_linear", 1)[0]
    b = _runners("g4_d128_linear", 1, window=32)[0]     # same buffers, another window
    La, ioa = _bind([a])
    Lb, iob = _bind([b])
    with pytest.raises(dms.DmsError):
        dms.StepLayers([a.cache, b.cache], [ioa[0], iob[0]])
    with pytest.raises(dms.DmsError):
        dms.StepLayers([a.cache, a.cache], [ioa[0], ioa[0]])
    bad = dict(ioa[0])
    bad["evict_out"] = None
    with pytest.raises(dms.DmsError):
        dms.StepLayers([a.cache], [bad])
