"""Serving accounting and multi-turn continuation (needs an MI355X).

A conversation in a serving loop: each sequence's prompt is prefilled, then
decoded, then a second user turn is prefilled onto the same compressed cache
(no reset), then decoded again.  After every phase the slot/page tables equal
the oracle's model bit for bit, and the attention of the prefill chunks and
decode steps is within the bf16 tolerance of the oracle.

Accounting (FastDMS post, subsystem table: admission by compact KV capacity,
memory accounting by surviving tokens):
* dms_seq_info_get  -> positions, live slots, largest head and pages of the
  oracle's model;
* dms_pages_needed  -> the oracle's worst case (every new token kept,
  simulated), for continuations shorter than, equal to and longer than the
  window, -1 past the sequence capacity; and it is reached: appending that
  many all-kept tokens takes exactly that many pages from the pool;
* a reset returns every page of the sequence to the pool.

bf16 layer, window 24, pages of 16 tokens, three sequences of log-uniform
prompt lengths 20..150.
"""
import numpy as np
import pytest

import oracle
from learned_kv_cache_amd import synth
from tests.harness import Runner, log, prepare, to_dev

pytestmark = pytest.mark.gpu

W, P = 24, 16
DECODE_1, TURN_2, DECODE_2, TAIL = 30, 25, 35, 30


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _runner(decide="linear", cfg_id=60):
    wl = synth.Workload(name="serving_multiturn", cfg_id=cfg_id, B=3, hidden=256, Hq=8, Hkv=2, D=128,
                        act_dtype="bf16", kv_dtype="bf16", window=W, block=P, prefill=0,
                        decode_steps=DECODE_1 + TURN_2 + DECODE_2 + TAIL, chunk=64,
                        p_range=(0.40, 0.70), ctx_range=(20, 150), decide=decide, alpha_per="head")
    return Runner(prepare(wl), max_chunk=64)


def _prefill(r, b, s, n):
    while n > 0:
        c = min(64, n)
        r.prefill_chunk([b], s, c, check_rows=c)
        s += c
        n -= c


def _check_accounting(r, what):
    dms, sim = r.dms, r.sim
    seqs = list(range(r.wl.B))
    info = dms.dms_seq_info_get(r.cache, seqs)
    for b, got in zip(seqs, info):
        L = [int(x) for x in sim.L[b]]
        want = dict(position=int(sim.pos[b]), live_slots=sum(L), max_head_slots=max(L),
                    pages=sum(len(p) for p in sim.pages[b]))
        assert got == want, (what, b, got, want)
    ns = [0, 1, 5, W - 1, W, W + 1, 2 * W, 3 * W + 7]
    for b in seqs:
        room = r.max_tokens - int(sim.pos[b])
        counts = [n for n in ns if n <= room] + [room, room + 1]
        got, free = dms.dms_pages_needed(r.cache, [b] * len(counts), counts)
        want = [oracle.pages_needed_worst(sim, b, n) for n in counts]
        assert got == want, (what, b, counts, got, want)
        assert free == len(sim.free)
        assert got[-1] == -1
    log(f"{what}: accounting {info}")


def test_multiturn_serving_accounting():
    torch = _cuda()
    r = _runner()
    dms, wl = r.dms, r.wl
    ctx = [int(c) for c in r.prep.draw.ctx]
    seqs = list(range(wl.B))
    log(f"prompts {ctx}, capacity {r.max_tokens}")
    _check_accounting(r, "empty")
    for b in seqs:                                            # turn 1: the prompts
        _prefill(r, b, 0, ctx[b])
    r.check_tables(pages=True)
    _check_accounting(r, "after prompts")
    for i in range(DECODE_1):                                 # turn 1: the answers
        r.decode_step(seqs, [ctx[b] + i for b in seqs], step=True)
    r.check_tables(pages=True)
    _check_accounting(r, "after first answers")
    for b in seqs:                                            # turn 2: the next user message
        _prefill(r, b, ctx[b] + DECODE_1, TURN_2)
    r.check_tables(pages=True)
    _check_accounting(r, "after second prompts")
    base = DECODE_1 + TURN_2
    for i in range(DECODE_2):                                 # turn 2: the answers
        r.decode_step(seqs, [ctx[b] + base + i for b in seqs], step=True)
    r.check_tables(pages=True)
    _check_accounting(r, "after second answers")
    assert dms.dms_cache_status(r.cache) == 0

    # the bound is reached: TAIL all-kept tokens on sequence 1 take exactly the
    # pages it promised
    b = 1
    need, free = dms.dms_pages_needed(r.cache, [b], [TAIL])
    gen = np.random.default_rng(61)
    kv = synth.as_dtype(gen.standard_normal((1, TAIL, wl.Hkv, wl.D), dtype=np.float32), "bf16")
    keep = np.zeros((1, wl.Hkv, TAIL), np.uint8)
    dms.dms_append_evict(r.cache, to_dev(np.array([b], np.int32), "i32"), to_dev(kv, "bf16"),
                         to_dev(kv, "bf16"), to_dev(keep, "u8"), 1, TAIL)
    r.sim.append([b], keep, kv, kv)
    r.check_tables(pages=False)
    after = dms.dms_cache_dump(r.cache)
    assert free - int(after["free_count"][0]) == need[0] > 0
    _check_accounting(r, "after all-kept tail")

    # a finished conversation hands its pages back
    held = sum(len(p) for p in r.sim.pages[0])
    dms.dms_seq_reset(r.cache, to_dev(np.array([0], np.int32), "i32"), 1)
    r.sim.reset([0])
    r.check_tables(pages=False)
    info = dms.dms_seq_info_get(r.cache, [0])[0]
    assert info == dict(position=0, live_slots=0, max_head_slots=0, pages=0)
    assert int(dms.dms_cache_dump(r.cache)["free_count"][0]) == int(after["free_count"][0]) + held
    _check_accounting(r, "after reset")
    torch.cuda.synchronize()


def test_accounting_arguments():
    _cuda()
    r = _runner(decide="qneuron", cfg_id=62)
    dms = r.dms
    with pytest.raises(dms.DmsError):
        dms.dms_seq_info_get(r.cache, [0, 3])
    with pytest.raises(dms.DmsError):
        dms.dms_pages_needed(r.cache, [0], [-1])
    got, free = dms.dms_pages_needed(r.cache, [], [])
    assert got == [] and free == len(r.sim.free)
