"""Prefill attention shapes against the CPU oracle (needs an MI355X).

Small bf16 / fp8 layers that route through the matrix-core prefill kernel
(GQA group 1, 2, 4; head_dim 64 and 128; block 32) and one that falls back to
the vector kernel (group 8).  Chunks of ragged sizes (37, 100, 64, 99) are
appended for two sequences given in reverse order, so a chunk starts at a
non-multiple of the key block and of the query block, the last query block of
a chunk is partly empty, and cache keys with pending eviction (inside the
window) mix with chunk keys in one key block.  Every row of every chunk is
compared; then the slot tables, page bytes, and a few decode steps.
"""
import pytest

from learned_kv_cache_amd import synth
from tests.harness import Runner, log, prepare

pytestmark = pytest.mark.gpu

CHUNKS = (37, 100, 64, 99)

SHAPES = {
    "g4_d64_bf16": (8, 2, 64, "bf16"),
    "g2_d128_bf16": (8, 4, 128, "bf16"),
    "g1_d64_bf16": (4, 4, 64, "bf16"),
    "g4_d128_fp8": (8, 2, 128, "fp8"),
    "g2_d64_fp8": (4, 2, 64, "fp8"),
    "g8_d64_bf16_vector_kernel": (16, 2, 64, "bf16"),
}


def _workload(name, idx):
    Hq, Hkv, D, kv = SHAPES[name]
    return synth.Workload(
        name=f"prefill_{name}", cfg_id=20 + idx, B=2, hidden=256, Hq=Hq, Hkv=Hkv, D=D, act_dtype="bf16",
        kv_dtype=kv, window=48, block=32, prefill=sum(CHUNKS), decode_steps=8, chunk=128,
        p_range=(0.40, 0.70))


@pytest.mark.parametrize("name", list(SHAPES))
def test_prefill_shapes_ragged_chunks(name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = _workload(name, list(SHAPES).index(name))
    prep = prepare(wl)
    r = Runner(prep, max_chunk=128)
    seqs = [1, 0]
    s = 0
    for n in CHUNKS:
        st = r.prefill_chunk(seqs, s, n, check_rows=n)
        log(f"{name}: chunk [{s}, {s + n}) err {st}")
        s += n
    r.check_tables(pages=True)
    for i in range(wl.decode_steps):
        r.decode_step(seqs, [s + i] * 2, fused=i % 3 == 1, step=i % 3 == 2)
    r.check_tables(pages=True)
