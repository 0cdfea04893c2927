"""Seeded synthetic inputs for the DMS hot path.

This module is shared by the HIP path's tests/benchmark and by the CPU oracle's
tests.  It draws random numbers and rounds them to the storage dtype; it holds
none of the method's arithmetic (no normalisation, projection, thresholding,
slot assignment or attention).  Where an input depends on the method (per-head
offsets that give a target eviction fraction, tokens kept away from the
decision threshold) the caller computes the logits and this module only does
the order statistics or the redraw.

Workload shapes follow the DMS inference setting of the Model-Optimizer
walkthrough page ("基于 DMS 的 KV Cache 压缩实战", Qwen3ConfigDMS parameter
table: window 512, paged block 256, alpha scale 100, offset 5) at the Qwen3-8B
and Llama-3.2-1B layer shapes, plus the FastDMS serving setting (page "FastDMS",
ctx 8192 / gen 128 tables).  No dataset is used anywhere.

Seeds: ``numpy.random.Generator(PCG64(SeedSequence([1000 + cfg_id, run_id])))``
spawned into child streams in the fixed order of ``STREAMS``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

STREAMS = ("p_h", "W", "h", "q", "k", "v", "ctx", "resample")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, dtype and distribution recipe of one synthetic workload."""

    name: str
    cfg_id: int
    B: int
    hidden: int
    Hq: int
    Hkv: int
    D: int
    act_dtype: str          # "f32" | "bf16": hidden states, Q/K/V inputs, outputs
    kv_dtype: str           # "f32" | "bf16" | "fp8": cache storage
    window: int
    block: int
    prefill: int            # prompt tokens per sequence (0: ragged, see ctx_range)
    decode_steps: int
    chunk: int              # prefill chunk size
    p_range: Tuple[float, float]   # per-head eviction fraction, U[lo, hi]
    p_fixed: Optional[Tuple[float, ...]] = None   # fixed per-head fractions
    decide: str = "linear"         # "linear" | "qneuron"
    alpha_scale: float = 100.0
    fixed_offset: Optional[float] = None   # use this offset for every head (no calibration)
    w_std: Optional[float] = None          # std of projection entries (None: 1/sqrt(hidden))
    ctx_range: Optional[Tuple[int, int]] = None   # log-uniform per-sequence contexts
    alpha_per: str = "head"
    disable_eviction: bool = False

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    def weight_std(self) -> float:
        return self.w_std if self.w_std is not None else 1.0 / math.sqrt(self.hidden)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Tiny fp32 single layer (window 16, block 8, fractions 0.70 / 0.85).
TINY = Workload(
    name="tiny_fp32_h256_g2_d32", cfg_id=1, B=1, hidden=256, Hq=4, Hkv=2, D=32,
    act_dtype="f32", kv_dtype="f32", window=16, block=8, prefill=64,
    decode_steps=64, chunk=64, p_range=(0.70, 0.85), p_fixed=(0.70, 0.85),
    w_std=0.25,
)
# Llama-3.2-1B attention layer shape, decode after an 8K prompt.
LLAMA1B_DECODE = Workload(
    name="llama3.2-1b_layer_ctx8k_b1_decode", cfg_id=2, B=1, hidden=2048, Hq=32,
    Hkv=8, D=64, act_dtype="bf16", kv_dtype="bf16", window=512, block=256,
    prefill=8192, decode_steps=128, chunk=4096, p_range=(0.80, 0.90),
)
# Qwen3-8B attention layer shape, 8 sequences decoding after an 8K prompt.
QWEN8B_DECODE = Workload(
    name="qwen3-8b_layer_ctx8k_b8_decode", cfg_id=3, B=8, hidden=4096, Hq=32,
    Hkv=8, D=128, act_dtype="bf16", kv_dtype="bf16", window=512, block=256,
    prefill=8192, decode_steps=128, chunk=4096, p_range=(0.85, 0.92),
)
# Qwen3-8B layer, one 32K prompt in 4096-token chunks; decisions from the
# repurposed last query neuron (offset 5 on every head).
QWEN8B_PREFILL32K = Workload(
    name="qwen3-8b_layer_prefill32k_c4096", cfg_id=4, B=1, hidden=4096, Hq=32,
    Hkv=8, D=128, act_dtype="bf16", kv_dtype="bf16", window=512, block=256,
    prefill=32768, decode_steps=256, chunk=4096, p_range=(0.0, 0.0),
    decide="qneuron", fixed_offset=5.0,
)
# Same, decisions from the separate linear adapter at its default offset 5.
QWEN8B_PREFILL32K_LINEAR = QWEN8B_PREFILL32K.replace(
    name="qwen3-8b_layer_prefill32k_c4096_linear", decide="linear")
# Qwen3-8B layer, 64 sequences with log-uniform contexts, fp8 e4m3 KV pages.
QWEN8B_FP8_SERVING = Workload(
    name="qwen3-8b_layer_fp8kv_b64_serving", cfg_id=5, B=64, hidden=4096, Hq=32,
    Hkv=8, D=128, act_dtype="bf16", kv_dtype="fp8", window=512, block=256,
    prefill=0, decode_steps=256, chunk=4096, p_range=(0.50, 0.95),
    ctx_range=(1024, 16384),
)

WORKLOADS = {w.name: w for w in (TINY, LLAMA1B_DECODE, QWEN8B_DECODE, QWEN8B_PREFILL32K,
                                 QWEN8B_PREFILL32K_LINEAR, QWEN8B_FP8_SERVING)}


# ---------------------------------------------------------------------------
# dtype helpers (storage rounding only)

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                                  # finite inputs: no wrap-around
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bfloat16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# streams and draws

def normal(gen: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return as_dtype(gen.standard_normal(shape, dtype=np.float32), dtype)


def context_lengths(wl: Workload, gen: np.random.Generator) -> np.ndarray:
    """Prompt length per sequence: fixed, or log-uniform over ``ctx_range``."""
    if wl.ctx_range is None:
        return np.full(wl.B, wl.prefill, dtype=np.int64)
    lo, hi = wl.ctx_range
    u = gen.uniform(math.log(lo), math.log(hi), size=wl.B)
    return np.rint(np.exp(u)).astype(np.int64)


def eviction_fractions(wl: Workload, gen: np.random.Generator) -> np.ndarray:
    if wl.p_fixed is not None:
        return np.asarray(wl.p_fixed, dtype=np.float64)
    lo, hi = wl.p_range
    return gen.uniform(lo, hi, size=wl.Hkv)


class Draw:
    """All random inputs of one run.

    Scalars and small tensors (p_h, ctx, W, gamma) are held; per-token tensors
    (h, q, k, v) are regenerated on demand, one sequence at a time, from that
    sequence's child seed, so a run with hundreds of thousands of tokens never
    sits in memory whole.  Values are float32 holding the storage dtype's
    values; per-token tensors of sequence b have ``ctx[b] + decode_steps`` rows.
    Redraws (``set_rows``) are kept as overlays and applied on every access.
    """

    TAILS = ("h", "q", "k", "v")

    def __init__(self, wl: Workload, run_id: int = 0):
        self.wl = wl
        ss = np.random.SeedSequence([1000 + wl.cfg_id, run_id])
        kids = dict(zip(STREAMS, ss.spawn(len(STREAMS))))
        self.gens = {name: np.random.Generator(np.random.PCG64(kids[name])) for name in STREAMS}
        self.p_h = eviction_fractions(wl, self.gens["p_h"])
        self.ctx = context_lengths(wl, self.gens["ctx"])
        self.W = self.gens["W"].normal(0.0, wl.weight_std(), size=(wl.Hkv, wl.hidden)).astype(np.float32)
        self.gamma = np.ones(wl.hidden, dtype=np.float32)
        # per sequence, one child for the prompt rows and one for the decode rows
        self._seeds = {name: kids[name].spawn(2 * wl.B) for name in self.TAILS}
        self._overlay: Dict[Tuple[str, int], Dict[int, np.ndarray]] = {}
        self._cache: Dict[Tuple[str, int], np.ndarray] = {}
        self._last: Dict[str, Tuple[int, np.ndarray]] = {}    # most recent sequence per tensor

    def T(self, b: int) -> int:
        return int(self.ctx[b]) + self.wl.decode_steps

    def _tail(self, name: str):
        wl = self.wl
        return {"h": (wl.hidden,), "q": (wl.Hq, wl.D), "k": (wl.Hkv, wl.D), "v": (wl.Hkv, wl.D)}[name]

    def tensor(self, name: str, b: int, keep: bool = False) -> np.ndarray:
        """Per-token tensor ``name`` of sequence b: [T_b, ...] float32."""
        key = (name, b)
        if key in self._cache:
            return self._cache[key]
        last = self._last.get(name)
        if last is not None and last[0] == b:
            return last[1]
        x = np.concatenate([self._rows(name, b, 0), self._rows(name, b, 1)], axis=0)
        for t, row in self._overlay.get(key, {}).items():
            x[t] = row
        if keep:
            self._cache[key] = x
        else:
            self._last[name] = (b, x)
        return x

    def _rows(self, name: str, b: int, part: int) -> np.ndarray:
        n = int(self.ctx[b]) if part == 0 else self.wl.decode_steps
        gen = np.random.Generator(np.random.PCG64(self._seeds[name][2 * b + part]))
        return normal(gen, (n,) + self._tail(name), self.wl.act_dtype)

    def decode_rows(self, name: str, b: int) -> np.ndarray:
        """Rows ctx[b] .. ctx[b] + decode_steps - 1 of ``name`` (cheap: drawn alone)."""
        key = (name, b)
        if key in self._cache:
            return self._cache[key][int(self.ctx[b]):]
        x = self._rows(name, b, 1)
        c0 = int(self.ctx[b])
        for t, row in self._overlay.get(key, {}).items():
            if t >= c0:
                x[t - c0] = row
        return x

    def set_rows(self, name: str, b: int, rows: Dict[int, np.ndarray]) -> None:
        """Record redrawn rows (position -> values) of ``name`` for sequence b."""
        self._overlay.setdefault((name, b), {}).update(rows)
        self._cache.pop((name, b), None)
        if self._last.get(name, (None,))[0] == b:
            del self._last[name]

    def stacked(self, name: str) -> np.ndarray:
        """[B, T, ...] of a per-token tensor (all sequences equally long)."""
        return np.stack([self.tensor(name, b) for b in range(self.wl.B)], axis=0)


def draw(wl: Workload, run_id: int = 0) -> Draw:
    """Inputs of one run: p_h, W and contexts from their own streams; each
    per-token stream (h, q, k, v) spawned into one child per sequence."""
    return Draw(wl, run_id)


# ---------------------------------------------------------------------------
# order statistics and redraws (the caller supplies the logits)

def offset_for_fraction(pre_offset_logits: np.ndarray, p: float) -> float:
    """Offset o such that exactly round(p*n) of the values u satisfy u - o > 0.

    ``pre_offset_logits`` are the scaled decision values of one head before the
    offset is subtracted, pooled over every token of the run.  The offset is the
    midpoint of the two order statistics that bracket the (1-p) quantile.
    """
    u = np.sort(np.asarray(pre_offset_logits, dtype=np.float64).ravel())
    n = u.size
    kept = int(round((1.0 - p) * n))
    if kept <= 0:
        return float(u[0] - 1.0)
    if kept >= n:
        return float(u[-1] + 1.0)
    return float(0.5 * (u[kept - 1] + u[kept]))


def redraw(gen: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Fresh N(0,1) values from the resample stream (for rows that sit too close
    to the decision threshold)."""
    return normal(gen, shape, dtype)
