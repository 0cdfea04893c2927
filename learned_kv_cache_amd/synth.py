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
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


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


@dataclasses.dataclass
class Draw:
    """All random inputs of one run (numpy float32 arrays holding the storage dtype's values).

    Per-token tensors are lists with one array per sequence, of length
    ``ctx[b] + decode_steps`` (ragged when the contexts are).
    """

    wl: Workload
    ctx: np.ndarray                  # [B] prompt lengths
    p_h: np.ndarray                  # [Hkv] target eviction fractions
    W: np.ndarray                    # [Hkv, hidden] float32 (linear adapter)
    gamma: np.ndarray                # [hidden] float32 (RMSNorm weight)
    h: Optional[List[np.ndarray]]    # B x [T_b, hidden]
    q: List[np.ndarray]              # B x [T_b, Hq, D]
    k: List[np.ndarray]              # B x [T_b, Hkv, D]
    v: List[np.ndarray]              # B x [T_b, Hkv, D]
    gens: Dict[str, np.random.Generator]

    def T(self, b: int) -> int:
        return int(self.ctx[b]) + self.wl.decode_steps

    def stacked(self, name: str) -> np.ndarray:
        """[B, T, ...] view of a per-token tensor (all sequences equally long)."""
        xs = getattr(self, name)
        return np.stack(xs, axis=0)


def draw(wl: Workload, run_id: int = 0, with_hidden: Optional[bool] = None) -> Draw:
    """Draw every random input of a run, stream by stream, in a fixed order.

    p_h, W and contexts come from their own streams.  Each per-token tensor
    stream (h, q, k, v) is spawned into one child per sequence.
    """
    ss = np.random.SeedSequence([1000 + wl.cfg_id, run_id])
    kids = dict(zip(STREAMS, ss.spawn(len(STREAMS))))
    gens = {name: np.random.Generator(np.random.PCG64(kids[name])) for name in STREAMS}
    p_h = eviction_fractions(wl, gens["p_h"])
    ctx = context_lengths(wl, gens["ctx"])
    if with_hidden is None:
        with_hidden = wl.decide == "linear"
    W = gens["W"].normal(0.0, wl.weight_std(), size=(wl.Hkv, wl.hidden)).astype(np.float32)
    gamma = np.ones(wl.hidden, dtype=np.float32)

    def per_seq(name, tail):
        out = []
        for b, child in enumerate(kids[name].spawn(wl.B)):
            gen = np.random.Generator(np.random.PCG64(child))
            out.append(normal(gen, (int(ctx[b]) + wl.decode_steps,) + tail, wl.act_dtype))
        return out

    h = per_seq("h", (wl.hidden,)) if with_hidden else None
    q = per_seq("q", (wl.Hq, wl.D))
    k = per_seq("k", (wl.Hkv, wl.D))
    v = per_seq("v", (wl.Hkv, wl.D))
    return Draw(wl=wl, ctx=ctx, p_h=p_h, W=W, gamma=gamma, h=h, q=q, k=k, v=v, gens=gens)


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


def redraw_rows(x: np.ndarray, rows: np.ndarray, gen: np.random.Generator, dtype: str) -> int:
    """Redraw x[rows] (boolean mask over the leading axes) from N(0,1) in place."""
    idx = np.argwhere(rows)
    for ix in idx:
        sl = tuple(int(i) for i in ix)
        x[sl] = normal(gen, x[sl].shape, dtype)
    return len(idx)


def redraw_elements(x: np.ndarray, mask: np.ndarray, gen: np.random.Generator, dtype: str) -> int:
    """Redraw the elements of x selected by a boolean mask of x's shape, in place."""
    n = int(mask.sum())
    if n:
        x[mask] = normal(gen, (n,), dtype)
    return n
