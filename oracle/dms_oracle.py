"""CPU oracle for the Dynamic Memory Sparsification (DMS) inference hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares
no code with the HIP library (no kernels, headers, helpers, tables or constant
generators) and never imports it.  It is plain, slow and sequential on purpose,
computes in float64, and every function cites the passage of the pages it
follows.

Pages cited (by title and section):

* "基于 DMS 的 KV Cache 压缩实战：为 Qwen3-8B 训练驱逐适配器" (the Model-Optimizer
  experimental/dms walkthrough; below: *DMS walkthrough*), sections
  决策来源一 / 决策来源二 (decision sources), 决策粒度 (granularity),
  Qwen3ConfigDMS parameter table and its hard constraints, Gumbel 噪声与可微门控
  (inference hard threshold), 训练模式 score_mod (window term), 推理模式
  (paged cache, in-place overwrite), 延迟驱逐 (delayed eviction),
  损失函数与压缩比调度 (dms_cr monitoring formula).
* FastDMS post on ai-navigate-news (below: *FastDMS post*), quality table
  (no-evict reference) and subsystem table (compact KV, FP8 after eviction).
* "Nvidia 的新技术将 LLM 推理成本降低 8 倍且不失准确性" (below: *VentureBeat
  piece*), sections on delayed eviction and the sliding-window heuristic.

Readings where the pages are silent or garbled are listed next to the function
that takes them (R-numbers match the design notes).

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
something other than itself (library routines, closed forms, brute force,
invariants) — see that file.  Attention values at the full workload sizes are
pinned only through those reductions (the pages print no worked example).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# 1. Decision (DMS walkthrough, 决策来源一 / 决策来源二 / 决策粒度; hard threshold
#    at inference in the Gumbel section).


def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x = h / sqrt(mean(h^2) + eps) * gamma over the last axis (float64).

    The separate adapter normalises the pre-attention hidden state with its own
    RMSNorm (DMS walkthrough, 决策来源二: ``dms_proj_alpha_norm``).  Reading R5:
    eps is a parameter (1e-6 in every workload).
    """
    h = np.asarray(h, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return h * r * np.asarray(gamma, dtype=np.float64)


def _threshold(logits: np.ndarray, alpha_per: str, disable_eviction: bool):
    """Granularity, then the hard threshold ``decision = logit > 0``.

    DMS walkthrough, 决策粒度: ``head`` lets each KV head decide on its own;
    ``layer`` makes every head of the layer share one decision.  Reading R8:
    the shared decision is head 0's.  Gumbel section: at inference the decision
    is the plain threshold ``logits > 0`` (reading R12: a logit of exactly 0
    keeps the token).  Qwen3ConfigDMS table: ``dms_disable_eviction`` turns the
    model back into a vanilla one, i.e. nothing is ever evicted.
    """
    if alpha_per == "layer":
        logits = np.repeat(logits[:, :1, :], logits.shape[1], axis=1)
    elif alpha_per != "head":
        raise ValueError("alpha_per must be 'head' or 'layer'")
    evict = (logits > 0.0).astype(np.uint8)
    if disable_eviction:
        evict[...] = 0
    return logits, evict


def decide_linear(h: np.ndarray, gamma: np.ndarray, W: np.ndarray, offsets: np.ndarray, *,
                  alpha_scale: float, eps: float, bias: Optional[np.ndarray] = None,
                  alpha_per: str = "head", disable_eviction: bool = False):
    """Decision logits from the separate linear adapter.

    DMS walkthrough, 决策来源二: logit = Linear(RMSNorm(h)) * scale - offset,
    with ``Linear(hidden, num_kv_heads)``; the (B, T, Hkv) projection is
    transposed to (B, Hkv, T).  Reading R10: one offset per KV head.  Reading
    R7: no bias unless given.

    h: [B, T, H]; W: [Hkv, H]; offsets: [Hkv].  Returns (logits [B, Hkv, T]
    float64, evict [B, Hkv, T] uint8).
    """
    x = rmsnorm(h, gamma, eps)                              # [B, T, H]
    z = x @ np.asarray(W, dtype=np.float64).T               # [B, T, Hkv]
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)
    logits = alpha_scale * z - np.asarray(offsets, dtype=np.float64)
    logits = np.ascontiguousarray(np.transpose(logits, (0, 2, 1)))
    return _threshold(logits, alpha_per, disable_eviction)


def decide_qneuron(q: np.ndarray, offsets: np.ndarray, *, num_kv_heads: int, alpha_scale: float,
                   alpha_per: str = "head", disable_eviction: bool = False):
    """Decision logits from the repurposed last query neuron.

    DMS walkthrough, 决策来源一: the logit is the last element of the first query
    head of every KV group (``query_states[:, ::gqa_factor, :, -1]``) times the
    scale minus the offset, and that element is then set to zero so it plays no
    further part in attention.  Reading R9: query head k*g belongs to KV head k
    (kv = q // g); RoPE is outside this path, so the zeroed q is what attention
    sees.

    q: [B, T, Hq, D].  Returns (logits [B, Hkv, T], evict [B, Hkv, T] uint8,
    q_zeroed [B, T, Hq, D] float64).
    """
    q = np.array(q, dtype=np.float64, copy=True)
    g = q.shape[2] // num_kv_heads
    z = q[:, :, ::g, -1]                                    # [B, T, Hkv]
    logits = alpha_scale * z - np.asarray(offsets, dtype=np.float64)
    logits = np.ascontiguousarray(np.transpose(logits, (0, 2, 1)))
    q[:, :, ::g, -1] = 0.0
    logits, evict = _threshold(logits, alpha_per, disable_eviction)
    return logits, evict, q


# ---------------------------------------------------------------------------
# 2. Visibility and attention.


def visible(e_row: np.ndarray, i: int, w: int) -> np.ndarray:
    """Boolean over keys j = 0..len(e_row)-1: is key j visible to query i?

    Delayed eviction (DMS walkthrough, 延迟驱逐; VentureBeat piece): a token
    marked for eviction stays usable until it leaves the sliding window, so key
    j is visible to query i iff j <= i and (j is kept, or i - j < w).  Reading
    R1: the window test is strict (``i - j < w``); the training score_mod keeps
    scores "within the sliding window" by the same test.
    """
    j = np.arange(len(e_row))
    return (j <= i) & ((np.asarray(e_row) == 0) | (i - j < w))


def visibility_mask(e_row: np.ndarray, w: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """[R, T] mask with M[r, j] = visible(e_row, rows[r], w)[j]."""
    T = len(e_row)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    i = rows[:, None]
    j = np.arange(T)[None, :]
    e = (np.asarray(e_row) != 0)[None, :]
    return (j <= i) & (~e | (i - j < w))


def attention_rows(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, e: np.ndarray, w: int,
                   rows: Sequence[int], scale: float) -> np.ndarray:
    """Masked softmax attention of selected query positions (GQA), float64.

    For query position i and query head h (KV head h // g):
    o = softmax_{j visible}(scale * <q, K_j>) · V_j.  Inference attention over
    the paged per-head cache computes exactly this (DMS walkthrough, 推理模式):
    the cache holds the visible set and nothing else.  Reading R11: scale is
    1/sqrt(D) unless given otherwise.

    q_rows: [R, Hq, D] queries at positions ``rows``; K, V: [T, Hkv, D];
    e: [Hkv, T] eviction flags.  Returns [R, Hq, D] float64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    rows = np.asarray(rows)
    R, Hq, D = q_rows.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    out = np.zeros((R, Hq, D), dtype=np.float64)
    for kh in range(Hkv):
        m = visibility_mask(e[kh], w, rows)                 # [R, T]
        for hq in range(kh * g, (kh + 1) * g):
            s = scale * (q_rows[:, hq, :] @ K[:, kh, :].T)  # [R, T]
            s = np.where(m, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[:, hq, :] = p @ V[:, kh, :]
    return out


def attention_over_keys(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * keys · q) · values for one query vector over a key list (float64)."""
    s = scale * (np.asarray(keys, dtype=np.float64) @ np.asarray(q, dtype=np.float64))
    s = s - s.max()
    p = np.exp(s)
    return (p / p.sum()) @ np.asarray(values, dtype=np.float64)


# ---------------------------------------------------------------------------
# 3. FP8 e4m3 storage (FastDMS post: FP8 compact KV, eviction applied before
#    quantisation).  Reading R15: OCP e4m3 "fn" (bias 7, no infinities, one NaN
#    pattern per sign, largest finite 448), round to nearest even, saturate to
#    the largest finite value; one power-of-two scale per (page, K or V).

E4M3_MAX = 448.0
SCALE_HEADROOM_BINADES = 2


def e4m3_value(code: int) -> float:
    """Value of an 8-bit e4m3fn code from the format's definition."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E are increasing in value.
_E4M3_POS = _E4M3_TABLE[:0x7F]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3fn value (ties to the even code), saturating at ±448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = (x < 0) & (code != 0)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(code, dtype=np.uint8)]


def page_scale(amax: float) -> float:
    """Power-of-two scale of a newly allocated page (reading R15).

    The smallest 2^e with amax <= 448 * 2^e, times 2^2 of headroom: the scale is
    fixed when the page is allocated and later writes into the page reuse it,
    so two spare binades keep later tokens from saturating.  amax = 0 takes
    e = -100.
    """
    if not amax > 0.0:
        return 2.0 ** (-100 + SCALE_HEADROOM_BINADES)
    m, k = math.frexp(amax)          # amax = m * 2^k, m in [0.5, 1)
    e = k - 9 + (1 if m > 0.875 else 0)   # 448 = 0.875 * 2^9
    return 2.0 ** (e + SCALE_HEADROOM_BINADES)


def fp8_roundtrip(x: np.ndarray, scale: float) -> np.ndarray:
    """dequant(quant(x)) with a per-page power-of-two scale: code(x / s) * s."""
    return e4m3_decode(e4m3_encode(np.asarray(x, dtype=np.float64) / scale)) * scale


# ---------------------------------------------------------------------------
# 4. Paged per-head store with delayed eviction and a shared page pool.


class PoolExhausted(RuntimeError):
    pass


class CapacityExceeded(RuntimeError):
    pass


class CacheSim:
    """Sequential model of the paged per-head KV store.

    DMS walkthrough, 推理模式: the cache is managed in blocks (default 256);
    every batch element records its blocks in a block table; per-head lengths
    may differ.  On append, if the element at the end of the sliding window is
    marked for eviction the new token overwrites that slot in place, otherwise
    it takes the next free position.  Reading R3: the element at the end of the
    window for token t is t - w (only when t >= w).  The block table grows on
    demand; capacity is fixed up front (preallocation section).

    Pool order (reading, O5): the free stack starts so that pops return pages
    0, 1, 2, ...; within one append call, pages are handed out to (batch row,
    KV head) pairs in row-major order and, inside a pair, in token order.
    ``reset`` pushes a sequence's pages back in reverse page-table order
    (pairs in reverse order) so the next pops return them in original order.

    Reading R4: a multi-token (chunk) append gives exactly the slot table of
    token-by-token appends; only each slot's final occupant in the call is
    written.

    FP8 (reading R15): when a page is allocated, its K and V scales come from
    the largest magnitude among the values the allocating call writes into it;
    later writes reuse them.
    """

    def __init__(self, max_batch: int, num_kv_heads: int, window: int, block: int,
                 max_tokens: int, pool_pages: int, fp8: bool = False):
        if block <= 0 or window <= block:
            raise ValueError("need block > 0 and window > block")
        self.B_max, self.Hkv, self.w, self.P = max_batch, num_kv_heads, window, block
        self.max_tokens = max_tokens
        self.pool_pages = pool_pages
        self.fp8 = fp8
        self.free: List[int] = [pool_pages - 1 - i for i in range(pool_pages)]
        self.pos = [0] * max_batch
        self.L = [[0] * num_kv_heads for _ in range(max_batch)]
        self.pages: List[List[List[int]]] = [[[] for _ in range(num_kv_heads)] for _ in range(max_batch)]
        self.slot_of: List[List[List[int]]] = [[[] for _ in range(num_kv_heads)] for _ in range(max_batch)]
        self.e_hist: List[List[List[int]]] = [[[] for _ in range(num_kv_heads)] for _ in range(max_batch)]
        self.occupant: List[List[List[int]]] = [[[] for _ in range(num_kv_heads)] for _ in range(max_batch)]
        self.page_scale: Dict[int, Tuple[float, float]] = {}
        # per (b, k, t): scales of the page token t was written into (fp8), or None
        self.tok_scale: List[List[List[Optional[Tuple[float, float]]]]] = [
            [[] for _ in range(num_kv_heads)] for _ in range(max_batch)]

    # -- one append call -------------------------------------------------
    def append(self, seq_ids: Sequence[int], evict: np.ndarray,
               k: Optional[np.ndarray] = None, v: Optional[np.ndarray] = None) -> None:
        """Append T tokens to each listed sequence.

        evict: [B, Hkv, T] flags of the new tokens.  k, v: [B, T, Hkv, D] values
        (needed only to set fp8 page scales).
        """
        evict = np.asarray(evict)
        B, Hkv, T = evict.shape
        assert Hkv == self.Hkv and B == len(seq_ids)
        for b in seq_ids:
            if self.pos[b] + T > self.max_tokens:
                raise CapacityExceeded(f"sequence {b}: {self.pos[b]} + {T} > {self.max_tokens}")
        new_pages: List[Tuple[int, int, int, int]] = []     # (row, b, k, page)
        written: List[Tuple[int, int, int, int, int]] = []  # (row, b, k, t, slot)
        for row, b in enumerate(seq_ids):
            s0 = self.pos[b]
            for kh in range(Hkv):
                last_in_call: Dict[int, int] = {}
                for tt in range(T):
                    t = s0 + tt
                    e_t = int(evict[row, kh, tt] != 0)
                    hist = self.e_hist[b][kh]
                    if t >= self.w and hist[t - self.w] == 1:
                        slot = self.slot_of[b][kh][t - self.w]
                    else:
                        slot = self.L[b][kh]
                        self.L[b][kh] += 1
                        if slot % self.P == 0:
                            if not self.free:
                                raise PoolExhausted("no free page")
                            page = self.free.pop()
                            self.pages[b][kh].append(page)
                            new_pages.append((row, b, kh, page))
                    self.slot_of[b][kh].append(slot)
                    hist.append(e_t)
                    self.tok_scale[b][kh].append(None)
                    occ = self.occupant[b][kh]
                    if slot == len(occ):
                        occ.append(t)
                    else:
                        occ[slot] = t
                    last_in_call[slot] = t
                for slot, t in last_in_call.items():
                    written.append((row, b, kh, t, slot))
        for b in seq_ids:
            self.pos[b] += T
        if self.fp8:
            self._set_scales(seq_ids, new_pages, written, k, v)

    def _set_scales(self, seq_ids, new_pages, written, k, v):
        if k is None or v is None:
            raise ValueError("fp8 store needs the appended K/V values")
        s0 = {b: self.pos[b] - k.shape[1] for b in seq_ids}
        fresh = {page for (_, _, _, page) in new_pages}
        amax: Dict[int, List[float]] = {p: [0.0, 0.0] for p in fresh}
        for (row, b, kh, t, slot) in written:
            page = self.pages[b][kh][slot // self.P]
            if page in fresh:
                tt = t - s0[b]
                amax[page][0] = max(amax[page][0], float(np.max(np.abs(k[row, tt, kh]))))
                amax[page][1] = max(amax[page][1], float(np.max(np.abs(v[row, tt, kh]))))
        for page in fresh:
            self.page_scale[page] = (page_scale(amax[page][0]), page_scale(amax[page][1]))
        for (row, b, kh, t, slot) in written:
            page = self.pages[b][kh][slot // self.P]
            self.tok_scale[b][kh][t] = self.page_scale[page]

    # -- reset -------------------------------------------------------------
    def reset(self, seq_ids: Sequence[int]) -> None:
        """Free the listed sequences (DMS walkthrough, 当前限制: the cache is reset
        between independent sequences)."""
        for b in reversed(list(seq_ids)):
            for kh in reversed(range(self.Hkv)):
                for page in reversed(self.pages[b][kh]):
                    self.free.append(page)
                    self.page_scale.pop(page, None)
                self.pages[b][kh] = []
                self.L[b][kh] = 0
                self.slot_of[b][kh] = []
                self.e_hist[b][kh] = []
                self.occupant[b][kh] = []
                self.tok_scale[b][kh] = []
            self.pos[b] = 0

    # -- views ---------------------------------------------------------------
    def slot_table(self, b: int, kh: int) -> np.ndarray:
        """Position held by each slot 0..L-1."""
        return np.asarray(self.occupant[b][kh][: self.L[b][kh]], dtype=np.int64)

    def slot_meta(self, b: int, kh: int) -> np.ndarray:
        """Per slot: position | (eviction flag << 31), as int64."""
        occ = self.slot_table(b, kh)
        e = np.asarray(self.e_hist[b][kh], dtype=np.int64)
        return occ | (e[occ] << 31) if len(occ) else occ

    def ring(self, b: int, kh: int) -> Dict[int, Tuple[int, int]]:
        """(slot, flag) of the last w positions, keyed by position."""
        t_end = self.pos[b]
        out = {}
        for t in range(max(0, t_end - self.w), t_end):
            out[t] = (self.slot_of[b][kh][t], self.e_hist[b][kh][t])
        return out

    def resident_positions(self, b: int, kh: int) -> np.ndarray:
        return np.sort(self.slot_table(b, kh))

    def stats(self) -> Dict[str, float]:
        """Token and slot counts and the realised compression ratios.

        DMS walkthrough, 损失函数与压缩比调度: training logs
        dms_cr = 1 / (1 - closed_frac), a token-level ratio that ignores the
        window.  The cache-level ratio is tokens / live slots (reading R18).
        """
        tokens = sum(self.pos[b] * self.Hkv for b in range(self.B_max))
        live = sum(self.L[b][k] for b in range(self.B_max) for k in range(self.Hkv))
        closed = sum(sum(self.e_hist[b][k]) for b in range(self.B_max) for k in range(self.Hkv))
        return {
            "tokens": tokens,
            "live_slots": live,
            "pages": sum(len(self.pages[b][k]) for b in range(self.B_max) for k in range(self.Hkv)),
            "cache_cr": tokens / live if live else float("inf"),
            "token_cr": 1.0 / max(1e-12, 1.0 - closed / tokens) if tokens else 1.0,
        }


def pages_needed_worst(sim: "CacheSim", b: int, n: int) -> int:
    """Pool pages that appending n more tokens to sequence b takes when every
    new token is kept (the most any decisions can take: a marked new token can
    only save a slot later).  FastDMS post, subsystem table: admission by
    compact KV capacity.  Simulated on a copy of the cache model; -1 when the
    sequence would pass its capacity."""
    import copy
    if sim.pos[b] + n > sim.max_tokens:
        return -1
    trial = copy.deepcopy(sim)
    trial.free = list(range(10 ** 9, 10 ** 9 - n * sim.Hkv - 1, -1))   # never runs dry
    before = sum(len(trial.pages[b][k]) for k in range(sim.Hkv))
    if n:
        trial.append([b], np.zeros((1, sim.Hkv, n), dtype=np.uint8))
    return sum(len(trial.pages[b][k]) for k in range(sim.Hkv)) - before


def length_closed_form(e_row: np.ndarray, t: int, w: int) -> int:
    """Live slots of one head after token t: (t+1) - #{j <= t-w : e_j = 1}.

    Each token past the first w either takes a new slot or reuses the slot of
    the evicted token w positions back (推理模式), so every eviction that has
    left the window frees exactly one slot for reuse.
    """
    return (t + 1) - int(np.sum(np.asarray(e_row[: max(0, t - w + 1)]) != 0))


def effective_kv(sim: CacheSim, b: int, kh: int, x: np.ndarray, which: int, t0: int = 0) -> np.ndarray:
    """Values attention reads for one head's tokens: raw, or fp8-rounded with their page scale.

    x: [T, D] raw values of positions t0..t0+T-1; which: 0 for K, 1 for V.
    Tokens never written (overwritten inside the call that appended them) keep
    their raw value; they are never visible from later calls.  A token's scale
    is fixed when the call that appends it ends, so a range can be taken once.
    """
    x = np.asarray(x, dtype=np.float64)
    if not sim.fp8:
        return x
    sc = np.array([s[which] if s is not None else np.nan
                   for s in sim.tok_scale[b][kh][t0: t0 + x.shape[0]]])
    if len(sc) < x.shape[0]:
        sc = np.concatenate([sc, np.full(x.shape[0] - len(sc), np.nan)])
    written = ~np.isnan(sc)
    out = x.copy()
    if written.any():
        s = sc[written][:, None]
        out[written] = e4m3_decode(e4m3_encode(x[written] / s)) * s
    return out
