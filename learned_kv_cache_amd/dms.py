"""ctypes binding of libdms (include/dms.h): argument marshalling only.

Every function here checks shapes/dtypes/devices of torch tensors, turns them
into raw pointers and calls the C ABI function of the same name.  All the
work runs in the HIP kernels of libdms.so; there is no fallback.  PyTorch
supplies device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdms.so")
_PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdms_probe.so")
_lib = None
_probe = None

PROBE_EXPORTS = ("dms_probe_read", "dms_probe_read_bytes", "dms_probe_mfma_bf16", "dms_probe_mfma_bf16_flops")

DMS_OK = 0
DMS_ERR_ARG = -1
DMS_ERR_CONFIG = -2
DMS_ERR_CAPACITY = -3
DMS_ERR_POOL = -4
DMS_ERR_HIP = -5
DMS_ERR_UNSUPPORTED = -6

DMS_DEV_POOL_EXHAUSTED = 0x1
DMS_DEV_CAPACITY = 0x2
DMS_DEV_BAD_SEQ = 0x4
DMS_DEV_STEP_SYNC = 0x8

DMS_F32, DMS_BF16, DMS_FP8_E4M3 = 0, 1, 2
DMS_DECIDE_LINEAR, DMS_DECIDE_QNEURON = 0, 1
DMS_ALPHA_PER_HEAD, DMS_ALPHA_PER_LAYER = 0, 1

KV_DTYPES = {"f32": DMS_F32, "bf16": DMS_BF16, "fp8": DMS_FP8_E4M3}

EXPORTS = (
    "dms_config_validate", "dms_cache_bytes", "dms_max_pages_per_seq", "dms_cache_create",
    "dms_cache_destroy", "dms_cache_config", "dms_decide", "dms_append_evict", "dms_decode_attn",
    "dms_prefill_attn", "dms_seq_reset", "dms_cache_status", "dms_cache_clear_status",
    "dms_cache_dump", "dms_cache_stats", "dms_last_error", "dms_decode_prepare", "dms_decode_step",
    "dms_train_gate", "dms_train_gate_bwd", "dms_train_attn_fwd", "dms_seq_info_get", "dms_pages_needed",
    "dms_kvzap_score", "dms_kvzap_workspace_bytes", "dms_train_attn_bwd", "dms_train_attn_bwd_workspace_bytes",
    "dms_decode_workspace_bytes", "dms_decode_attn_noalloc", "dms_cache_check",
    "dms_step_layers_create", "dms_step_layers_run", "dms_step_layers_one_launch", "dms_step_layers_destroy",
)


class DmsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class dms_config(ctypes.Structure):
    _fields_ = [
        ("max_batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("hidden", ctypes.c_int32), ("window", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("max_tokens_per_seq", ctypes.c_int32), ("pool_pages", ctypes.c_int32),
        ("max_chunk", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("decide_mode", ctypes.c_int32),
        ("alpha_per", ctypes.c_int32), ("disable_eviction", ctypes.c_int32), ("alpha_scale", ctypes.c_float),
        ("rms_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
    ]


class dms_dump(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "lengths", "page_table", "slot_meta", "ring", "positions", "free_stack", "free_count",
        "k_pages", "v_pages", "page_scales")]


class dms_seq_info(ctypes.Structure):
    _fields_ = [("position", ctypes.c_int32), ("live_slots", ctypes.c_int32), ("max_head_slots", ctypes.c_int32),
                ("pages", ctypes.c_int32)]


class dms_layer_io(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "hidden", "rms_gamma", "W", "bias", "offsets", "q_inout", "k", "v", "out", "logits_out", "evict_out")]


class dms_stats(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("live_slots", ctypes.c_int64), ("pages_in_use", ctypes.c_int64),
                ("bytes_live", ctypes.c_int64), ("bytes_allocated", ctypes.c_int64), ("cache_cr", ctypes.c_double)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Loads libdms.so (built by ``python -m learned_kv_cache_amd.build``); raises if missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m learned_kv_cache_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        cfgp = ctypes.POINTER(dms_config)
        sig = {
            "dms_config_validate": [cfgp],
            "dms_cache_bytes": [cfgp, ctypes.POINTER(sz)],
            "dms_max_pages_per_seq": [cfgp, ctypes.POINTER(ctypes.c_int32)],
            "dms_cache_create": [cfgp, vp, sz, vp, ctypes.POINTER(vp)],
            "dms_cache_destroy": [vp],
            "dms_cache_config": [vp, cfgp],
            "dms_decide": [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp],
            "dms_append_evict": [vp, vp, vp, vp, vp, i32, i32, vp],
            "dms_decode_attn": [vp, vp, vp, vp, i32, vp, sz, vp],
            "dms_decode_workspace_bytes": [cfgp, i32, ctypes.POINTER(sz)],
            "dms_decode_attn_noalloc": [vp, vp, vp, vp, i32, vp],
            "dms_decode_prepare": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp],
            "dms_decode_step": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp],
            "dms_train_gate": [vp, vp, ctypes.c_float, ctypes.c_int64, vp, vp, vp, vp],
            "dms_train_gate_bwd": [vp, vp, ctypes.c_float, ctypes.c_int64, vp, vp, vp, vp, vp],
            "dms_cache_check": [vp, vp, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_int32)],
            "dms_step_layers_create": [ctypes.POINTER(vp), ctypes.POINTER(dms_layer_io), i32, ctypes.POINTER(vp)],
            "dms_step_layers_run": [vp, vp, i32, vp, sz, vp],
            "dms_step_layers_one_launch": [vp, i32, ctypes.POINTER(ctypes.c_int32)],
            "dms_step_layers_destroy": [vp],
            "dms_seq_info_get": [vp, vp, i32, vp, ctypes.POINTER(dms_seq_info)],
            "dms_pages_needed": [vp, vp, vp, i32, vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)],
            "dms_train_attn_fwd": [i32, i32, i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp],
            "dms_kvzap_score": [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                ctypes.c_size_t, vp],
            "dms_kvzap_workspace_bytes": [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)],
            "dms_train_attn_bwd": [i32, i32, i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   vp, vp, vp, ctypes.c_size_t, vp],
            "dms_train_attn_bwd_workspace_bytes": [i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)],
            "dms_prefill_attn": [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp],
            "dms_seq_reset": [vp, vp, i32, vp],
            "dms_cache_status": [vp, vp, ctypes.POINTER(ctypes.c_int32)],
            "dms_cache_clear_status": [vp, vp],
            "dms_cache_dump": [vp, vp, ctypes.POINTER(dms_dump)],
            "dms_cache_stats": [vp, vp, ctypes.POINTER(dms_stats)],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.dms_last_error.argtypes = []
        L.dms_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def probe_lib():
    """Loads libdms_probe.so (include/dms_probe.h: HBM read and bf16 matrix-core rate probes)."""
    global _probe
    if _probe is None:
        if not os.path.exists(_PROBE_PATH):
            raise RuntimeError(f"{_PROBE_PATH} is not built; run `python -m learned_kv_cache_amd.build`")
        L = ctypes.CDLL(_PROBE_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.dms_probe_read.argtypes = [vp, sz, i32, i32, vp, vp]
        L.dms_probe_read.restype = ctypes.c_int
        L.dms_probe_read_bytes.argtypes = [sz, i32, i32]
        L.dms_probe_read_bytes.restype = sz
        L.dms_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
        L.dms_probe_mfma_bf16.restype = ctypes.c_int
        L.dms_probe_mfma_bf16_flops.argtypes = [i32, i32]
        L.dms_probe_mfma_bf16_flops.restype = ctypes.c_double
        _probe = L
    return _probe


def probe_read(buf: torch.Tensor, grid: int, unroll: int, sink: torch.Tensor, stream=None) -> int:
    """One streaming read of `buf` (dms_probe_read); returns the bytes read."""
    L = probe_lib()
    nbytes = buf.numel() * buf.element_size()
    if L.dms_probe_read(_ptr(buf, "buf"), nbytes, grid, unroll, _ptr(sink, "sink"), _stream(stream)) != 0:
        raise RuntimeError("dms_probe_read failed")
    return int(L.dms_probe_read_bytes(nbytes, grid, unroll))


def probe_mfma_bf16(grid: int, iters: int, sink: torch.Tensor, stream=None) -> float:
    """One bf16 matrix-core loop (dms_probe_mfma_bf16); returns its flops."""
    L = probe_lib()
    if L.dms_probe_mfma_bf16(grid, iters, _ptr(sink, "sink"), _stream(stream)) != 0:
        raise RuntimeError("dms_probe_mfma_bf16 failed")
    return float(L.dms_probe_mfma_bf16_flops(grid, iters))


def _check(status: int) -> int:
    if status != DMS_OK:
        raise DmsError(status, lib().dms_last_error().decode())
    return status


def make_config(*, max_batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, hidden: int,
                window: int, block_size: int, max_tokens_per_seq: int, pool_pages: int, max_chunk: int,
                kv_dtype: str = "bf16", decide_mode: str = "linear", alpha_per: str = "head",
                disable_eviction: bool = False, alpha_scale: float = 100.0, rms_eps: float = 1e-6,
                softmax_scale: float = 0.0) -> dms_config:
    return dms_config(
        max_batch, num_q_heads, num_kv_heads, head_dim, hidden, window, block_size, max_tokens_per_seq,
        pool_pages, max_chunk, KV_DTYPES[kv_dtype], DMS_DECIDE_LINEAR if decide_mode == "linear" else DMS_DECIDE_QNEURON,
        DMS_ALPHA_PER_HEAD if alpha_per == "head" else DMS_ALPHA_PER_LAYER, int(disable_eviction),
        alpha_scale, rms_eps, softmax_scale)


def dms_config_validate(cfg: dms_config) -> int:
    return _check(lib().dms_config_validate(ctypes.byref(cfg)))


def dms_cache_bytes(cfg: dms_config) -> int:
    n = ctypes.c_size_t()
    _check(lib().dms_cache_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def dms_decode_workspace_bytes(cfg: dms_config, B: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().dms_decode_workspace_bytes(ctypes.byref(cfg), B, ctypes.byref(n)))
    return n.value


def decode_workspace(cfg: dms_config, B: int, device: str = "cuda") -> torch.Tensor:
    """A device uint8 tensor of dms_decode_workspace_bytes(cfg, B) bytes (torch's
    allocator returns 256-byte aligned blocks).  One can serve every cache of a
    stream in turn."""
    return torch.empty(dms_decode_workspace_bytes(cfg, B), dtype=torch.uint8, device=device)


def _ws(cache: "DmsCache", workspace, B: int):
    """(pointer, bytes) of the caller's decode workspace, or of the cache's own
    one (allocated on first use, for B = max_batch) when none is given."""
    if workspace is None:
        if cache.workspace is None:
            cache.workspace = decode_workspace(cache.cfg, cache.cfg.max_batch)
        workspace = cache.workspace
    return _ptr(workspace, "workspace"), ctypes.c_size_t(workspace.numel() * workspace.element_size())


def dms_max_pages_per_seq(cfg: dms_config) -> int:
    n = ctypes.c_int32()
    _check(lib().dms_max_pages_per_seq(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel=None, device=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t.data_ptr()


class DmsCache:
    """One layer's cache: owns the device buffer (a torch uint8 tensor) and the handle."""

    def __init__(self, cfg: dms_config, device: str = "cuda", stream=None):
        self.cfg = cfg
        nbytes = dms_cache_bytes(cfg)
        self.buffer = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = self.buffer.data_ptr()
        self._base = (base + 255) // 256 * 256
        self.max_pages = dms_max_pages_per_seq(cfg)
        h = ctypes.c_void_p()
        _check(lib().dms_cache_create(ctypes.byref(cfg), self._base, nbytes, _stream(stream), ctypes.byref(h)))
        self.handle = h
        self.act_dtype = torch.float32 if cfg.kv_dtype == DMS_F32 else torch.bfloat16
        self.workspace = None   # decode workspace used when a call passes none

    def close(self):
        if self.handle:
            lib().dms_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dms_decide(cache: DmsCache, hidden, rms_gamma, W, bias, offsets, q_inout, B: int, T: int,
               logits_out, evict_out, stream=None) -> int:
    c = cache.cfg
    ad = cache.act_dtype
    if c.decide_mode == DMS_DECIDE_LINEAR:
        hp = _ptr(hidden, "hidden", ad, B * T * c.hidden)
        gp = _ptr(rms_gamma, "rms_gamma", torch.float32, c.hidden)
        wp = _ptr(W, "W", torch.float32, c.num_kv_heads * c.hidden)
        qp = None
    else:
        hp = gp = wp = None
        qp = _ptr(q_inout, "q_inout", ad, B * T * c.num_q_heads * c.head_dim)
    bp = _ptr(bias, "bias", torch.float32, c.num_kv_heads)
    op = _ptr(offsets, "offsets", torch.float32, c.num_kv_heads)
    lp = _ptr(logits_out, "logits_out", torch.float32, B * c.num_kv_heads * T)
    ep = _ptr(evict_out, "evict_out", torch.uint8, B * c.num_kv_heads * T)
    return _check(lib().dms_decide(cache.handle, hp, gp, wp, bp, op, qp, B, T, lp, ep, _stream(stream)))


def dms_append_evict(cache: DmsCache, seq_ids, k, v, evict, B: int, T: int, stream=None) -> int:
    c = cache.cfg
    n = B * T * c.num_kv_heads * c.head_dim
    sp = _ptr(seq_ids, "seq_ids", torch.int32, B)
    return _check(lib().dms_append_evict(
        cache.handle, sp, _ptr(k, "k", cache.act_dtype, n), _ptr(v, "v", cache.act_dtype, n),
        _ptr(evict, "evict", torch.uint8, B * c.num_kv_heads * T), B, T, _stream(stream)))


def dms_decode_prepare(cache: DmsCache, seq_ids, hidden, rms_gamma, W, bias, offsets, q_inout, k, v, B: int,
                       logits_out, evict_out, stream=None) -> int:
    c = cache.cfg
    ad = cache.act_dtype
    if c.decide_mode == DMS_DECIDE_LINEAR:
        hp = _ptr(hidden, "hidden", ad, B * c.hidden)
        gp = _ptr(rms_gamma, "rms_gamma", torch.float32, c.hidden)
        wp = _ptr(W, "W", torch.float32, c.num_kv_heads * c.hidden)
        qp = None
    else:
        hp = gp = wp = None
        qp = _ptr(q_inout, "q_inout", ad, B * c.num_q_heads * c.head_dim)
    n = B * c.num_kv_heads * c.head_dim
    return _check(lib().dms_decode_prepare(
        cache.handle, _ptr(seq_ids, "seq_ids", torch.int32, B), hp, gp, wp, _ptr(bias, "bias", torch.float32, c.num_kv_heads),
        _ptr(offsets, "offsets", torch.float32, c.num_kv_heads), qp, _ptr(k, "k", ad, n), _ptr(v, "v", ad, n), B,
        _ptr(logits_out, "logits_out", torch.float32, B * c.num_kv_heads),
        _ptr(evict_out, "evict_out", torch.uint8, B * c.num_kv_heads), _stream(stream)))


def dms_decode_step(cache: DmsCache, seq_ids, hidden, rms_gamma, W, bias, offsets, q_inout, k, v, out, B: int,
                    logits_out, evict_out, workspace=None, stream=None) -> int:
    c = cache.cfg
    ad = cache.act_dtype
    if c.decide_mode == DMS_DECIDE_LINEAR:
        hp = _ptr(hidden, "hidden", ad, B * c.hidden)
        gp = _ptr(rms_gamma, "rms_gamma", torch.float32, c.hidden)
        wp = _ptr(W, "W", torch.float32, c.num_kv_heads * c.hidden)
    else:
        hp = gp = wp = None
    nq = B * c.num_q_heads * c.head_dim
    n = B * c.num_kv_heads * c.head_dim
    return _check(lib().dms_decode_step(
        cache.handle, _ptr(seq_ids, "seq_ids", torch.int32, B), hp, gp, wp,
        _ptr(bias, "bias", torch.float32, c.num_kv_heads), _ptr(offsets, "offsets", torch.float32, c.num_kv_heads),
        _ptr(q_inout, "q_inout", ad, nq), _ptr(k, "k", ad, n), _ptr(v, "v", ad, n), _ptr(out, "out", ad, nq), B,
        _ptr(logits_out, "logits_out", torch.float32, B * c.num_kv_heads),
        _ptr(evict_out, "evict_out", torch.uint8, B * c.num_kv_heads), *_ws(cache, workspace, B), _stream(stream)))


class StepLayers:
    """dms_step_layers: the decode step of every layer in one launch.

    caches: the layers' DmsCache objects (one shape); io: per layer a dict of
    device tensors sized for max_batch rows, with the keys of dms_layer_io
    (hidden, rms_gamma, W, bias, offsets, q_inout, k, v, out, logits_out,
    evict_out; hidden / rms_gamma / W only for the linear decision, bias and
    logits_out optional).  The tensors are bound, not copied: each run reads
    and writes them (rows [0, B) of a call)."""

    def __init__(self, caches: Sequence[DmsCache], io: Sequence[dict]):
        if len(caches) != len(io):
            raise ValueError("one io dict per cache")
        c = caches[0].cfg
        ad = caches[0].act_dtype
        Bm = c.max_batch
        nq = Bm * c.num_q_heads * c.head_dim
        n = Bm * c.num_kv_heads * c.head_dim
        arr = (dms_layer_io * len(caches))()
        self._keep = []
        for i, d in enumerate(io):
            lin = c.decide_mode == DMS_DECIDE_LINEAR
            arr[i].hidden = _ptr(d.get("hidden"), "hidden", ad, Bm * c.hidden) if lin else None
            arr[i].rms_gamma = _ptr(d.get("rms_gamma"), "rms_gamma", torch.float32, c.hidden) if lin else None
            arr[i].W = _ptr(d.get("W"), "W", torch.float32, c.num_kv_heads * c.hidden) if lin else None
            arr[i].bias = _ptr(d.get("bias"), "bias", torch.float32, c.num_kv_heads)
            arr[i].offsets = _ptr(d.get("offsets"), "offsets", torch.float32, c.num_kv_heads)
            arr[i].q_inout = _ptr(d.get("q_inout"), "q_inout", ad, nq)
            arr[i].k = _ptr(d.get("k"), "k", ad, n)
            arr[i].v = _ptr(d.get("v"), "v", ad, n)
            arr[i].out = _ptr(d.get("out"), "out", ad, nq)
            arr[i].logits_out = _ptr(d.get("logits_out"), "logits_out", torch.float32, Bm * c.num_kv_heads)
            arr[i].evict_out = _ptr(d.get("evict_out"), "evict_out", torch.uint8, Bm * c.num_kv_heads)
            self._keep.append(dict(d))
        handles = (ctypes.c_void_p * len(caches))(*[x.handle.value for x in caches])
        h = ctypes.c_void_p()
        _check(lib().dms_step_layers_create(handles, arr, len(caches), ctypes.byref(h)))
        self.handle = h
        self.caches = list(caches)

    def run(self, seq_ids, B: int, workspace=None, stream=None) -> int:
        c = self.caches[0]
        return _check(lib().dms_step_layers_run(self.handle, _ptr(seq_ids, "seq_ids", torch.int32, B), B,
                                                *_ws(c, workspace, B), _stream(stream)))

    def one_launch(self, B: int) -> bool:
        r = ctypes.c_int32()
        _check(lib().dms_step_layers_one_launch(self.handle, B, ctypes.byref(r)))
        return bool(r.value)

    def close(self):
        if self.handle:
            lib().dms_step_layers_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dms_train_gate(logits, noise, tau: float, y_out=None, probs_out=None, hard_out=None, stream=None) -> int:
    n = logits.numel()
    return _check(lib().dms_train_gate(
        _ptr(logits, "logits", torch.float32), _ptr(noise, "noise", torch.float32, n), ctypes.c_float(tau),
        ctypes.c_int64(n), _ptr(y_out, "y_out", torch.float32, n), _ptr(probs_out, "probs_out", torch.float32, n),
        _ptr(hard_out, "hard_out", torch.float32, n), _stream(stream)))


def dms_cache_check(cache: DmsCache, stream=None):
    """(violation bits, first unit found wrong or -1); bits 0 = consistent."""
    bits, unit = ctypes.c_uint32(), ctypes.c_int32()
    _check(lib().dms_cache_check(cache.handle, _stream(stream), ctypes.byref(bits), ctypes.byref(unit)))
    return int(bits.value), int(unit.value)


def dms_train_gate_bwd(logits, noise, tau: float, dlogits_out, dy=None, dhard=None, dprobs=None,
                       stream=None) -> int:
    n = logits.numel()
    return _check(lib().dms_train_gate_bwd(
        _ptr(logits, "logits", torch.float32), _ptr(noise, "noise", torch.float32, n), ctypes.c_float(tau),
        ctypes.c_int64(n), _ptr(dy, "dy", torch.float32, n), _ptr(dhard, "dhard", torch.float32, n),
        _ptr(dprobs, "dprobs", torch.float32, n), _ptr(dlogits_out, "dlogits_out", torch.float32, n),
        _stream(stream)))


def dms_train_attn_fwd(q, k, v, gate_logits, out, lse, *, window: int, softmax_scale: float = 0.0,
                       stream=None) -> int:
    """q [B, T, Hq, D], k/v [B, T, Hkv, D] bf16; gate_logits [B, Hkv, T] f32; out like q; lse [B, Hq, T] f32."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, T, Hkv, D) or tuple(v.shape) != (B, T, Hkv, D):
        raise ValueError("k and v must be [B, T, Hkv, D] like q")
    return _check(lib().dms_train_attn_fwd(
        B, T, Hq, Hkv, D, window, ctypes.c_float(softmax_scale), _ptr(q, "q", torch.bfloat16),
        _ptr(k, "k", torch.bfloat16), _ptr(v, "v", torch.bfloat16),
        _ptr(gate_logits, "gate_logits", torch.float32, B * Hkv * T), _ptr(out, "out", torch.bfloat16, q.numel()),
        _ptr(lse, "lse", torch.float32, B * Hq * T), _stream(stream)))


def dms_train_attn_bwd_workspace_bytes(B: int, T: int, Hq: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().dms_train_attn_bwd_workspace_bytes(B, T, Hq, ctypes.byref(n)))
    return n.value


def dms_train_attn_bwd(q, k, v, out, dout, gate_logits, lse, dq, dk, dv, dgate, *, window: int,
                       softmax_scale: float = 0.0, workspace=None, stream=None) -> int:
    """Gradients of dms_train_attn_fwd.  q, out, dout [B, T, Hq, D] and k, v
    [B, T, Hkv, D] bf16; gate_logits [B, Hkv, T] and lse [B, Hq, T] f32; dq,
    dk, dv f32 like q, k, v; dgate f32 like gate_logits.  workspace: a device
    uint8 tensor of dms_train_attn_bwd_workspace_bytes bytes (allocated here
    when not given)."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if workspace is None:
        n = dms_train_attn_bwd_workspace_bytes(B, T, Hq)
        workspace = torch.empty(max(1, n), dtype=torch.uint8, device=q.device)
    nq, nk = B * T * Hq * D, B * T * Hkv * D
    return _check(lib().dms_train_attn_bwd(
        B, T, Hq, Hkv, D, window, ctypes.c_float(softmax_scale), _ptr(q, "q", torch.bfloat16, nq),
        _ptr(k, "k", torch.bfloat16, nk), _ptr(v, "v", torch.bfloat16, nk), _ptr(out, "out", torch.bfloat16, nq),
        _ptr(dout, "dout", torch.bfloat16, nq), _ptr(gate_logits, "gate_logits", torch.float32, B * Hkv * T),
        _ptr(lse, "lse", torch.float32, B * Hq * T), _ptr(dq, "dq", torch.float32, nq),
        _ptr(dk, "dk", torch.float32, nk), _ptr(dv, "dv", torch.float32, nk),
        _ptr(dgate, "dgate", torch.float32, B * Hkv * T), _ptr(workspace, "workspace"),
        ctypes.c_size_t(workspace.numel()), _stream(stream)))


def dms_kvzap_workspace_bytes(B: int, T: int, Hkv: int, Hm: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().dms_kvzap_workspace_bytes(B, T, Hkv, Hm, ctypes.byref(n)))
    return n.value


def dms_kvzap_score(hidden, W1, b1, evict_out, *, W2=None, b2=None, threshold: float = -4.0, scores_out=None,
                    workspace=None, stream=None) -> int:
    """KVzap scores and decisions.  hidden [B, T, H] f32 or bf16; linear: W1 [Hkv, H],
    b1 [Hkv] or None; MLP (W2 given): W1 [Hm, H], b1 [Hm] or None, W2 [Hkv, Hm],
    b2 [Hkv] or None.  evict_out uint8 and scores_out f32 (optional) are [B, Hkv, T].
    The MLP needs a device workspace of dms_kvzap_workspace_bytes bytes (a uint8
    tensor; allocated here when not given)."""
    B, T, H = hidden.shape
    if hidden.dtype == torch.float32:
        act = DMS_F32
    elif hidden.dtype == torch.bfloat16:
        act = DMS_BF16
    else:
        raise ValueError("hidden must be float32 or bfloat16")
    mlp = W2 is not None
    Hkv = W2.shape[0] if mlp else W1.shape[0]
    Hm = W1.shape[0] if mlp else 0
    if W1.shape[1] != H or (mlp and W2.shape[1] != Hm):
        raise ValueError("weight shapes do not match the hidden size")
    n = B * Hkv * T
    ws_bytes = dms_kvzap_workspace_bytes(B, T, Hkv, Hm)
    if mlp and workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=hidden.device)
    ws_ptr = _ptr(workspace, "workspace") if mlp else None
    ws_len = workspace.numel() * workspace.element_size() if (mlp and workspace is not None) else 0
    return _check(lib().dms_kvzap_score(
        B, T, H, Hkv, Hm, act, _ptr(hidden, "hidden"), _ptr(W1, "W1", torch.float32, W1.shape[0] * H),
        _ptr(b1, "b1", torch.float32, W1.shape[0]), _ptr(W2, "W2", torch.float32, Hkv * Hm if mlp else None),
        _ptr(b2, "b2", torch.float32, Hkv), ctypes.c_float(threshold), _ptr(scores_out, "scores_out", torch.float32, n),
        _ptr(evict_out, "evict_out", torch.uint8, n), ws_ptr, ctypes.c_size_t(ws_len), _stream(stream)))


def _host_ids(seq_ids):
    ids = (ctypes.c_int32 * len(seq_ids))(*[int(x) for x in seq_ids])
    return ids


def dms_seq_info_get(cache: DmsCache, seq_ids, stream=None):
    """Per-sequence accounting (synchronises): list of dicts with position,
    live_slots, max_head_slots, pages."""
    n = len(seq_ids)
    out = (dms_seq_info * n)()
    _check(lib().dms_seq_info_get(cache.handle, _host_ids(seq_ids), n, _stream(stream), out))
    return [{f: getattr(r, f) for f, _ in dms_seq_info._fields_} for r in out]


def dms_pages_needed(cache: DmsCache, seq_ids, n_new, stream=None):
    """Worst-case pool pages for appending n_new[i] tokens to seq_ids[i]
    (synchronises).  Returns (pages list, free pages)."""
    n = len(seq_ids)
    pages = (ctypes.c_int64 * n)()
    free = ctypes.c_int64(0)
    counts = (ctypes.c_int32 * n)(*[int(x) for x in n_new])
    _check(lib().dms_pages_needed(cache.handle, _host_ids(seq_ids), counts, n, _stream(stream), pages,
                                  ctypes.byref(free)))
    return list(pages), free.value


def dms_decode_attn(cache: DmsCache, seq_ids, q, out, B: int, workspace=None, stream=None) -> int:
    c = cache.cfg
    n = B * c.num_q_heads * c.head_dim
    return _check(lib().dms_decode_attn(
        cache.handle, _ptr(seq_ids, "seq_ids", torch.int32, B), _ptr(q, "q", cache.act_dtype, n),
        _ptr(out, "out", cache.act_dtype, n), B, *_ws(cache, workspace, B), _stream(stream)))


def dms_decode_attn_noalloc(cache: DmsCache, seq_ids, q, out, B: int, stream=None) -> int:
    """dms_decode_attn with the library's static per-device scratch (no workspace, no allocation)."""
    c = cache.cfg
    n = B * c.num_q_heads * c.head_dim
    return _check(lib().dms_decode_attn_noalloc(
        cache.handle, _ptr(seq_ids, "seq_ids", torch.int32, B), _ptr(q, "q", cache.act_dtype, n),
        _ptr(out, "out", cache.act_dtype, n), B, _stream(stream)))


def dms_prefill_attn(cache: DmsCache, seq_ids, q, k, v, evict, out, B: int, C: int, stream=None) -> int:
    c = cache.cfg
    nq = B * C * c.num_q_heads * c.head_dim
    nk = B * C * c.num_kv_heads * c.head_dim
    return _check(lib().dms_prefill_attn(
        cache.handle, _ptr(seq_ids, "seq_ids", torch.int32, B), _ptr(q, "q", cache.act_dtype, nq),
        _ptr(k, "k", cache.act_dtype, nk), _ptr(v, "v", cache.act_dtype, nk),
        _ptr(evict, "evict", torch.uint8, B * c.num_kv_heads * C), _ptr(out, "out", cache.act_dtype, nq),
        B, C, _stream(stream)))


def dms_seq_reset(cache: DmsCache, seq_ids, n: int, stream=None) -> int:
    return _check(lib().dms_seq_reset(cache.handle, _ptr(seq_ids, "seq_ids", torch.int32, n), n, _stream(stream)))


def dms_cache_status(cache: DmsCache, stream=None) -> int:
    s = ctypes.c_int32()
    _check(lib().dms_cache_status(cache.handle, _stream(stream), ctypes.byref(s)))
    return s.value


def dms_cache_clear_status(cache: DmsCache, stream=None) -> int:
    return _check(lib().dms_cache_clear_status(cache.handle, _stream(stream)))


def dms_cache_stats(cache: DmsCache, stream=None) -> dict:
    st = dms_stats()
    _check(lib().dms_cache_stats(cache.handle, _stream(stream), ctypes.byref(st)))
    return {f: getattr(st, f) for f, _ in dms_stats._fields_}


_KV_NP = {DMS_F32: np.float32, DMS_BF16: np.uint16, DMS_FP8_E4M3: np.uint8}


def dms_cache_dump(cache: DmsCache, pages: bool = False, stream=None) -> dict:
    """Host copies of the tables (numpy).  pages=True also copies K/V page bytes and scales."""
    c = cache.cfg
    units = c.max_batch * c.num_kv_heads
    out = {
        "lengths": np.zeros((c.max_batch, c.num_kv_heads), np.int32),
        "page_table": np.zeros((c.max_batch, c.num_kv_heads, cache.max_pages), np.int32),
        "slot_meta": np.zeros((c.pool_pages, c.block_size), np.int32),
        "ring": np.zeros((c.max_batch, c.num_kv_heads, c.window), np.int32),
        "positions": np.zeros(c.max_batch, np.int32),
        "free_stack": np.zeros(c.pool_pages, np.int32),
        "free_count": np.zeros(1, np.int32),
    }
    if pages:
        et = _KV_NP[c.kv_dtype]
        out["k_pages"] = np.zeros((c.pool_pages, c.block_size, c.head_dim), et)
        out["v_pages"] = np.zeros((c.pool_pages, c.block_size, c.head_dim), et)
        out["page_scales"] = np.zeros((c.pool_pages, 2), np.float32)
    d = dms_dump(**{k: v.ctypes.data for k, v in out.items()})
    _check(lib().dms_cache_dump(cache.handle, _stream(stream), ctypes.byref(d)))
    assert units == out["lengths"].size
    return out
