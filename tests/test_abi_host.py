"""Host-side checks of the C ABI (no GPU work): exports, configuration checks,
buffer sizing, and that the binding refuses to run without the library."""
import ctypes
import os
import re

import pytest

from learned_kv_cache_amd import dms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dms.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(dms_\w+)\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 15
    L = ctypes.CDLL(dms.library_path())
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(dms.EXPORTS)


def test_probe_library_exports_its_header():
    text = open(os.path.join(ROOT, "include", "dms_probe.h")).read()
    names = sorted(set(re.findall(r"^(?:int|size_t|double)\s+(dms_\w+)\(", text, flags=re.M)))
    assert set(names) == set(dms.PROBE_EXPORTS)
    L = ctypes.CDLL(os.path.join(os.path.dirname(dms.library_path()), "libdms_probe.so"))
    for n in names:
        assert hasattr(L, n), n
    P = dms.probe_lib()
    assert P.dms_probe_read(None, 1 << 20, 4, 8, None, None) == -1          # refused before any launch
    assert P.dms_probe_read_bytes(10 * 4096 * 16 + 5, 4, 4) == 10 * 4096 * 16
    assert P.dms_probe_mfma_bf16_flops(2, 3) == 2 * 4 * 8 * 3 * 16 * 16 * 32 * 2


def base(**kw):
    c = dict(max_batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, hidden=256, window=16, block_size=8,
             max_tokens_per_seq=100, pool_pages=32, max_chunk=64)
    c.update(kw)
    return dms.make_config(**c)


def test_valid_config_and_sizes():
    cfg = base()
    assert dms.dms_config_validate(cfg) == 0
    assert dms.dms_max_pages_per_seq(cfg) == 13
    n1 = dms.dms_cache_bytes(cfg)
    n2 = dms.dms_cache_bytes(base(pool_pages=64))
    # doubling the pool adds K+V pages (bf16) plus metadata
    assert n2 - n1 >= 32 * 8 * 64 * 2 * 2


@pytest.mark.parametrize("kw,msg", [
    (dict(block_size=0), "block_size"),
    (dict(window=8), "window must be greater"),
    (dict(window=7), "window must be greater"),
    (dict(num_q_heads=6, num_kv_heads=4), "multiple"),
    (dict(num_q_heads=24, num_kv_heads=2), "group size"),
    (dict(head_dim=96), "head_dim"),
    (dict(hidden=130), "hidden"),
    (dict(max_chunk=10000), "max_chunk"),
    (dict(max_batch=0), "positive"),
    (dict(max_batch=300, num_kv_heads=8, num_q_heads=32), "2048"),
])
def test_invalid_configs_are_rejected(kw, msg):
    with pytest.raises(dms.DmsError) as ei:
        dms.dms_config_validate(base(**kw))
    assert ei.value.status == dms.DMS_ERR_CONFIG
    assert msg in str(ei.value)


def test_bad_enums_are_rejected():
    cfg = base()
    cfg.kv_dtype = 7
    with pytest.raises(dms.DmsError):
        dms.dms_config_validate(cfg)
    cfg = base()
    cfg.alpha_per = 2
    with pytest.raises(dms.DmsError):
        dms.dms_config_validate(cfg)


def test_null_arguments_fail_before_any_launch():
    L = dms.lib()
    assert L.dms_cache_bytes(None, None) == dms.DMS_ERR_ARG
    assert L.dms_decide(None, None, None, None, None, None, None, 1, 1, None, None, None) == dms.DMS_ERR_ARG
    assert L.dms_append_evict(None, None, None, None, None, 1, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_decode_attn(None, None, None, None, 1, None, 0, None) == dms.DMS_ERR_ARG
    assert L.dms_prefill_attn(None, None, None, None, None, None, None, 1, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_seq_reset(None, None, 1, None) == dms.DMS_ERR_ARG
    cfg = base()
    out = ctypes.c_void_p()
    assert L.dms_cache_create(ctypes.byref(cfg), None, 0, None, ctypes.byref(out)) == dms.DMS_ERR_ARG
    assert L.dms_cache_create(ctypes.byref(cfg), ctypes.c_void_p(256), 16, None, ctypes.byref(out)) == \
        dms.DMS_ERR_CAPACITY
    assert b"smaller" in L.dms_last_error()


def test_cache_holds_no_decode_scratch():
    """The Qwen3-8B decode layer (B 8, 8K prompt + 136 steps, block 256): the
    cache buffer is the K/V pages plus tables a few MB in size; the decode
    partial records live in the caller's workspace (dms_decode_workspace_bytes)."""
    P, D, B, Hkv = 256, 128, 8, 8
    max_tokens = 8192 + 136
    pool = B * Hkv * -(-max_tokens // P)
    cfg = dms.make_config(max_batch=B, num_q_heads=32, num_kv_heads=Hkv, head_dim=D, hidden=4096, window=512,
                          block_size=P, max_tokens_per_seq=max_tokens, pool_pages=pool, max_chunk=4096)
    pages = 2 * pool * P * D * 2
    slot_meta = pool * P * 4
    chunk_slot = B * Hkv * 4096 * 4
    overhead = dms.dms_cache_bytes(cfg) - pages
    assert slot_meta + chunk_slot <= overhead < slot_meta + chunk_slot + (1 << 20)


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(dms, "_lib", None)
    monkeypatch.setattr(dms, "_LIB_PATH", os.path.join(ROOT, "no_such_lib.so"))
    with pytest.raises(RuntimeError, match="not built"):
        dms.lib()


def test_training_scorer_and_accounting_arguments_fail_before_any_launch():
    """Argument checks of the training, KVzap and accounting entry points run
    on the host before any HIP call (placeholder addresses are never
    dereferenced: every call below fails a check or has nothing to do)."""
    L = dms.lib()
    vp = ctypes.c_void_p
    a16 = vp(4096)                      # 16-byte aligned placeholder
    a8 = vp(4096 + 8)                   # 8-byte aligned only
    f = ctypes.c_float(0.0)
    # training forward
    assert L.dms_train_attn_fwd(1, 8, 4, 2, 128, 4, f, None, a16, a16, a16, a16, a16, None) == dms.DMS_ERR_ARG
    assert L.dms_train_attn_fwd(1, 8, 4, 3, 128, 4, f, a16, a16, a16, a16, a16, a16, None) == dms.DMS_ERR_ARG
    assert L.dms_train_attn_fwd(1, 8, 4, 2, 96, 4, f, a16, a16, a16, a16, a16, a16, None) == dms.DMS_ERR_UNSUPPORTED
    assert L.dms_train_attn_fwd(1, 8, 4, 2, 128, 0, f, a16, a16, a16, a16, a16, a16, None) == dms.DMS_ERR_ARG
    assert L.dms_train_attn_fwd(1, 8, 4, 2, 128, 4, f, a8, a16, a16, a16, a16, a16, None) == dms.DMS_ERR_ARG
    # training backward and its workspace size
    n = ctypes.c_size_t()
    assert L.dms_train_attn_bwd_workspace_bytes(2, 10, 4, ctypes.byref(n)) == dms.DMS_OK and n.value == 2 * 2 * 10 * 4 * 4
    assert L.dms_train_attn_bwd_workspace_bytes(2, 10, 0, ctypes.byref(n)) == dms.DMS_ERR_ARG
    t11 = [a16] * 11                    # q k v out dout y lse dq dk dv dgate
    ws = (a16, ctypes.c_size_t(1 << 20))
    assert L.dms_train_attn_bwd(-1, 8, 4, 2, 128, 4, f, *t11, *ws, None) == dms.DMS_ERR_ARG
    assert L.dms_train_attn_bwd(1, 8, 4, 3, 128, 4, f, *t11, *ws, None) == dms.DMS_ERR_ARG
    assert L.dms_train_attn_bwd(1, 8, 4, 2, 96, 4, f, *t11, *ws, None) == dms.DMS_ERR_UNSUPPORTED
    assert L.dms_train_attn_bwd(0, 8, 4, 2, 128, 4, f, *([None] * 11), None, ctypes.c_size_t(0), None) == dms.DMS_OK
    assert L.dms_train_attn_bwd(1, 8, 4, 2, 128, 4, f, *t11[:5], None, *t11[6:], *ws, None) == dms.DMS_ERR_ARG
    assert L.dms_train_attn_bwd(1, 8, 4, 2, 128, 4, f, *t11, a16, ctypes.c_size_t(8 * 4 * 4 - 1), None) == \
        dms.DMS_ERR_CAPACITY
    assert L.dms_train_attn_bwd(1, 8, 4, 2, 128, 4, f, a8, *t11[1:], *ws, None) == dms.DMS_ERR_UNSUPPORTED
    # KVzap scorers
    assert L.dms_kvzap_workspace_bytes(1, 8, 0, 512, ctypes.byref(n)) == dms.DMS_ERR_ARG
    thr = ctypes.c_float(-4.0)
    kz = lambda B, T, H, Hkv, Hm, dt, h, W1, W2, th, ev, wsb: L.dms_kvzap_score(  # noqa: E731
        B, T, H, Hkv, Hm, dt, h, W1, None, W2, None, th, None, ev, a16, ctypes.c_size_t(wsb), None)
    assert kz(0, 8, 4096, 8, 512, dms.DMS_BF16, None, None, None, thr, None, 0) == dms.DMS_OK
    assert kz(1, 8, 4096, 8, 512, dms.DMS_BF16, None, a16, a16, thr, a16, 1 << 20) == dms.DMS_ERR_ARG
    assert kz(1, 8, 4096, 8, 512, dms.DMS_FP8_E4M3, a16, a16, a16, thr, a16, 1 << 20) == dms.DMS_ERR_UNSUPPORTED
    assert kz(1, 8, 4096, 17, 512, dms.DMS_BF16, a16, a16, a16, thr, a16, 1 << 20) == dms.DMS_ERR_UNSUPPORTED
    assert kz(1, 8, 4016, 8, 512, dms.DMS_BF16, a16, a16, a16, thr, a16, 1 << 20) == dms.DMS_ERR_UNSUPPORTED
    assert kz(1, 8, 4096, 8, 500, dms.DMS_BF16, a16, a16, a16, thr, a16, 1 << 20) == dms.DMS_ERR_UNSUPPORTED
    assert kz(1, 8, 4096, 8, 512, dms.DMS_BF16, a8, a16, a16, thr, a16, 1 << 20) == dms.DMS_ERR_UNSUPPORTED
    assert kz(1, 8, 4096, 8, 512, dms.DMS_BF16, a16, a16, a16, ctypes.c_float(float("nan")), a16, 1 << 20) == \
        dms.DMS_ERR_ARG
    assert kz(1, 8, 4096, 8, 512, dms.DMS_BF16, a16, a16, None, thr, a16, 1 << 20) == dms.DMS_ERR_ARG
    assert kz(1, 8, 4096, 8, 512, dms.DMS_BF16, a16, a16, a16, thr, a16, 0) == dms.DMS_ERR_CAPACITY
    # serving accounting without a cache
    info = dms.dms_seq_info()
    assert L.dms_seq_info_get(None, None, 1, None, ctypes.byref(info)) == dms.DMS_ERR_ARG
    p, fr = ctypes.c_int64(), ctypes.c_int64()
    assert L.dms_pages_needed(None, None, a16, 1, None, ctypes.byref(p), ctypes.byref(fr)) == dms.DMS_ERR_ARG
