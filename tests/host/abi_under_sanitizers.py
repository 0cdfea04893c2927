"""Host-side paths of the C ABI, run against the sanitizer build of libdms
(tests/test_host_sanitizers.py starts it with the address-sanitizer runtime
preloaded): configuration checks, buffer and workspace sizes, and every entry
point's argument checks, none of which launches anything.  Placeholder
addresses are never dereferenced."""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from learned_kv_cache_amd import dms  # noqa: E402

dms._LIB_PATH = sys.argv[1]
L = dms.lib()
vp = ctypes.c_void_p
f = ctypes.c_float(0.0)
a16 = vp(4096)


def cfg(**kw):
    c = dict(max_batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, hidden=256, window=16, block_size=8,
             max_tokens_per_seq=100, pool_pages=32, max_chunk=64)
    c.update(kw)
    return dms.make_config(**c)


ok = 0
assert dms.dms_config_validate(cfg()) == 0
for kw in (dict(block_size=0), dict(window=8), dict(num_q_heads=6, num_kv_heads=4), dict(head_dim=96),
           dict(hidden=130), dict(max_chunk=10000), dict(max_batch=0), dict(pool_pages=1 << 28)):
    assert L.dms_config_validate(ctypes.byref(cfg(**kw))) == dms.DMS_ERR_CONFIG, kw
    assert len(L.dms_last_error()) > 0
for D in (32, 64, 128):
    for kv in ("f32", "bf16", "fp8"):
        c = cfg(head_dim=D, kv_dtype=kv, pool_pages=1000, max_tokens_per_seq=33333)
        n = ctypes.c_size_t()
        assert L.dms_cache_bytes(ctypes.byref(c), ctypes.byref(n)) == 0 and n.value > 0
        p = ctypes.c_int32()
        assert L.dms_max_pages_per_seq(ctypes.byref(c), ctypes.byref(p)) == 0 and p.value == -(-33333 // 8)
n = ctypes.c_size_t()
assert L.dms_decode_workspace_bytes(ctypes.byref(cfg()), 0, ctypes.byref(n)) == dms.DMS_ERR_ARG
assert L.dms_decode_workspace_bytes(ctypes.byref(cfg()), 3, ctypes.byref(n)) == dms.DMS_ERR_ARG
assert L.dms_kvzap_workspace_bytes(2, 10, 8, 64, ctypes.byref(n)) == 0 and n.value == 2 * 10 * 8 * 4
assert L.dms_train_attn_bwd_workspace_bytes(2, 10, 4, ctypes.byref(n)) == 0
# argument checks of every cache entry point (no cache: refused before anything else)
assert L.dms_cache_bytes(None, None) == dms.DMS_ERR_ARG
assert L.dms_decide(None, None, None, None, None, None, None, 1, 1, None, None, None) == dms.DMS_ERR_ARG
assert L.dms_append_evict(None, None, None, None, None, 1, 1, None) == dms.DMS_ERR_ARG
assert L.dms_decode_attn(None, None, None, None, 1, None, 0, None) == dms.DMS_ERR_ARG
assert L.dms_decode_attn_noalloc(None, None, None, None, 1, None) == dms.DMS_ERR_ARG
assert L.dms_decode_prepare(None, *([None] * 9), 1, None, None, None) == dms.DMS_ERR_ARG
assert L.dms_decode_step(None, *([None] * 10), 1, None, None, None, 0, None) == dms.DMS_ERR_ARG
assert L.dms_prefill_attn(None, None, None, None, None, None, None, 1, 1, None) == dms.DMS_ERR_ARG
assert L.dms_seq_reset(None, None, 1, None) == dms.DMS_ERR_ARG
assert L.dms_cache_status(None, None, None) == dms.DMS_ERR_ARG
assert L.dms_cache_clear_status(None, None) == dms.DMS_ERR_ARG
assert L.dms_cache_dump(None, None, None) == dms.DMS_ERR_ARG
assert L.dms_cache_stats(None, None, None) == dms.DMS_ERR_ARG
assert L.dms_cache_config(None, None) == dms.DMS_ERR_ARG
assert L.dms_cache_check(None, None, None, None) == dms.DMS_ERR_ARG
info = dms.dms_seq_info()
assert L.dms_seq_info_get(None, None, 1, None, ctypes.byref(info)) == dms.DMS_ERR_ARG
pg, fr = ctypes.c_int64(), ctypes.c_int64()
assert L.dms_pages_needed(None, None, a16, 1, None, ctypes.byref(pg), ctypes.byref(fr)) == dms.DMS_ERR_ARG
out = vp()
assert L.dms_cache_create(ctypes.byref(cfg()), None, 0, None, ctypes.byref(out)) == dms.DMS_ERR_ARG
assert L.dms_cache_create(ctypes.byref(cfg()), vp(256), 16, None, ctypes.byref(out)) == dms.DMS_ERR_CAPACITY
assert L.dms_cache_create(ctypes.byref(cfg(window=3)), vp(256), 1 << 30, None, ctypes.byref(out)) == \
    dms.DMS_ERR_CONFIG
# training and KVzap argument checks
assert L.dms_train_attn_fwd(1, 8, 4, 3, 128, 4, f, a16, a16, a16, a16, a16, a16, None) == dms.DMS_ERR_ARG
assert L.dms_train_attn_fwd(1, 8, 4, 2, 96, 4, f, a16, a16, a16, a16, a16, a16, None) == dms.DMS_ERR_UNSUPPORTED
t11 = [a16] * 11
assert L.dms_train_attn_bwd(-1, 8, 4, 2, 128, 4, f, *t11, a16, ctypes.c_size_t(1 << 20), None) == dms.DMS_ERR_ARG
assert L.dms_train_attn_bwd(1, 8, 4, 2, 128, 4, f, *t11, a16, ctypes.c_size_t(1), None) == dms.DMS_ERR_CAPACITY
assert L.dms_kvzap_score(1, 8, 4016, 8, 512, dms.DMS_BF16, a16, a16, None, a16, None, ctypes.c_float(-4.0), None,
                         a16, a16, ctypes.c_size_t(1 << 20), None) == dms.DMS_ERR_UNSUPPORTED
assert L.dms_train_gate(None, None, ctypes.c_float(0.1), ctypes.c_int64(4), None, None, None, None) != 0
assert L.dms_train_gate_bwd(None, None, ctypes.c_float(0.1), ctypes.c_int64(4), None, None, None, a16, None) == \
    dms.DMS_ERR_ARG
assert L.dms_train_gate_bwd(a16, None, ctypes.c_float(0.0), ctypes.c_int64(4), None, None, None, a16, None) == \
    dms.DMS_ERR_ARG
assert L.dms_train_gate_bwd(a16, None, ctypes.c_float(1.0), ctypes.c_int64(-1), None, None, None, a16, None) == \
    dms.DMS_ERR_ARG
assert L.dms_train_gate_bwd(a16, None, ctypes.c_float(1.0), ctypes.c_int64(0), None, None, None, a16, None) == 0
maps = open("/proc/self/maps").read()
assert "libdms_san.so" in maps and "/libdms.so" not in maps, "not the sanitizer build"
print("abi checks ok", flush=True)
