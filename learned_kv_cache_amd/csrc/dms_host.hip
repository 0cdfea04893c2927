// Host side of the DMS C ABI: configuration checks, the layout of the single
// cache buffer, creation/initialisation, reset, status, dump and stats.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "dms_internal.h"

namespace dms {

static thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return DMS_OK;
  return fail(DMS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

static int validate(const dms_config* c) {
  int status = DMS_OK;
  const char* why = config_error(c, &status);
  return why ? fail(status, why) : DMS_OK;
}

int decode_grid_for(const dms_cache* c) { return c->decode_grid; }

// The decode grid of a call over `units` (row, KV head) units: two
// workgroups per CU, or about one per CU (the CUs plus a quarter of the
// units) when the units are at most a quarter of the CUs.  Then every unit
// gets workgroups of its own, and fewer, longer ranges per workgroup
// measured faster (Qwen3-8B layer, B 8: 18.2-18.5 us per layer step at 272
// workgroups, 18.7-19.1 at 256, 20.1-20.4 at 512; Llama-3.2-1B, B 1: within
// 0.2 us), while 512 units (B 64) measured slower at one per CU.
// DMS_DECODE_WGS fixes the grid for every call.  Never above decode_grid,
// which sizes the workspace.
int decode_grid_call(const dms_cache* c, int units) {
  if (c->decode_grid_fixed || 4 * units > c->num_cus) return c->decode_grid;
  return std::min(c->decode_grid, c->num_cus + units / 4);
}

int decode_grid_default(int cus) {
  int grid = 2 * cus;
  if (const char* e = std::getenv("DMS_DECODE_WGS")) grid = std::atoi(e);
  return std::max(1, std::min(grid, kMaxDecodeGrid));
}

size_t decode_workspace_bytes(int grid, int units, int g, int D) {
  const size_t records = 2 * static_cast<size_t>(grid) + static_cast<size_t>(units);
  return align256(records * static_cast<size_t>(g) * (D + 2) * sizeof(float));
}

// Fills the control words, the free stack (pops return 0, 1, 2, ...), empty
// lengths/positions, unused page-table entries and zero decode counters.
__global__ void init_kernel(DevCache d, Geo g, int units) {
  const int64_t n = static_cast<int64_t>(blockDim.x) * gridDim.x;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (int64_t i = i0; i < g.pool; i += n) d.free_stack[i] = g.pool - 1 - static_cast<int32_t>(i);
  for (int64_t i = i0; i < static_cast<int64_t>(units) * g.maxp; i += n) d.page_table[i] = -1;
  for (int64_t i = i0; i < units; i += n) {
    d.lengths[i] = 0;
    d.cur_page[i] = -1;
  }
  for (int64_t i = i0; i < g.Bmax; i += n) d.pos[i] = 0;
  for (int64_t i = i0; i < kCtlWords; i += n) d.ctl[i] = (i == kCtlFreeCount) ? g.pool : 0;
  for (int64_t i = i0; i < static_cast<int64_t>(kMaxUnits) * 4; i += n) d.unit_info[i] = 0;
  for (int64_t i = i0; i < static_cast<int64_t>(kArriveGroups) * kArriveStride; i += n) d.arrive[i] = 0;
  if (i0 == 0) plan_invalidate(d);
  for (int64_t i = i0; i < static_cast<int64_t>(g.pool) * 2; i += n) {
    d.scales[i] = 1.0f;
    d.page_amax[i] = 0u;
  }
}

// Returns the listed sequences' pages to the pool.  Pairs (sequence, head) are
// visited in reverse list order; each pair pushes its pages in reverse page
// order, so later pops return them in their original order.
__global__ __launch_bounds__(1024) void reset_kernel(DevCache d, Geo g, const int32_t* seq_ids, int n) {
  __shared__ int s_wave[16];
  __shared__ int s_base;
  __shared__ int s_free;
  const int tid = threadIdx.x;
  const int npairs = n * g.Hkv;
  if (tid == 0) {
    plan_invalidate(d);
    s_free = d.ctl[kCtlFreeCount];
    s_base = 0;
  }
  __syncthreads();
  for (int r0 = 0; r0 < npairs; r0 += 1024) {
    // r indexes pairs in push order: r = 0 is the last pair of the list.
    const int r = r0 + tid;
    int seq = -1, kh = 0, npg = 0;
    if (r < npairs) {
      const int p = npairs - 1 - r;
      const int row = p / g.Hkv;
      kh = p % g.Hkv;
      seq = seq_ids ? seq_ids[row] : row;
      if (seq < 0 || seq >= g.Bmax) {
        set_status(d.ctl, DMS_DEV_BAD_SEQ);
        seq = -1;
      } else {
        const int L = d.lengths[seq * g.Hkv + kh];
        npg = (L + g.P - 1) / g.P;
      }
    }
    // exclusive scan of npg over the block
    int x = npg;
    const int lane = tid & 63, wave = tid >> 6;
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int wave_off = 0, round_total = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < wave) wave_off += s_wave[i];
      round_total += s_wave[i];
    }
    const int excl = s_base + wave_off + x - npg;
    if (seq >= 0) {
      const int32_t* pt = d.page_table + (static_cast<int64_t>(seq) * g.Hkv + kh) * g.maxp;
      for (int j = 0; j < npg; ++j) {
        const int dst = s_free + excl + j;
        if (dst < g.pool) d.free_stack[dst] = pt[npg - 1 - j];
      }
    }
    __syncthreads();
    if (tid == 0) s_base += round_total;
    __syncthreads();
  }
  // clear the pairs after every push has read its page table
  for (int r = tid; r < npairs; r += 1024) {
    const int row = r / g.Hkv, kh = r % g.Hkv;
    const int seq = seq_ids ? seq_ids[row] : row;
    if (seq < 0 || seq >= g.Bmax) continue;
    int32_t* pt = d.page_table + (static_cast<int64_t>(seq) * g.Hkv + kh) * g.maxp;
    for (int j = 0; j < g.maxp; ++j) pt[j] = -1;
    d.lengths[seq * g.Hkv + kh] = 0;
    d.cur_page[seq * g.Hkv + kh] = -1;
    if (kh == 0) d.pos[seq] = 0;
  }
  if (tid == 0) d.ctl[kCtlFreeCount] = min(g.pool, s_free + s_base);
}

// Clears the status word and the one-launch decode step's arrival counters
// (left set when a step's commit gave up waiting; every workgroup of that
// launch has finished before this kernel runs).
__global__ void clear_status_kernel(int32_t* ctl, int32_t* arrive) {
  const int i = threadIdx.x;
  if (i == 0) {
    ctl[kCtlStatus] = 0;
    ctl[kCtlPrepArrive] = 0;
  }
  if (i < kArriveGroups) {
    arrive[i * kArriveStride] = 0;
    arrive[i * kArriveStride + kPrepArriveWord] = 0;
  }
}

}  // namespace dms

using namespace dms;

extern "C" {

const char* dms_last_error(void) { return g_last_error.c_str(); }

int dms_config_validate(const dms_config* cfg) {
  int s = validate(cfg);
  if (s == DMS_OK) g_last_error.clear();
  return s;
}

int dms_cache_bytes(const dms_config* cfg, size_t* bytes) {
  if (!bytes) return fail(DMS_ERR_ARG, "bytes is NULL");
  int s = validate(cfg);
  if (s) return s;
  Layout L;
  compute_layout(*cfg, &L);
  *bytes = L.total;
  return DMS_OK;
}

int dms_decode_workspace_bytes(const dms_config* cfg, int B, size_t* bytes) {
  if (!bytes) return fail(DMS_ERR_ARG, "bytes is NULL");
  int s = validate(cfg);
  if (s) return s;
  if (B <= 0 || B > cfg->max_batch) return fail(DMS_ERR_ARG, "B must be in [1, max_batch]");
  int dev = 0, cus = 256;
  if ((s = check_hip(hipGetDevice(&dev), "hipGetDevice"))) return s;
  if ((s = check_hip(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev),
                     "hipDeviceGetAttribute")))
    return s;
  *bytes = decode_workspace_bytes(decode_grid_default(cus), B * cfg->num_kv_heads,
                                  cfg->num_q_heads / cfg->num_kv_heads, cfg->head_dim);
  return DMS_OK;
}

int dms_max_pages_per_seq(const dms_config* cfg, int32_t* pages) {
  if (!pages) return fail(DMS_ERR_ARG, "pages is NULL");
  int s = validate(cfg);
  if (s) return s;
  *pages = (cfg->max_tokens_per_seq + cfg->block_size - 1) / cfg->block_size;
  return DMS_OK;
}

int dms_cache_create(const dms_config* cfg, void* dev_buf, size_t bytes, void* stream, dms_cache** out) {
  if (!out) return fail(DMS_ERR_ARG, "out is NULL");
  *out = nullptr;
  int s = validate(cfg);
  if (s) return s;
  if (!dev_buf) return fail(DMS_ERR_ARG, "device buffer is NULL");
  if (reinterpret_cast<uintptr_t>(dev_buf) % 256 != 0) return fail(DMS_ERR_ARG, "device buffer must be 256-byte aligned");
  Layout L;
  compute_layout(*cfg, &L);
  if (bytes < L.total)
    return fail(DMS_ERR_CAPACITY, "device buffer smaller than dms_cache_bytes (" + std::to_string(L.total) + ")");
  auto* c = new dms_cache();
  c->cfg = *cfg;
  c->layout = L;
  uint8_t* base = static_cast<uint8_t*>(dev_buf);
  c->dev.k_pages = base + L.k_pages;
  c->dev.v_pages = base + L.v_pages;
  c->dev.scales = reinterpret_cast<float*>(base + L.scales);
  c->dev.page_amax = reinterpret_cast<uint32_t*>(base + L.page_amax);
  c->dev.slot_meta = reinterpret_cast<int32_t*>(base + L.slot_meta);
  c->dev.page_table = reinterpret_cast<int32_t*>(base + L.page_table);
  c->dev.lengths = reinterpret_cast<int32_t*>(base + L.lengths);
  c->dev.ring = reinterpret_cast<int32_t*>(base + L.ring);
  c->dev.ring_row = reinterpret_cast<int32_t*>(base + L.ring_row);
  c->dev.cur_page = reinterpret_cast<int32_t*>(base + L.cur_page);
  c->dev.pos = reinterpret_cast<int32_t*>(base + L.pos);
  c->dev.free_stack = reinterpret_cast<int32_t*>(base + L.free_stack);
  c->dev.ctl = reinterpret_cast<int32_t*>(base + L.ctl);
  c->dev.chunk_slot = reinterpret_cast<int32_t*>(base + L.chunk_slot);
  c->dev.chunk_info = reinterpret_cast<int32_t*>(base + L.chunk_info);
  c->dev.unit_info = reinterpret_cast<int32_t*>(base + L.unit_info);
  c->dev.arrive = reinterpret_cast<int32_t*>(base + L.arrive);
  c->dev.plan = reinterpret_cast<int32_t*>(base + L.plan);
  c->dev.decide_w = reinterpret_cast<uint4*>(base + L.decide_w);
  Geo& g = c->geo;
  g.Bmax = cfg->max_batch;
  g.Hq = cfg->num_q_heads;
  g.Hkv = cfg->num_kv_heads;
  g.D = cfg->head_dim;
  g.g = cfg->num_q_heads / cfg->num_kv_heads;
  g.H = cfg->hidden;
  g.w = cfg->window;
  g.P = cfg->block_size;
  g.maxp = (cfg->max_tokens_per_seq + cfg->block_size - 1) / cfg->block_size;
  g.pool = cfg->pool_pages;
  g.max_tokens = cfg->max_tokens_per_seq;
  g.max_chunk = cfg->max_chunk;
  g.kv_dtype = cfg->kv_dtype;
  g.Pshift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == cfg->block_size) g.Pshift = sh;
  const float sc = cfg->softmax_scale > 0.0f ? cfg->softmax_scale : 1.0f / std::sqrt(static_cast<float>(cfg->head_dim));
  g.scale_log2 = sc * 1.4426950408889634f;
  int dev = 0;
  if ((s = check_hip(hipGetDevice(&dev), "hipGetDevice"))) { delete c; return s; }
  c->device = dev;
  int cus = 256;
  if ((s = check_hip(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev),
                     "hipDeviceGetAttribute"))) { delete c; return s; }
  c->num_cus = cus;
  c->decode_grid = decode_grid_default(cus);
  c->decode_grid_fixed = std::getenv("DMS_DECODE_WGS") != nullptr;
  c->decode_np = 0;
  if (const char* e = std::getenv("DMS_DECODE_NP")) c->decode_np = std::atoi(e);
  c->decode_lpr = 0;
  if (const char* e = std::getenv("DMS_DECODE_LPR")) c->decode_lpr = std::atoi(e);
  c->decode_mfma = 1;
  if (const char* e = std::getenv("DMS_DECODE_MFMA")) c->decode_mfma = std::atoi(e);
  const char* fg = std::getenv("DMS_GENERIC_KERNELS");
  c->force_generic = fg && fg[0] == '1';
  c->step_fuse = -1;
  if (const char* e = std::getenv("DMS_DECODE_STEP_FUSE")) c->step_fuse = std::atoi(e) ? 1 : 0;
  c->step_blocks_per_cu = -1;
  const int units = cfg->max_batch * cfg->num_kv_heads;
  hipLaunchKernelGGL(init_kernel, dim3(256), dim3(256), 0, as_stream(stream), c->dev, g, units);
  if ((s = check_hip(hipGetLastError(), "init_kernel launch"))) { delete c; return s; }
  *out = c;
  return DMS_OK;
}

int dms_cache_destroy(dms_cache* cache) {
  delete cache;
  return DMS_OK;
}

int dms_cache_config(const dms_cache* cache, dms_config* cfg) {
  if (!cache || !cfg) return fail(DMS_ERR_ARG, "NULL argument");
  *cfg = cache->cfg;
  return DMS_OK;
}

int dms_seq_reset(dms_cache* cache, const int32_t* seq_ids, int n, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  if (n < 0 || n > cache->geo.Bmax) return fail(DMS_ERR_ARG, "n must be in [0, max_batch]");
  if (n == 0) return DMS_OK;
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1024), 0, as_stream(stream), cache->dev, cache->geo, seq_ids, n);
  return check_hip(hipGetLastError(), "reset_kernel launch");
}

int dms_cache_status(dms_cache* cache, void* stream, int32_t* device_status) {
  if (!cache || !device_status) return fail(DMS_ERR_ARG, "NULL argument");
  int s = check_hip(hipMemcpyAsync(device_status, cache->dev.ctl + kCtlStatus, sizeof(int32_t),
                                   hipMemcpyDeviceToHost, as_stream(stream)), "hipMemcpyAsync");
  if (s) return s;
  return check_hip(hipStreamSynchronize(as_stream(stream)), "hipStreamSynchronize");
}

int dms_cache_clear_status(dms_cache* cache, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, as_stream(stream), cache->dev.ctl, cache->dev.arrive);
  return check_hip(hipGetLastError(), "clear_status_kernel launch");
}

int dms_cache_dump(dms_cache* cache, void* stream, const dms_dump* out) {
  if (!cache || !out) return fail(DMS_ERR_ARG, "NULL argument");
  const Geo& g = cache->geo;
  const int64_t units = static_cast<int64_t>(g.Bmax) * g.Hkv;
  const size_t elem = static_cast<size_t>(kv_elem_bytes(g.kv_dtype));
  hipStream_t st = as_stream(stream);
  struct Item { void* dst; const void* src; size_t bytes; };
  const Item items[] = {
      {out->lengths, cache->dev.lengths, units * sizeof(int32_t)},
      {out->page_table, cache->dev.page_table, units * g.maxp * sizeof(int32_t)},
      {out->slot_meta, cache->dev.slot_meta, static_cast<size_t>(g.pool) * g.P * sizeof(int32_t)},
      {out->ring, cache->dev.ring, units * g.w * sizeof(int32_t)},
      {out->positions, cache->dev.pos, static_cast<size_t>(g.Bmax) * sizeof(int32_t)},
      {out->free_stack, cache->dev.free_stack, static_cast<size_t>(g.pool) * sizeof(int32_t)},
      {out->free_count, cache->dev.ctl + kCtlFreeCount, sizeof(int32_t)},
      {out->k_pages, cache->dev.k_pages, static_cast<size_t>(g.pool) * g.P * g.D * elem},
      {out->v_pages, cache->dev.v_pages, static_cast<size_t>(g.pool) * g.P * g.D * elem},
      {out->page_scales, cache->dev.scales, static_cast<size_t>(g.pool) * 2 * sizeof(float)},
  };
  for (const Item& it : items) {
    if (!it.dst) continue;
    int s = check_hip(hipMemcpyAsync(it.dst, it.src, it.bytes, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
    if (s) return s;
  }
  return check_hip(hipStreamSynchronize(st), "hipStreamSynchronize");
}

int dms_cache_check(dms_cache* cache, void* stream, uint32_t* violations, int32_t* first_unit) {
  if (!cache || !violations) return fail(DMS_ERR_ARG, "NULL argument");
  const Geo& g = cache->geo;
  const size_t units = static_cast<size_t>(g.Bmax) * g.Hkv;
  std::vector<int32_t> len(units), pt(units * g.maxp), meta(static_cast<size_t>(g.pool) * g.P),
      ring(units * g.w), ring_row(units * g.w), cur(units), pos(g.Bmax), fs(g.pool);
  int32_t free_count = 0;
  dms_dump d;
  std::memset(&d, 0, sizeof(d));
  d.lengths = len.data();
  d.page_table = pt.data();
  d.slot_meta = meta.data();
  d.ring = ring.data();
  d.positions = pos.data();
  d.free_stack = fs.data();
  d.free_count = &free_count;
  hipStream_t st = as_stream(stream);
  int s = check_hip(hipMemcpyAsync(ring_row.data(), cache->dev.ring_row, ring_row.size() * sizeof(int32_t),
                                   hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
  if (!s) s = check_hip(hipMemcpyAsync(cur.data(), cache->dev.cur_page, cur.size() * sizeof(int32_t),
                                       hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
  if (!s) s = dms_cache_dump(cache, stream, &d);
  if (s) return s;
  const TableView t{g.Bmax, g.Hkv, g.w, g.P, g.maxp, g.pool, len.data(), pt.data(), meta.data(), ring.data(),
                    ring_row.data(), cur.data(), pos.data(), fs.data(), free_count};
  int where = -1;
  *violations = check_tables(t, &where);
  if (first_unit) *first_unit = where;
  return DMS_OK;
}

int dms_cache_stats(dms_cache* cache, void* stream, dms_stats* out) {
  if (!cache || !out) return fail(DMS_ERR_ARG, "NULL argument");
  const Geo& g = cache->geo;
  std::vector<int32_t> len(static_cast<size_t>(g.Bmax) * g.Hkv), pos(g.Bmax);
  dms_dump d;
  std::memset(&d, 0, sizeof(d));
  d.lengths = len.data();
  d.positions = pos.data();
  int s = dms_cache_dump(cache, stream, &d);
  if (s) return s;
  stats_from_tables(g.Bmax, g.Hkv, g.P, static_cast<int64_t>(g.D) * kv_elem_bytes(g.kv_dtype), len.data(),
                    pos.data(), out);
  return DMS_OK;
}

// ---------------------------------------------------------------------------
// Serving accounting (FastDMS post, subsystem table: admission by compact KV
// capacity, continuous-batching memory accounting by surviving tokens).

int dms_seq_info_get(dms_cache* cache, const int32_t* seq_ids, int n, void* stream, dms_seq_info* out) {
  if (!cache || !out || n < 0) return fail(DMS_ERR_ARG, "NULL argument or negative n");
  const Geo& g = cache->geo;
  std::vector<int32_t> len(static_cast<size_t>(g.Bmax) * g.Hkv), pos(g.Bmax);
  dms_dump d;
  std::memset(&d, 0, sizeof(d));
  d.lengths = len.data();
  d.positions = pos.data();
  int s = dms_cache_dump(cache, stream, &d);
  if (s) return s;
  for (int i = 0; i < n; ++i) {
    const int seq = seq_ids ? seq_ids[i] : i;
    if (seq < 0 || seq >= g.Bmax) return fail(DMS_ERR_ARG, "sequence id outside [0, max_batch)");
    out[i] = seq_info_from_tables(seq, g.Hkv, g.P, len.data(), pos.data());
  }
  return DMS_OK;
}

int dms_pages_needed(dms_cache* cache, const int32_t* seq_ids, const int32_t* n_new, int n, void* stream,
                     int64_t* pages_out, int64_t* free_pages) {
  if (!cache || !n_new || !pages_out || n < 0) return fail(DMS_ERR_ARG, "NULL argument or negative n");
  const Geo& g = cache->geo;
  const size_t units = static_cast<size_t>(g.Bmax) * g.Hkv;
  std::vector<int32_t> len(units), pos(g.Bmax), ring(units * g.w);
  int32_t freec = 0;
  dms_dump d;
  std::memset(&d, 0, sizeof(d));
  d.lengths = len.data();
  d.positions = pos.data();
  d.ring = ring.data();
  d.free_count = &freec;
  int s = dms_cache_dump(cache, stream, &d);
  if (s) return s;
  for (int i = 0; i < n; ++i) {
    const int seq = seq_ids ? seq_ids[i] : i;
    if (seq < 0 || seq >= g.Bmax) return fail(DMS_ERR_ARG, "sequence id outside [0, max_batch)");
    const int64_t m = n_new[i];
    if (m < 0) return fail(DMS_ERR_ARG, "negative token count");
    // beyond max_tokens_per_seq (-1): the append would be refused
    pages_out[i] = worst_pages_for_seq(seq, m, g.Hkv, g.w, g.P, g.max_tokens, len.data(), pos.data(), ring.data());
  }
  if (free_pages) *free_pages = freec;
  return DMS_OK;
}

}  // extern "C"
