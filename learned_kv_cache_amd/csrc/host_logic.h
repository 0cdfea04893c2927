// Host-side logic of the DMS C ABI that needs no GPU: configuration checks,
// the layout of the single cache buffer, and the statistics and serving
// accounting computed from host copies of the cache tables.  Plain C++17 (no
// HIP), so that it can also be built and checked on its own, under the
// address and undefined-behaviour sanitizers.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <vector>

#include "dms.h"

namespace dms {

constexpr int kMaxUnits = 2048;        // B * Hkv of one decode/append call
constexpr int kMaxStepLayers = 512;    // layers of one dms_step_layers binding
constexpr int kMaxChunk = 8192;        // largest T of one append / prefill call
constexpr int kMaxDecodeGrid = 2048;   // workgroups of the decode attention kernel
constexpr int kCtlWords = 64;
// Arrival counters of the fused decode step's attention workgroups: workgroup
// i adds one to group i % kArriveGroups (an atomic whose result it does not
// wait for); the committing workgroup polls the groups.  One counter per
// 256-byte line, so the adds of different groups do not queue behind each
// other.
constexpr int kArriveGroups = 32;
constexpr int kArriveStride = 64;      // int32 words between counters
// The prepare workgroups' arrival counters share those lines, 128 bytes on:
// prepare workgroup p adds to group p % 32 and the last of a group adds to
// the control word kCtlPrepArrive, so no counter takes more than a group's
// returning atomics (one counter for all 512 pairs of a 64-row step
// serialised them).
constexpr int kPrepArriveWord = 32;
// Decode plan of the fused step (written by one step's commit for the next):
// a header, the sequence id of each batch row, and one record per attention
// workgroup; used only for launches of at most kPlanMaxWgs workgroups.
constexpr int kPlanHeader = 64;        // int32 words
constexpr int kPlanMaxWgs = 1024;
constexpr int kPlanRec = 16;           // int32 words per workgroup record

// Byte offsets of the regions carved out of one cache buffer.
struct Layout {
  size_t k_pages, v_pages, scales, page_amax, slot_meta, page_table, lengths, ring, ring_row, cur_page, pos,
      free_stack, ctl, chunk_slot, chunk_info, unit_info, arrive, plan, decide_w, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

inline int kv_elem_bytes(int kv_dtype) {
  switch (kv_dtype) {
    case DMS_F32: return 4;
    case DMS_BF16: return 2;
    case DMS_FP8_E4M3: return 1;
    default: return 0;
  }
}

// nullptr when the configuration is valid; otherwise the reason, with the
// status code in *status (walkthrough, Qwen3ConfigDMS hard constraints:
// block_size > 0 and window > block_size; the rest are this library's limits).
inline const char* config_error(const dms_config* c, int* status) {
  *status = DMS_ERR_CONFIG;
  if (!c) {
    *status = DMS_ERR_ARG;
    return "config is NULL";
  }
  if (c->max_batch <= 0 || c->num_q_heads <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0 || c->hidden <= 0 ||
      c->max_tokens_per_seq <= 0 || c->pool_pages <= 0 || c->max_chunk <= 0)
    return "sizes must be positive";
  if (c->block_size <= 0) return "block_size must be > 0";
  if (c->window <= c->block_size) return "window must be greater than block_size";
  if (c->num_q_heads % c->num_kv_heads != 0) return "num_q_heads must be a multiple of num_kv_heads";
  const int g = c->num_q_heads / c->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return "group size must be 1, 2, 4 or 8";
  if (c->num_kv_heads > 16) return "num_kv_heads must be <= 16";
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return "head_dim must be 32, 64 or 128";
  if (c->hidden % 4 != 0) return "hidden must be a multiple of 4";
  if (kv_elem_bytes(c->kv_dtype) == 0) return "bad kv_dtype";
  if (c->decide_mode != DMS_DECIDE_LINEAR && c->decide_mode != DMS_DECIDE_QNEURON) return "bad decide_mode";
  if (c->alpha_per != DMS_ALPHA_PER_HEAD && c->alpha_per != DMS_ALPHA_PER_LAYER) return "alpha_per must be head or layer";
  if (c->max_chunk > kMaxChunk) return "max_chunk above 8192";
  if (static_cast<int64_t>(c->max_batch) * c->num_kv_heads > kMaxUnits) return "max_batch * num_kv_heads above 2048";
  if (!(c->alpha_scale == c->alpha_scale) || !(c->rms_eps >= 0.0f) || !(c->softmax_scale >= 0.0f))
    return "alpha_scale, rms_eps and softmax_scale must be finite, eps and scale >= 0";
  if (static_cast<int64_t>(c->pool_pages) * c->block_size >= (1ll << 31))
    return "pool_pages * block_size must stay below 2^31";
  if (c->max_tokens_per_seq >= (1 << 30)) return "max_tokens_per_seq too large";
  *status = DMS_OK;
  return nullptr;
}

// int32 words of the decode plan region: header, rows (rounded up to 64), records.
inline size_t plan_words(int Bmax) {
  return static_cast<size_t>(kPlanHeader) + ((static_cast<size_t>(Bmax) + 63) & ~static_cast<size_t>(63)) +
         static_cast<size_t>(kPlanMaxWgs) * kPlanRec;
}

// The linear adapter's gamma * W of a prefill chunk decision as the matrix
// cores read it: per 8 hidden elements, 16 columns (8 heads, two bf16 parts
// each) of 8 bf16.
inline size_t decide_w_bytes(int hidden) { return (static_cast<size_t>(hidden) + 7) / 8 * 16 * 16; }

// The regions of one cache buffer, each 256-byte aligned, in this order (the
// configuration must be valid).
inline void compute_layout(const dms_config& c, Layout* L) {
  const size_t elem = static_cast<size_t>(kv_elem_bytes(c.kv_dtype));
  const size_t pool = static_cast<size_t>(c.pool_pages);
  const size_t P = static_cast<size_t>(c.block_size);
  const size_t D = static_cast<size_t>(c.head_dim);
  const size_t units = static_cast<size_t>(c.max_batch) * c.num_kv_heads;
  const size_t maxp = (static_cast<size_t>(c.max_tokens_per_seq) + P - 1) / P;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L->k_pages = take(pool * P * D * elem);
  L->v_pages = take(pool * P * D * elem);
  L->scales = take(pool * 2 * sizeof(float));
  L->page_amax = take(pool * 2 * sizeof(uint32_t));
  L->slot_meta = take(pool * P * sizeof(int32_t));
  L->page_table = take(units * maxp * sizeof(int32_t));
  L->lengths = take(units * sizeof(int32_t));
  L->ring = take(units * static_cast<size_t>(c.window) * sizeof(int32_t));
  L->ring_row = take(units * static_cast<size_t>(c.window) * sizeof(int32_t));
  L->cur_page = take(units * sizeof(int32_t));
  L->pos = take(static_cast<size_t>(c.max_batch) * sizeof(int32_t));
  L->free_stack = take(pool * sizeof(int32_t));
  L->ctl = take(kCtlWords * sizeof(int32_t));
  L->chunk_slot = take(units * static_cast<size_t>(c.max_chunk) * sizeof(int32_t));
  L->chunk_info = take(units * 8 * sizeof(int32_t));
  L->unit_info = take(static_cast<size_t>(kMaxUnits) * 4 * sizeof(int32_t));
  L->arrive = take(static_cast<size_t>(kArriveGroups) * kArriveStride * sizeof(int32_t));
  L->plan = take(plan_words(c.max_batch) * sizeof(int32_t));
  L->decide_w = take(decide_w_bytes(c.hidden));
  L->total = off;
}

// Occupancy from the per-head lengths [Bmax][Hkv] and positions [Bmax]
// (walkthrough, 损失函数与压缩比调度: realised compression, here tokens / live
// slots).
inline void stats_from_tables(int Bmax, int Hkv, int P, int64_t row_bytes, const int32_t* len, const int32_t* pos,
                              dms_stats* out) {
  int64_t tokens = 0, live = 0, pages = 0;
  for (int b = 0; b < Bmax; ++b) tokens += static_cast<int64_t>(pos[b]) * Hkv;
  for (int64_t i = 0; i < static_cast<int64_t>(Bmax) * Hkv; ++i) {
    live += len[i];
    pages += (len[i] + P - 1) / P;
  }
  out->tokens = tokens;
  out->live_slots = live;
  out->pages_in_use = pages;
  out->bytes_live = live * row_bytes * 2;
  out->bytes_allocated = pages * P * row_bytes * 2;
  out->cache_cr = live ? static_cast<double>(tokens) / static_cast<double>(live) : 0.0;
}

// Footprint of sequence seq (FastDMS post, subsystem table: memory accounting
// by surviving tokens).
inline dms_seq_info seq_info_from_tables(int seq, int Hkv, int P, const int32_t* len, const int32_t* pos) {
  dms_seq_info r{};
  r.position = pos[seq];
  for (int k = 0; k < Hkv; ++k) {
    const int32_t L = len[static_cast<size_t>(seq) * Hkv + k];
    r.live_slots += L;
    if (L > r.max_head_slots) r.max_head_slots = L;
    r.pages += (L + P - 1) / P;
  }
  return r;
}

// The most pool pages that appending n more tokens to sequence seq can take
// (FastDMS post, subsystem table: admission by compact capacity): every new
// token kept, except that the first w of them overwrite in place the slots of
// already-marked tokens in the window (walkthrough, 推理模式); -1 past
// max_tokens.  len [Bmax][Hkv], pos [Bmax], ring [Bmax][Hkv][w] (slot |
// evict << 31 of position p at p % w).
inline int64_t worst_pages_for_seq(int seq, int64_t n, int Hkv, int w, int P, int max_tokens, const int32_t* len,
                                   const int32_t* pos, const int32_t* ring) {
  const int64_t t0 = pos[seq];
  if (t0 + n > max_tokens) return -1;
  int64_t pages = 0;
  for (int k = 0; k < Hkv; ++k) {
    const size_t u = static_cast<size_t>(seq) * Hkv + k;
    int64_t overwrites = 0;
    const int64_t first = n < w ? n : w;
    for (int64_t j = 0; j < first; ++j) {
      const int64_t p = t0 + j - w;
      if (p >= 0 && ring[u * w + static_cast<size_t>(p % w)] < 0) ++overwrites;
    }
    const int64_t L = len[u], slots = L + (n - overwrites);
    pages += (slots + P - 1) / P - (L + P - 1) / P;
  }
  return pages;
}

// ---- structural invariants of the cache tables ----------------------------
// (walkthrough, 推理模式: the delayed-eviction slot rule; the shared pool).  A
// bit per kind of violation; 0 means consistent.
constexpr uint32_t kChkLength = 1u << 0;      // L outside [min(pos, w), pos]
constexpr uint32_t kChkPageId = 1u << 1;      // a held page id outside [0, pool)
constexpr uint32_t kChkOwnership = 1u << 2;   // a page held twice, held and free, or pages lost
constexpr uint32_t kChkSlot = 1u << 3;        // a live slot whose occupant is not one visible token
constexpr uint32_t kChkRing = 1u << 4;        // a window entry that does not name its token's slot
constexpr uint32_t kChkCurPage = 1u << 5;     // the current page is not the page of slot L - 1
constexpr uint32_t kChkFreeStack = 1u << 6;   // free count or a free id out of range

struct TableView {
  int Bmax, Hkv, w, P, maxp, pool;
  const int32_t* lengths;     // [Bmax][Hkv]
  const int32_t* page_table;  // [Bmax][Hkv][maxp]
  const int32_t* slot_meta;   // [pool][P] position | evict << 31
  const int32_t* ring;        // [Bmax][Hkv][w] slot | evict << 31 of position p at p % w
  const int32_t* ring_row;    // [Bmax][Hkv][w] page * P + slot % P of that slot
  const int32_t* cur_page;    // [Bmax][Hkv]
  const int32_t* pos;         // [Bmax]
  const int32_t* free_stack;  // [pool]
  int32_t free_count;
};

// Checks every sequence's heads: live slots 0..L-1 each hold one distinct
// token visible to the sequence's last query (kept, or inside the window),
// the window entries of the last w positions name the slots holding them,
// the page ids are the pool's, each page has one owner or is free, and no
// page is lost.  *first_unit gets the first (sequence * Hkv + head) with a
// slot, ring or page violation, else -1.
inline uint32_t check_tables(const TableView& t, int* first_unit) {
  uint32_t bad = 0;
  *first_unit = -1;
  auto flag = [&](uint32_t bit, int unit) {
    bad |= bit;
    if (*first_unit < 0 && unit >= 0) *first_unit = unit;
  };
  if (t.free_count < 0 || t.free_count > t.pool) {
    flag(kChkFreeStack, -1);
    return bad;
  }
  std::vector<int> owner(static_cast<size_t>(t.pool), -1);
  int64_t held = 0;
  for (int i = 0; i < t.free_count; ++i) {
    const int pg = t.free_stack[i];
    if (pg < 0 || pg >= t.pool) {
      flag(kChkFreeStack, -1);
      continue;
    }
    if (owner[pg] != -1) flag(kChkOwnership, -1);
    owner[pg] = -2;
  }
  std::vector<int32_t> seen;
  for (int seq = 0; seq < t.Bmax; ++seq) {
    const int32_t T = t.pos[seq];
    for (int k = 0; k < t.Hkv; ++k) {
      const int unit = seq * t.Hkv + k;
      const int32_t L = t.lengths[unit];
      if (L < 0 || L > T || L < std::min(T, t.w)) {
        flag(kChkLength, unit);
        continue;
      }
      const int np = static_cast<int>((static_cast<int64_t>(L) + t.P - 1) / t.P);
      if (np > t.maxp) {
        flag(kChkLength, unit);
        continue;
      }
      const int32_t* pt = t.page_table + static_cast<size_t>(unit) * t.maxp;
      bool ids_ok = true;
      for (int i = 0; i < np; ++i) {
        const int pg = pt[i];
        if (pg < 0 || pg >= t.pool) {
          flag(kChkPageId, unit);
          ids_ok = false;
          continue;
        }
        if (owner[pg] != -1) flag(kChkOwnership, unit);
        owner[pg] = unit;
        ++held;
      }
      if (!ids_ok) continue;
      if (L > 0 && t.cur_page[unit] != pt[(L - 1) / t.P]) flag(kChkCurPage, unit);
      // live slots: distinct tokens, each visible to the query at T - 1
      seen.assign(static_cast<size_t>(T > 0 ? T : 1), 0);
      for (int32_t s = 0; s < L; ++s) {
        const uint32_t meta = static_cast<uint32_t>(t.slot_meta[static_cast<size_t>(pt[s / t.P]) * t.P + s % t.P]);
        const int32_t p = static_cast<int32_t>(meta & 0x7FFFFFFFu);
        const bool marked = (meta >> 31) != 0;
        if (p >= T || seen[p] || (marked && (T - 1) - p >= t.w)) {
          flag(kChkSlot, unit);
          break;
        }
        seen[p] = 1;
      }
      // the window: position p at p % w names the slot holding p
      for (int32_t p = std::max(0, T - t.w); p < T; ++p) {
        const size_t ri = static_cast<size_t>(unit) * t.w + static_cast<size_t>(p % t.w);
        const uint32_t e = static_cast<uint32_t>(t.ring[ri]);
        const int32_t s = static_cast<int32_t>(e & 0x7FFFFFFFu);
        if (s >= L) {
          flag(kChkRing, unit);
          break;
        }
        const int32_t row = pt[s / t.P] * t.P + s % t.P;
        const uint32_t meta = static_cast<uint32_t>(t.slot_meta[static_cast<size_t>(row)]);
        if (static_cast<int32_t>(meta & 0x7FFFFFFFu) != p || (meta >> 31) != (e >> 31) ||
            (t.ring_row && t.ring_row[ri] != row)) {
          flag(kChkRing, unit);
          break;
        }
      }
    }
  }
  if (held + t.free_count != t.pool) flag(kChkOwnership, -1);
  return bad;
}

}  // namespace dms
