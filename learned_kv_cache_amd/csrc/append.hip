// dms_append_evict: delayed eviction into the per-head paged store.
//
// "基于 DMS 的 KV Cache 压缩实战" walkthrough, 推理模式: on append, if the token
// at the end of the sliding window (position t - w) was marked for eviction,
// the new token t overwrites its slot in place; otherwise t takes the next
// free slot of its head, and a page is opened from the pool whenever the head's
// length reaches a multiple of the block size.  (延迟驱逐: a marked token stays
// usable until it leaves the window.)  FastDMS post, subsystem table: the
// decode kernel evaluates keep/evict per head, manages the retention window
// and appends to compact storage; the prefill kernel streams the surviving K/V
// into compact storage.
//
// Page ids are handed out deterministically: pairs (batch row, KV head) in
// row-major order, tokens in order inside a pair, ranks from a wave ballot
// scan, pages popped from one free stack.  No racing atomics decide an id.
#include "dms_internal.h"
#include "decode_prep.h"

namespace dms {



// Stores one row of D activations as kv-dtype page bytes (fp8: with scale s).
template <typename ACT, int KV>
__device__ __forceinline__ void store_row(uint8_t* dst_pages, int64_t dst_row, const ACT* src, int D, int lane,
                                          float inv_scale) {
  for (int e = lane; e < D; e += 64) {
    const float x = load_act<ACT>(src, e);
    if (KV == DMS_F32) {
      reinterpret_cast<float*>(dst_pages)[dst_row * D + e] = x;
    } else if (KV == DMS_BF16) {
      reinterpret_cast<uint16_t*>(dst_pages)[dst_row * D + e] = f32_to_bf16(x);
    } else {
      dst_pages[dst_row * D + e] = f32_to_e4m3(x * inv_scale);
    }
  }
}

template <typename ACT>
__device__ __forceinline__ float row_amax(const ACT* src, int D, int lane) {
  float m = 0.0f;
  for (int e = lane; e < D; e += 64) m = fmaxf(m, fabsf(load_act<ACT>(src, e)));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

// ---------------------------------------------------------------------------
// Decode append (T = 1): one workgroup of 512 threads; pairs (row, KV head)
// in rounds of up to 512.
//
// Latency, not bandwidth, sets the cost of this step, so the loads the slot
// decision waits on are issued first (position, length, the page of the
// head's last slot, the flag), then the ring entry of position t - w (it
// carries the slot and its flat page row, so an in-place overwrite needs no
// page-table lookup), then the K/V rows as 16-byte pieces.  Only a head that
// opens a page reads the free stack.  Cross-lane reductions use DPP.

constexpr int kAppThreads = 512;
constexpr int kAppPieces = 4;       // prefetched 16-byte pieces of K (and V) per thread

template <typename ACT, int KV>
__global__ __launch_bounds__(kAppThreads) void append_decode_kernel(AppendArgs a) {
  constexpr int NW = kAppThreads / 64;
  __shared__ int s_wave[NW];
  __shared__ int s_dst[kAppThreads];
  __shared__ int s_page[kAppThreads];
  __shared__ uint8_t s_new[kAppThreads];
  __shared__ int s_free, s_used;
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int npairs = a.B * g.Hkv;
  const int in_row_bytes = g.D * static_cast<int>(sizeof(ACT));
  const int ppr = in_row_bytes / 16;                       // 16-byte pieces per row
  if (blockIdx.x == 0 && tid == 0) plan_invalidate(d);
  const int page_row_bytes = g.D * (KV == DMS_F32 ? 4 : (KV == DMS_BF16 ? 2 : 1));
  if (tid == 0) {
    s_free = d.ctl[kCtlFreeCount];
    s_used = 0;
  }
  for (int p0 = 0; p0 < npairs; p0 += kAppThreads) {
    const int nround = min(kAppThreads, npairs - p0);
    // 1. what the slot decision waits on
    const int p = p0 + tid;
    int seq = -1, t = 0, len = 0, cur = -1, e = 0, unit = 0;
    if (p < npairs) {
      const int row = p / g.Hkv;
      seq = a.seq_ids ? a.seq_ids[row] : row;
      if (seq >= 0 && seq < g.Bmax) {
        unit = seq * g.Hkv + p % g.Hkv;
        t = d.pos[seq];
        len = d.lengths[unit];
        cur = d.cur_page[unit];
      }
      if (seq >= 0 && seq < g.Bmax) {
        e = a.evict[p] ? 1 : 0;
      }
    }
    // 2. K/V pieces of this round (used after the decision)
    const int npieces = nround * ppr;
    uint4 kpc[kAppPieces], vpc[kAppPieces];
#pragma unroll
    for (int i = 0; i < kAppPieces; ++i) {
      const int pc = tid + i * kAppThreads;
      if (pc < npieces) {
        const uint8_t* src = static_cast<const uint8_t*>(a.k) + static_cast<size_t>(p0) * in_row_bytes;
        kpc[i] = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(pc) * 16);
        vpc[i] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.v) +
                                                 static_cast<size_t>(p0) * in_row_bytes + static_cast<size_t>(pc) * 16);
      } else {
        kpc[i] = make_uint4(0, 0, 0, 0);
        vpc[i] = make_uint4(0, 0, 0, 0);
      }
    }
    // 3. the slot
    bool valid = false, need = false, overwrite = false;
    int slot = 0, page = -1, dst = -1;
    if (p < npairs) {
      if (seq < 0 || seq >= g.Bmax) {
        set_status(d.ctl, DMS_DEV_BAD_SEQ);
      } else if (t + 1 > g.max_tokens) {
        set_status(d.ctl, DMS_DEV_CAPACITY);
      } else {
        if (t >= g.w) {
          const int64_t ri = static_cast<int64_t>(unit) * g.w + t % g.w;
          const int rv = d.ring[ri];
          if (rv < 0) {
            overwrite = true;
            slot = rv & 0x7FFFFFFF;
            dst = d.ring_row[ri];
            page = dst / g.P;
          }
        }
        if (!overwrite) {
          slot = len;
          need = (slot % g.P) == 0;
          page = need ? -1 : cur;
        }
        valid = true;
      }
    }
    int wtot;
    const int wr = wave_rank(need, &wtot);
    if (lane == 0) s_wave[wave] = wtot;
    __syncthreads();
    int off = 0, round_total = 0;
    for (int i = 0; i < NW; ++i) {
      if (i < wave) off += s_wave[i];
      round_total += s_wave[i];
    }
    if (valid && need) {
      const int R = s_used + off + wr;
      if (R < s_free) {
        page = d.free_stack[s_free - 1 - R];
        d.page_table[static_cast<int64_t>(unit) * g.maxp + slot / g.P] = page;
        d.cur_page[unit] = page;
      } else {
        set_status(d.ctl, DMS_DEV_POOL_EXHAUSTED);
        valid = false;
      }
    }
    if (valid) {
      if (!overwrite) dst = page * g.P + slot % g.P;
      if (!overwrite) d.lengths[unit] = slot + 1;
      d.ring[static_cast<int64_t>(unit) * g.w + t % g.w] = slot | (e << 31);
      d.ring_row[static_cast<int64_t>(unit) * g.w + t % g.w] = dst;
      d.slot_meta[dst] = t | (e << 31);
    }
    if (tid < nround) {
      s_dst[tid] = valid ? dst : -1;
      s_page[tid] = page;
      s_new[tid] = (valid && need) ? 1 : 0;
    }
    __syncthreads();
    // 4. copy: piece pc belongs to pair pc / ppr (pieces of a row are adjacent lanes)
    for (int i = 0; i * kAppThreads < npieces; ++i) {
      const int pc = tid + i * kAppThreads;
      const bool have = pc < npieces;
      uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
      if (have) {
        if (i < kAppPieces) {
          kx = kpc[i < kAppPieces ? i : 0];
          vx = vpc[i < kAppPieces ? i : 0];
        } else {
          kx = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.k) + static_cast<size_t>(p0) * in_row_bytes +
                                               static_cast<size_t>(pc) * 16);
          vx = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.v) + static_cast<size_t>(p0) * in_row_bytes +
                                               static_cast<size_t>(pc) * 16);
        }
      }
      const int pr = have ? pc / ppr : 0;
      const int piece = have ? pc % ppr : 0;
      const int dsti = have ? s_dst[pr] : -1;
      float inv_k = 1.0f, inv_v = 1.0f;
      if (KV == DMS_FP8_E4M3) {
        // row amax over the row's ppr lanes (one DPP row or part of it)
        const float mk = piece_row_max(piece_amax(kx, sizeof(ACT) == 2), ppr);
        const float mv = piece_row_max(piece_amax(vx, sizeof(ACT) == 2), ppr);
        if (dsti >= 0) {
          const int pg = s_page[pr];
          float sk, sv;
          if (s_new[pr]) {
            sk = page_scale_from_amax(mk);
            sv = page_scale_from_amax(mv);
            if (piece == 0) {
              d.scales[2 * pg] = sk;
              d.scales[2 * pg + 1] = sv;
            }
          } else {
            sk = d.scales[2 * pg];
            sv = d.scales[2 * pg + 1];
          }
          inv_k = 1.0f / sk;
          inv_v = 1.0f / sv;
        }
      }
      if (dsti >= 0) {
        store_piece<ACT, KV>(d.k_pages, dsti, page_row_bytes, piece, kx, inv_k);
        store_piece<ACT, KV>(d.v_pages, dsti, page_row_bytes, piece, vx, inv_v);
      }
    }
    __syncthreads();
    if (tid == 0) s_used += round_total;
    __syncthreads();
  }
  // positions advance after every pair has read them
  for (int row = tid; row < a.B; row += kAppThreads) {
    const int seq = a.seq_ids ? a.seq_ids[row] : row;
    if (seq >= 0 && seq < g.Bmax && d.pos[seq] + 1 <= g.max_tokens) d.pos[seq] += 1;
  }
  if (tid == 0) d.ctl[kCtlFreeCount] = s_free - min(s_used, s_free);
}


// ---------------------------------------------------------------------------
// dms_decode_prepare, linear decision with bf16 activations: decision and
// append of one decode token per sequence in one launch, one workgroup per
// (batch row, KV head) pair (prep_pair); the last workgroup to arrive opens
// pages and advances positions (prep_commit).

template <int KV>
__global__ __launch_bounds__(kPrepThreads) void decode_prepare_kernel(AppendArgs a, PrepIn in) {
  __shared__ PrepShared sh;
  const int npairs = a.B * a.g.Hkv;
  if (blockIdx.x == 0 && threadIdx.x == 0) plan_invalidate(a.d);
  prep_pair<KV>(a, in, blockIdx.x, false, sh);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) sh.last = prep_arrive(a.d, blockIdx.x, npairs);
  __syncthreads();
  if (!sh.last) return;
  prep_commit<KV>(a, in, npairs, sh);
  prep_arrive_reset(a.d, npairs, threadIdx.x);
}

// ---------------------------------------------------------------------------
// Chunk append (T > 1), three steps.
//
// plan  (one workgroup per pair): allocation flags, new slot ids by a scan,
//       overwrite chains resolved back to an allocating token or the ring.
// alloc (one workgroup): page ranks over pairs, pops, lengths, positions.
// write (pairs x token blocks): each slot's final occupant, slot metadata and
//       the ring entries of the chunk's last w positions.
//
// chunk_info[pair] = {valid, s0, L0, n_alloc, old_pages, new_pages, 0, 0}

__global__ __launch_bounds__(1024) void chunk_plan_kernel(AppendArgs a) {
  extern __shared__ int s_slot[];   // [T]
  __shared__ int s_wave[16];
  __shared__ int s_base;
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int pair = blockIdx.x;
  const int row = pair / g.Hkv, kh = pair % g.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (pair == 0 && tid == 0) plan_invalidate(d);
  int32_t* info = d.chunk_info + static_cast<int64_t>(pair) * 8;
  const int seq = a.seq_ids ? a.seq_ids[row] : row;
  if (seq < 0 || seq >= g.Bmax) {
    if (tid == 0) {
      set_status(d.ctl, DMS_DEV_BAD_SEQ);
      info[0] = 0;
    }
    return;
  }
  const int s0 = d.pos[seq];
  if (s0 + a.T > g.max_tokens) {
    if (tid == 0) {
      set_status(d.ctl, DMS_DEV_CAPACITY);
      info[0] = 0;
    }
    return;
  }
  const int unit = seq * g.Hkv + kh;
  const int L0 = d.lengths[unit];
  const int32_t* ring = d.ring + static_cast<int64_t>(unit) * g.w;
  const uint8_t* ev = a.evict + static_cast<int64_t>(pair) * a.T;
  if (tid == 0) s_base = 0;
  __syncthreads();
  // 1. allocation flags and new slot ids (exclusive scan)
  for (int t0 = 0; t0 < a.T; t0 += 1024) {
    const int tt = t0 + tid;
    bool alloc = false;
    if (tt < a.T) {
      const int t = s0 + tt;
      bool prev_evicted = false;
      if (t >= g.w) prev_evicted = (tt >= g.w) ? (ev[tt - g.w] != 0) : (ring[(t - g.w) % g.w] < 0);
      alloc = !prev_evicted;
    }
    int wtot;
    const int wr = wave_rank(alloc, &wtot);
    if (lane == 0) s_wave[wave] = wtot;
    __syncthreads();
    int off = 0, tot = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < wave) off += s_wave[i];
      tot += s_wave[i];
    }
    if (tt < a.T) s_slot[tt] = alloc ? L0 + s_base + off + wr : -1;
    __syncthreads();
    if (tid == 0) s_base += tot;
    __syncthreads();
  }
  // 2. overwrite chains: slot(t) = slot(t - w) back to an allocating token
  for (int t0 = 0; t0 < a.T; t0 += 1024) {
    const int tt = t0 + tid;
    int res = 0;
    if (tt < a.T) {
      res = s_slot[tt];
      if (res < 0) {
        int u = tt - g.w;
        while (u >= 0 && s_slot[u] < 0) u -= g.w;
        res = (u >= 0) ? s_slot[u] : (ring[(s0 + u) % g.w] & 0x7FFFFFFF);
      }
    }
    __syncthreads();
    if (tt < a.T) d.chunk_slot[static_cast<int64_t>(pair) * g.max_chunk + tt] = res;
  }
  if (tid == 0) {
    const int n = s_base;
    info[0] = 1;
    info[1] = s0;
    info[2] = L0;
    info[3] = n;
    info[4] = (L0 + g.P - 1) / g.P;
    info[5] = (L0 + n + g.P - 1) / g.P - (L0 + g.P - 1) / g.P;
  }
}

__global__ __launch_bounds__(1024) void chunk_alloc_kernel(AppendArgs a) {
  __shared__ int s_wave[16];
  __shared__ int s_free, s_used;
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int npairs = a.B * g.Hkv;
  if (tid == 0) {
    s_free = d.ctl[kCtlFreeCount];
    s_used = 0;
  }
  __syncthreads();
  for (int p0 = 0; p0 < npairs; p0 += 1024) {
    const int p = p0 + tid;
    int32_t* info = d.chunk_info + static_cast<int64_t>(p) * 8;
    const bool valid = p < npairs && info[0] != 0;
    const int need = valid ? info[5] : 0;
    int x = need;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < wave) off += s_wave[i];
      tot += s_wave[i];
    }
    if (valid) {
      const int row = p / g.Hkv, kh = p % g.Hkv;
      const int seq = a.seq_ids ? a.seq_ids[row] : row;
      const int unit = seq * g.Hkv + kh;
      const int R0 = s_used + off + x - need;
      int32_t* pt = d.page_table + static_cast<int64_t>(unit) * g.maxp;
      if (R0 + need <= s_free) {
        for (int j = 0; j < need; ++j) {
          const int page = d.free_stack[s_free - 1 - (R0 + j)];
          pt[info[4] + j] = page;
          d.page_amax[2 * page] = 0u;
          d.page_amax[2 * page + 1] = 0u;
        }
        d.lengths[unit] = info[2] + info[3];
        const int Lnew = info[2] + info[3];
        if (Lnew > 0) d.cur_page[unit] = need > 0 ? d.free_stack[s_free - 1 - (R0 + need - 1)] : pt[(Lnew - 1) / g.P];
        if (kh == 0) d.pos[seq] = info[1] + a.T;
      } else {
        set_status(d.ctl, DMS_DEV_POOL_EXHAUSTED);
        info[0] = 0;
        if (kh == 0) d.pos[seq] = info[1] + a.T;
      }
    }
    __syncthreads();
    if (tid == 0) s_used += tot;
    __syncthreads();
  }
  if (tid == 0) d.ctl[kCtlFreeCount] = s_free - min(s_used, s_free);
}

constexpr int kTokPerWG = 16;   // tokens per workgroup of the write/amax kernels (one wave per token)

// fp8 only: largest magnitude written into each freshly opened page.  The
// workgroup's tokens (consecutive, so mostly in one page) are folded per page
// in LDS first: one atomic per (workgroup, page) instead of one per token
// (a page's 256 tokens queued on the same two words otherwise).
template <typename ACT>
__global__ __launch_bounds__(kTokPerWG * 64) void chunk_amax_kernel(AppendArgs a) {
  __shared__ int s_page[kTokPerWG];
  __shared__ float s_mk[kTokPerWG], s_mv[kTokPerWG];
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int pair = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tt = blockIdx.x * kTokPerWG + wave;
  const int32_t* info = d.chunk_info + static_cast<int64_t>(pair) * 8;
  int page = -1;
  float mk = 0.0f, mv = 0.0f;
  // (waves with no freshly written row keep page -1 and still meet the barrier)
  if (tt < a.T && info[0]) {
    const uint8_t* ev = a.evict + static_cast<int64_t>(pair) * a.T;
    const int slot = d.chunk_slot[static_cast<int64_t>(pair) * g.max_chunk + tt];
    // skipped: rows overwritten later in this chunk, and pages opened by an earlier call
    if (!(ev[tt] && tt + g.w < a.T) && slot / g.P >= info[4]) {
      const int row = pair / g.Hkv, kh = pair % g.Hkv;
      const int seq = a.seq_ids ? a.seq_ids[row] : row;
      page = d.page_table[(static_cast<int64_t>(seq) * g.Hkv + kh) * g.maxp + slot / g.P];
      const size_t src = ((static_cast<size_t>(row) * a.T + tt) * g.Hkv + kh) * g.D;
      mk = row_amax<ACT>(static_cast<const ACT*>(a.k) + src, g.D, lane);
      mv = row_amax<ACT>(static_cast<const ACT*>(a.v) + src, g.D, lane);
    }
  }
  if (lane == 0) {
    s_page[wave] = page;
    s_mk[wave] = mk;
    s_mv[wave] = mv;
  }
  __syncthreads();
  if (threadIdx.x < kTokPerWG) {
    const int i = threadIdx.x, pg = s_page[i];
    bool first = pg >= 0;
    for (int j = 0; j < i; ++j) first = first && s_page[j] != pg;
    if (first) {
      float k2 = 0.0f, v2 = 0.0f;
      for (int j = i; j < kTokPerWG; ++j) {
        if (s_page[j] == pg) {
          k2 = fmaxf(k2, s_mk[j]);
          v2 = fmaxf(v2, s_mv[j]);
        }
      }
      atomicMax(d.page_amax + 2 * pg, __float_as_uint(k2));
      atomicMax(d.page_amax + 2 * pg + 1, __float_as_uint(v2));
    }
  }
}

template <typename ACT, int KV>
__global__ __launch_bounds__(kTokPerWG * 64) void chunk_write_kernel(AppendArgs a) {
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int pair = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int tt = blockIdx.x * kTokPerWG + (threadIdx.x >> 6);
  if (tt >= a.T) return;
  const int32_t* info = d.chunk_info + static_cast<int64_t>(pair) * 8;
  if (!info[0]) return;
  const int row = pair / g.Hkv, kh = pair % g.Hkv;
  const int seq = a.seq_ids ? a.seq_ids[row] : row;
  const int unit = seq * g.Hkv + kh;
  const uint8_t* ev = a.evict + static_cast<int64_t>(pair) * a.T;
  const int e = ev[tt] ? 1 : 0;
  const int slot = d.chunk_slot[static_cast<int64_t>(pair) * g.max_chunk + tt];
  const int t = info[1] + tt;
  const int page = d.page_table[static_cast<int64_t>(unit) * g.maxp + slot / g.P];
  const int64_t dst = static_cast<int64_t>(page) * g.P + slot % g.P;
  if (lane == 0 && tt >= a.T - g.w) {
    d.ring[static_cast<int64_t>(unit) * g.w + t % g.w] = slot | (e << 31);
    d.ring_row[static_cast<int64_t>(unit) * g.w + t % g.w] = static_cast<int32_t>(dst);
  }
  if (e && tt + g.w < a.T) return;                  // not the final occupant of its slot
  if (lane == 0) d.slot_meta[dst] = t | (e << 31);
  const size_t src = ((static_cast<size_t>(row) * a.T + tt) * g.Hkv + kh) * g.D;
  float inv_k = 1.0f, inv_v = 1.0f;
  if (KV == DMS_FP8_E4M3) {
    float sk, sv;
    if (slot / g.P >= info[4]) {
      sk = page_scale_from_amax(__uint_as_float(d.page_amax[2 * page]));
      sv = page_scale_from_amax(__uint_as_float(d.page_amax[2 * page + 1]));
      if (lane == 0) {
        d.scales[2 * page] = sk;
        d.scales[2 * page + 1] = sv;
      }
    } else {
      sk = d.scales[2 * page];
      sv = d.scales[2 * page + 1];
    }
    inv_k = 1.0f / sk;
    inv_v = 1.0f / sv;
  }
  store_row<ACT, KV>(d.k_pages, dst, static_cast<const ACT*>(a.k) + src, g.D, lane, inv_k);
  store_row<ACT, KV>(d.v_pages, dst, static_cast<const ACT*>(a.v) + src, g.D, lane, inv_v);
}

template <typename ACT, int KV>
static void launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.T == 1) {
    hipLaunchKernelGGL((append_decode_kernel<ACT, KV>), dim3(1), dim3(kAppThreads), 0, st, a);
    return;
  }
  const int npairs = a.B * a.g.Hkv;
  hipLaunchKernelGGL(chunk_plan_kernel, dim3(npairs), dim3(1024), a.T * sizeof(int), st, a);
  hipLaunchKernelGGL(chunk_alloc_kernel, dim3(1), dim3(1024), 0, st, a);
  const dim3 grid((a.T + kTokPerWG - 1) / kTokPerWG, npairs), block(kTokPerWG * 64);
  if (KV == DMS_FP8_E4M3) hipLaunchKernelGGL((chunk_amax_kernel<ACT>), grid, block, 0, st, a);
  hipLaunchKernelGGL((chunk_write_kernel<ACT, KV>), grid, block, 0, st, a);
}

}  // namespace dms

using namespace dms;

extern "C" int dms_append_evict(dms_cache* cache, const int32_t* seq_ids, const void* k, const void* v,
                                const uint8_t* evict, int B, int T, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  if (!k || !v || !evict) return fail(DMS_ERR_ARG, "k, v and evict are required");
  const Geo& g = cache->geo;
  if (B <= 0 || T <= 0) return fail(DMS_ERR_ARG, "B and T must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  if (T > g.max_chunk) return fail(DMS_ERR_CAPACITY, "T above max_chunk");
  AppendArgs a{};
  a.d = cache->dev;
  a.g = g;
  a.seq_ids = seq_ids;
  a.k = k;
  a.v = v;
  a.evict = evict;
  a.B = B;
  a.T = T;
  hipStream_t st = as_stream(stream);
  switch (g.kv_dtype) {
    case DMS_F32: launch_append<float, DMS_F32>(a, st); break;
    case DMS_BF16: launch_append<uint16_t, DMS_BF16>(a, st); break;
    case DMS_FP8_E4M3: launch_append<uint16_t, DMS_FP8_E4M3>(a, st); break;
    default: return fail(DMS_ERR_UNSUPPORTED, "kv dtype");
  }
  return check_hip(hipGetLastError(), "dms_append_evict launch");
}

extern "C" int dms_decode_prepare(dms_cache* cache, const int32_t* seq_ids, const void* hidden,
                                  const float* rms_gamma, const float* W, const float* bias, const float* offsets,
                                  void* q_inout, const void* k, const void* v, int B, float* logits_out,
                                  uint8_t* evict_out, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  const dms_config& c = cache->cfg;
  const Geo& g = cache->geo;
  if (!k || !v || !offsets || !evict_out) return fail(DMS_ERR_ARG, "k, v, offsets and evict_out are required");
  if (B <= 0) return fail(DMS_ERR_ARG, "B must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  hipStream_t st = as_stream(stream);
  const bool bf16_act = g.kv_dtype == DMS_BF16 || g.kv_dtype == DMS_FP8_E4M3;
  const bool linear = c.decide_mode == DMS_DECIDE_LINEAR;
  if (bf16_act) {
    if (linear) {
      if (!hidden || !rms_gamma || !W) return fail(DMS_ERR_ARG, "hidden, rms_gamma and W are required");
      if ((reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(rms_gamma) |
           reinterpret_cast<uintptr_t>(W)) % 16 != 0)
        return fail(DMS_ERR_ARG, "hidden, rms_gamma and W must be 16-byte aligned");
      if (c.hidden % 8 != 0) return fail(DMS_ERR_UNSUPPORTED, "hidden must be a multiple of 8");
    } else if (!q_inout) {
      return fail(DMS_ERR_ARG, "q_inout is required");
    }
    if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) % 16 != 0)
      return fail(DMS_ERR_ARG, "k and v must be 16-byte aligned");
    AppendArgs a{};
    a.d = cache->dev;
    a.g = g;
    a.seq_ids = seq_ids;
    a.k = k;
    a.v = v;
    a.evict = nullptr;
    a.B = B;
    a.T = 1;
    a.bias = bias;
    a.offsets = offsets;
    a.alpha = c.alpha_scale;
    a.eps = c.rms_eps;
    a.per_layer = c.alpha_per == DMS_ALPHA_PER_LAYER;
    a.disable = c.disable_eviction != 0;
    a.logits_out = logits_out;
    a.evict_out = evict_out;
    PrepIn in{static_cast<const uint16_t*>(hidden), rms_gamma, W, static_cast<uint16_t*>(q_inout), linear ? 0 : 1};
    if (g.kv_dtype == DMS_BF16)
      hipLaunchKernelGGL((decode_prepare_kernel<DMS_BF16>), dim3(B * g.Hkv), dim3(kPrepThreads), 0, st, a, in);
    else
      hipLaunchKernelGGL((decode_prepare_kernel<DMS_FP8_E4M3>), dim3(B * g.Hkv), dim3(kPrepThreads), 0, st, a, in);
    return check_hip(hipGetLastError(), "dms_decode_prepare launch");
  }
  // f32 activations: decide, then append
  int s = dms_decide(cache, hidden, rms_gamma, W, bias, offsets, q_inout, B, 1, logits_out, evict_out, stream);
  if (s) return s;
  return dms_append_evict(cache, seq_ids, k, v, evict_out, B, 1, stream);
}
