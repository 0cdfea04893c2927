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

namespace dms {

struct AppendArgs {
  DevCache d;
  Geo g;
  const int32_t* seq_ids;
  const void* k;
  const void* v;
  const uint8_t* evict;
  int B;
  int T;
};

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
// Decode append (T = 1): one workgroup of 1024 threads; pairs (row, KV head)
// in rounds of up to 1024.  One thread per pair decides the slot; CPP threads
// per pair copy its K and V rows, whose input values are loaded at the start
// of the round so the copy does not wait on the slot decision's loads.  The
// dependent loads are: position -> ring entry -> page (free stack or table).
template <typename ACT, int KV>
__device__ __forceinline__ void copy_part(uint8_t* pages, int64_t dst_row, int D, int e0, int ne, const float* x,
                                          float inv_scale) {
  for (int i = 0; i < ne; ++i) {
    const int e = e0 + i;
    if (KV == DMS_F32) reinterpret_cast<float*>(pages)[dst_row * D + e] = x[i];
    else if (KV == DMS_BF16) reinterpret_cast<uint16_t*>(pages)[dst_row * D + e] = f32_to_bf16(x[i]);
    else pages[dst_row * D + e] = f32_to_e4m3(x[i] * inv_scale);
  }
}

template <typename ACT, int KV>
__global__ __launch_bounds__(1024) void append_decode_kernel(AppendArgs a) {
  constexpr int MAXE = 16;                  // elements per thread in the copy (D <= 128, CPP >= 8)
  __shared__ int s_wave[16];
  __shared__ int s_dst[1024];               // destination row (page * P + offset), -1: nothing to write
  __shared__ int s_page[1024];
  __shared__ uint8_t s_new[1024];
  __shared__ int s_free, s_used;
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int npairs = a.B * g.Hkv;
  if (tid == 0) {
    s_free = d.ctl[kCtlFreeCount];
    s_used = 0;
  }
  for (int p0 = 0; p0 < npairs; p0 += 1024) {
    const int nround = min(1024, npairs - p0);
    // copy geometry of this round: CPP threads per pair, ne elements each
    int cpp = 1024 / nround;
    cpp = cpp >= 64 ? 64 : (cpp >= 32 ? 32 : (cpp >= 16 ? 16 : (cpp >= 8 ? 8 : (cpp >= 4 ? 4 : (cpp >= 2 ? 2 : 1)))));
    while (cpp > 1 && (g.D % cpp != 0 || g.D / cpp < 2)) cpp >>= 1;
    const int ne_max = g.D / cpp;
    const int cpair = tid / cpp, cpart = tid % cpp;
    const bool copier = cpair < nround && ne_max <= MAXE;
    float kx[MAXE], vx[MAXE];
    if (copier) {
      const size_t src = static_cast<size_t>(p0 + cpair) * g.D + cpart * ne_max;   // [B][1][Hkv][D]
      const ACT* ks = static_cast<const ACT*>(a.k) + src;
      const ACT* vs = static_cast<const ACT*>(a.v) + src;
#pragma unroll
      for (int i = 0; i < MAXE; ++i) {
        kx[i] = i < ne_max ? load_act<ACT>(ks, i) : 0.0f;
        vx[i] = i < ne_max ? load_act<ACT>(vs, i) : 0.0f;
      }
    }
    const int p = p0 + tid;
    bool valid = false, need = false, overwrite = false;
    int kh = 0, t = 0, slot = 0, e = 0, unit = 0;
    if (p < npairs) {
      const int row = p / g.Hkv;
      kh = p % g.Hkv;
      const int seq = a.seq_ids ? a.seq_ids[row] : row;
      if (seq < 0 || seq >= g.Bmax) {
        set_status(d.ctl, DMS_DEV_BAD_SEQ);
      } else {
        unit = seq * g.Hkv + kh;
        t = d.pos[seq];
        const int len = d.lengths[unit];
        e = a.evict[p] ? 1 : 0;
        if (t + 1 > g.max_tokens) {
          set_status(d.ctl, DMS_DEV_CAPACITY);
        } else {
          const int rv = (t >= g.w) ? d.ring[static_cast<int64_t>(unit) * g.w + t % g.w] : 0;
          if (t >= g.w && rv < 0) {
            overwrite = true;
            slot = rv & 0x7FFFFFFF;
          } else {
            slot = len;
            need = (slot % g.P) == 0;
          }
          valid = true;
        }
      }
    }
    int wtot;
    const int wr = wave_rank(need, &wtot);
    if (lane == 0) s_wave[wave] = wtot;
    __syncthreads();
    int off = 0, round_total = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < wave) off += s_wave[i];
      round_total += s_wave[i];
    }
    int page = -1;
    if (valid) {
      int32_t* pt = d.page_table + static_cast<int64_t>(unit) * g.maxp;
      if (need) {
        const int R = s_used + off + wr;
        if (R < s_free) {
          page = d.free_stack[s_free - 1 - R];
          pt[slot / g.P] = page;
        } else {
          set_status(d.ctl, DMS_DEV_POOL_EXHAUSTED);
          valid = false;
        }
      } else {
        page = pt[slot / g.P];
      }
    }
    if (valid) {
      if (!overwrite) d.lengths[unit] = slot + 1;
      d.ring[static_cast<int64_t>(unit) * g.w + t % g.w] = slot | (e << 31);
      d.slot_meta[static_cast<int64_t>(page) * g.P + slot % g.P] = t | (e << 31);
    }
    if (tid < nround) {
      s_dst[tid] = valid ? page * g.P + slot % g.P : -1;
      s_page[tid] = page;
      s_new[tid] = (valid && need) ? 1 : 0;
    }
    __syncthreads();
    if (cpair < nround) {
      const int dst = s_dst[cpair];
      const size_t src = static_cast<size_t>(p0 + cpair) * g.D + cpart * ne_max;
      const ACT* ks = static_cast<const ACT*>(a.k) + src;
      const ACT* vs = static_cast<const ACT*>(a.v) + src;
      float inv_k = 1.0f, inv_v = 1.0f;
      if (KV == DMS_FP8_E4M3) {
        // amax over the row's cpp threads (contiguous lanes of one wave)
        float mk = 0.0f, mv = 0.0f;
        for (int i = 0; i < ne_max; ++i) {
          mk = fmaxf(mk, fabsf(copier ? kx[i < MAXE ? i : 0] : load_act<ACT>(ks, i)));
          mv = fmaxf(mv, fabsf(copier ? vx[i < MAXE ? i : 0] : load_act<ACT>(vs, i)));
        }
        for (int o = 1; o < cpp; o <<= 1) {
          mk = fmaxf(mk, __shfl_xor(mk, o));
          mv = fmaxf(mv, __shfl_xor(mv, o));
        }
        if (dst >= 0) {
          const int pg = s_page[cpair];
          float sk, sv;
          if (s_new[cpair]) {
            sk = page_scale_from_amax(mk);
            sv = page_scale_from_amax(mv);
            if (cpart == 0) {
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
      if (dst >= 0) {
        if (copier) {
          copy_part<ACT, KV>(d.k_pages, dst, g.D, cpart * ne_max, ne_max, kx, inv_k);
          copy_part<ACT, KV>(d.v_pages, dst, g.D, cpart * ne_max, ne_max, vx, inv_v);
        } else {
          // rows split over few threads: copy in pieces of MAXE elements
          for (int i0 = 0; i0 < ne_max; i0 += MAXE) {
            const int n = min(MAXE, ne_max - i0);
            float tk[MAXE], tv[MAXE];
            for (int i = 0; i < n; ++i) {
              tk[i] = load_act<ACT>(ks, i0 + i);
              tv[i] = load_act<ACT>(vs, i0 + i);
            }
            copy_part<ACT, KV>(d.k_pages, dst, g.D, cpart * ne_max + i0, n, tk, inv_k);
            copy_part<ACT, KV>(d.v_pages, dst, g.D, cpart * ne_max + i0, n, tv, inv_v);
          }
        }
      }
    }
    __syncthreads();
    if (tid == 0) s_used += round_total;
    __syncthreads();
  }
  // positions advance after every pair has read them
  for (int row = tid; row < a.B; row += 1024) {
    const int seq = a.seq_ids ? a.seq_ids[row] : row;
    if (seq >= 0 && seq < g.Bmax && d.pos[seq] + 1 <= g.max_tokens) d.pos[seq] += 1;
  }
  if (tid == 0) d.ctl[kCtlFreeCount] = s_free - min(s_used, s_free);
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

// fp8 only: largest magnitude written into each freshly opened page.
template <typename ACT>
__global__ __launch_bounds__(kTokPerWG * 64) void chunk_amax_kernel(AppendArgs a) {
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int pair = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int tt = blockIdx.x * kTokPerWG + (threadIdx.x >> 6);
  if (tt >= a.T) return;
  const int32_t* info = d.chunk_info + static_cast<int64_t>(pair) * 8;
  if (!info[0]) return;
  const uint8_t* ev = a.evict + static_cast<int64_t>(pair) * a.T;
  if (ev[tt] && tt + g.w < a.T) return;            // overwritten later in this chunk
  const int slot = d.chunk_slot[static_cast<int64_t>(pair) * g.max_chunk + tt];
  if (slot / g.P < info[4]) return;                 // page opened by an earlier call
  const int row = pair / g.Hkv, kh = pair % g.Hkv;
  const int seq = a.seq_ids ? a.seq_ids[row] : row;
  const int page = d.page_table[(static_cast<int64_t>(seq) * g.Hkv + kh) * g.maxp + slot / g.P];
  const size_t src = ((static_cast<size_t>(row) * a.T + tt) * g.Hkv + kh) * g.D;
  const float mk = row_amax<ACT>(static_cast<const ACT*>(a.k) + src, g.D, lane);
  const float mv = row_amax<ACT>(static_cast<const ACT*>(a.v) + src, g.D, lane);
  if (lane == 0) {
    atomicMax(d.page_amax + 2 * page, __float_as_uint(mk));
    atomicMax(d.page_amax + 2 * page + 1, __float_as_uint(mv));
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
  if (lane == 0 && tt >= a.T - g.w) d.ring[static_cast<int64_t>(unit) * g.w + t % g.w] = slot | (e << 31);
  if (e && tt + g.w < a.T) return;                  // not the final occupant of its slot
  const int page = d.page_table[static_cast<int64_t>(unit) * g.maxp + slot / g.P];
  const int64_t dst = static_cast<int64_t>(page) * g.P + slot % g.P;
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
    hipLaunchKernelGGL((append_decode_kernel<ACT, KV>), dim3(1), dim3(1024), 0, st, a);
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
  AppendArgs a{cache->dev, g, seq_ids, k, v, evict, B, T};
  hipStream_t st = as_stream(stream);
  switch (g.kv_dtype) {
    case DMS_F32: launch_append<float, DMS_F32>(a, st); break;
    case DMS_BF16: launch_append<uint16_t, DMS_BF16>(a, st); break;
    case DMS_FP8_E4M3: launch_append<uint16_t, DMS_FP8_E4M3>(a, st); break;
    default: return fail(DMS_ERR_UNSUPPORTED, "kv dtype");
  }
  return check_hip(hipGetLastError(), "dms_append_evict launch");
}
