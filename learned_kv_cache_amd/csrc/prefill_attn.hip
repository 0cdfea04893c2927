// dms_prefill_attn: attention of one prefill chunk under the DMS visibility
// rule, against the cache as it was before the chunk.
//
// "基于 DMS 的 KV Cache 压缩实战" walkthrough: 高级选项 Chunked Prefill (the prompt
// goes through the layers in fixed-size chunks) and the repository's exact
// prefill with the eviction mask.  Query at position i sees key j iff j <= i
// and (j is kept or i - j < w) (延迟驱逐).  Cached keys come from the pages
// (their position and flag from the slot metadata); chunk keys from the
// caller's K/V with the chunk's own flags.
//
// This file holds the vector-ALU kernel: one wave per (query token, KV head)
// serving all g query heads.  It covers every dtype and head size.
#include "dms_internal.h"

namespace dms {

struct PrefillArgs {
  DevCache d;
  Geo g;
  const int32_t* seq_ids;
  const void* q;        // [B][C][Hq][D]
  const void* k;        // [B][C][Hkv][D]
  const void* v;
  const uint8_t* evict; // [B][Hkv][C]
  void* out;            // [B][C][Hq][D]
  int B, C;
};

template <int KV>
__device__ __forceinline__ float load_page(const uint8_t* pages, int64_t idx) {
  if (KV == DMS_F32) return reinterpret_cast<const float*>(pages)[idx];
  if (KV == DMS_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(pages)[idx]);
  return e4m3_to_f32(pages[idx]);
}

// Lanes 16 per key row (D/16 elements each), 4 rows per pass.
template <typename ACT, int KV, int D, int G>
__global__ __launch_bounds__(64) void prefill_attn_generic_kernel(PrefillArgs a) {
  constexpr int LPR = 16, EPL = D / LPR, RPP = 4;
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int lane = threadIdx.x;
  const int lane_row = lane / LPR, lane_col = lane % LPR;
  const int i = blockIdx.x;                 // query index inside the chunk
  const int pair = blockIdx.y;
  const int row = pair / g.Hkv, kh = pair % g.Hkv;
  const int seq = a.seq_ids ? a.seq_ids[row] : row;
  if (seq < 0 || seq >= g.Bmax) {
    if (lane == 0 && i == 0 && kh == 0) set_status(d.ctl, DMS_DEV_BAD_SEQ);
    return;
  }
  const int unit = seq * g.Hkv + kh;
  const int s0 = d.pos[seq];
  const int L = d.lengths[unit];
  const int qi = s0 + i;
  const int32_t* pt = d.page_table + static_cast<int64_t>(unit) * g.maxp;
  const ACT* qp = static_cast<const ACT*>(a.q);
  const ACT* kp = static_cast<const ACT*>(a.k);
  const ACT* vp = static_cast<const ACT*>(a.v);
  const uint8_t* ev = a.evict + static_cast<int64_t>(pair) * a.C;

  float qf[G][EPL], o[G][EPL], m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      qf[h][e] = load_act<ACT>(qp, ((static_cast<size_t>(row) * a.C + i) * g.Hq + kh * G + h) * D +
                                       lane_col * EPL + e) * g.scale_log2;
      o[h][e] = 0.0f;
    }
  }
  const int total = L + i + 1;               // cache slots then chunk keys 0..i
  for (int base = 0; base < total; base += RPP) {
    const int r = base + lane_row;
    bool vis = false;
    float kf[EPL], vf[EPL];
    if (r < L) {
      const int page = pt[r / g.P];
      const int64_t roff = static_cast<int64_t>(page) * g.P + r % g.P;
      const int meta = d.slot_meta[roff];
      const int pj = meta & 0x7FFFFFFF;
      vis = meta >= 0 || qi - pj < g.w;
      const float sk = (KV == DMS_FP8_E4M3) ? d.scales[2 * page] : 1.0f;
      const float sv = (KV == DMS_FP8_E4M3) ? d.scales[2 * page + 1] : 1.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kf[e] = load_page<KV>(d.k_pages, roff * D + lane_col * EPL + e) * sk;
        vf[e] = load_page<KV>(d.v_pages, roff * D + lane_col * EPL + e) * sv;
      }
    } else if (r < total) {
      const int j = r - L;
      vis = ev[j] == 0 || i - j < g.w;
      const size_t src = ((static_cast<size_t>(row) * a.C + j) * g.Hkv + kh) * D + lane_col * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kf[e] = load_act<ACT>(kp, src + e);
        vf[e] = load_act<ACT>(vp, src + e);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) kf[e] = vf[e] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc = fmaf(qf[h][e], kf[e], acc);
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
      const float s = vis ? acc : -INFINITY;
      float mx = s;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m[h], mx);
      if (m_new == -INFINITY) continue;
      const float alpha = exp2f(m[h] - m_new);
      m[h] = m_new;
      const float pe = vis ? exp2f(s - m_new) : 0.0f;
      l[h] = l[h] * alpha + pe;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(pe, vf[e], o[h][e] * alpha);
    }
  }
  ACT* op = static_cast<ACT*>(a.out);
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      l[h] += __shfl_xor(l[h], off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] += __shfl_xor(o[h][e], off);
    }
    if (lane_row == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        store_act<ACT>(op, ((static_cast<size_t>(row) * a.C + i) * g.Hq + kh * G + h) * D + lane_col * EPL + e,
                       l[h] > 0.0f ? o[h][e] / l[h] : 0.0f);
    }
  }
}

template <typename ACT, int KV, int D>
static int launch_generic_d(const PrefillArgs& a, hipStream_t st) {
  const dim3 grid(a.C, a.B * a.g.Hkv), block(64);
  switch (a.g.g) {
    case 1: hipLaunchKernelGGL((prefill_attn_generic_kernel<ACT, KV, D, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_attn_generic_kernel<ACT, KV, D, 2>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((prefill_attn_generic_kernel<ACT, KV, D, 4>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((prefill_attn_generic_kernel<ACT, KV, D, 8>), grid, block, 0, st, a); break;
    default: return fail(DMS_ERR_UNSUPPORTED, "group size");
  }
  return DMS_OK;
}

template <typename ACT, int KV>
static int launch_generic(const PrefillArgs& a, hipStream_t st) {
  switch (a.g.D) {
    case 32: return launch_generic_d<ACT, KV, 32>(a, st);
    case 64: return launch_generic_d<ACT, KV, 64>(a, st);
    case 128: return launch_generic_d<ACT, KV, 128>(a, st);
    default: return fail(DMS_ERR_UNSUPPORTED, "head_dim");
  }
}

}  // namespace dms

using namespace dms;

extern "C" int dms_prefill_attn(dms_cache* cache, const int32_t* seq_ids, const void* q, const void* k,
                                const void* v, const uint8_t* evict, void* out, int B, int C, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  if (!q || !k || !v || !evict || !out) return fail(DMS_ERR_ARG, "q, k, v, evict and out are required");
  const Geo& g = cache->geo;
  if (B <= 0 || C <= 0) return fail(DMS_ERR_ARG, "B and C must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  if (C > g.max_chunk) return fail(DMS_ERR_CAPACITY, "C above max_chunk");
  PrefillArgs a{cache->dev, g, seq_ids, q, k, v, evict, out, B, C};
  hipStream_t st = as_stream(stream);
  int s;
  switch (g.kv_dtype) {
    case DMS_F32: s = launch_generic<float, DMS_F32>(a, st); break;
    case DMS_BF16: s = launch_generic<uint16_t, DMS_BF16>(a, st); break;
    case DMS_FP8_E4M3: s = launch_generic<uint16_t, DMS_FP8_E4M3>(a, st); break;
    default: return fail(DMS_ERR_UNSUPPORTED, "kv dtype");
  }
  if (s) return s;
  return check_hip(hipGetLastError(), "dms_prefill_attn launch");
}
