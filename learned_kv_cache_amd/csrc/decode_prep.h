// Decode-token preparation shared by dms_decode_prepare and dms_decode_step:
// the keep/evict decision of one (batch row, KV head) pair and the placement
// of its K/V row under delayed eviction, and the commit of the shared state.
//
// "基于 DMS 的 KV Cache 压缩实战" walkthrough: 决策来源一 / 决策来源二 (query-neuron and
// linear-adapter logits), 决策粒度 (layer mode), 推理模式 (in-place overwrite of the
// slot of position t - w when that token was marked, else the next slot).
//
// prep_pair runs in one 256-thread workgroup per pair.  It writes what no
// other workgroup of the launch reads (the K/V row into its slot, the slot's
// metadata) and leaves a plan record for the rest.  prep_commit runs in the
// last workgroup to arrive, when every read of shared state has happened: it
// opens pages (pops in row-major rank order, as dms_append_evict), writes the
// lengths and ring entries the pairs left to it, advances the positions and
// zeroes the query neurons of a query-neuron decision.  Plan records are
// written and read with device-scope atomic stores and loads, coherent across
// XCDs without an L2 write-back.
#pragma once

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
  const float* bias;
  const float* offsets;
  float alpha, eps;
  int per_layer, disable;
  float* logits_out;
  uint8_t* evict_out;
};


template <int LPR>
__device__ __forceinline__ float row_max_dyn_helper(float x) { return row_max_dpp<LPR>(x); }

__device__ __forceinline__ float piece_row_max(float x, int ppr) {
  switch (ppr) {
    case 2: return row_max_dpp<2>(x);
    case 4: return row_max_dpp<4>(x);
    case 8: return row_max_dpp<8>(x);
    case 16: return row_max_dpp<16>(x);
    default: return x;
  }
}

// 16 input bytes (8 bf16 or 4 f32) -> page bytes at dst (fp8: 8 or 4 bytes)
template <typename ACT, int KV>
__device__ __forceinline__ void store_piece(uint8_t* pages, int64_t row, int row_bytes, int piece, const uint4& x,
                                            float inv_scale) {
  if (KV == DMS_FP8_E4M3) {
    constexpr int N = 16 / sizeof(ACT);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float f[N];
    if (sizeof(ACT) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) f[i] = __uint_as_float(w[i]);
    }
    uint8_t* dst = pages + row * row_bytes + piece * N;
    if (N == 8) {
      uint2 o;
      o.x = f32_to_e4m3(f[0] * inv_scale) | (f32_to_e4m3(f[1] * inv_scale) << 8) |
            (f32_to_e4m3(f[2] * inv_scale) << 16) | (static_cast<uint32_t>(f32_to_e4m3(f[3] * inv_scale)) << 24);
      o.y = f32_to_e4m3(f[4] * inv_scale) | (f32_to_e4m3(f[5] * inv_scale) << 8) |
            (f32_to_e4m3(f[6] * inv_scale) << 16) | (static_cast<uint32_t>(f32_to_e4m3(f[7] * inv_scale)) << 24);
      *reinterpret_cast<uint2*>(dst) = o;
    } else {
      for (int i = 0; i < N; ++i) dst[i] = f32_to_e4m3(f[i] * inv_scale);
    }
  } else {
    // same element type in and out: a raw copy
    *reinterpret_cast<uint4*>(pages + row * row_bytes + piece * 16) = x;
  }
}

__device__ __forceinline__ float piece_amax(const uint4& x, bool bf16) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (bf16) {
      m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
    } else {
      m = fmaxf(m, fabsf(__uint_as_float(w[i])));
    }
  }
  return m;
}

constexpr int kPrepThreads = 256;

// Inputs of the decode decision.
struct PrepIn {
  const uint16_t* hidden;   // [B][H] bf16 (linear adapter)
  const float* gamma;       // [H]
  const float* W;           // [Hkv][H]
  uint16_t* q;              // [B][Hq][D] bf16 (query-neuron decision; its neurons are zeroed at commit)
  int qneuron;
};

// LDS of the prepare role.
struct PrepShared {
  float red[4][2];
  float rowred[4][17];      // prep_row: per-wave sums of h^2 and of the KV heads' products
  float lg[16];             // prep_row: the row's logits
  int last, free_top, used, n;
  int wave_cnt[4];
  int q[kPrepThreads], dst[kPrepThreads], page[kPrepThreads];
};

// Prepare workgroup p of nprep counts its arrival (thread 0, after its
// stores are complete): in group p % ng of the arrive lines, and the last of
// a group in the control word.  True for the one workgroup that completes
// the count, which commits.
__device__ __forceinline__ bool prep_arrive(const DevCache& d, int p, int nprep) {
  const int ng = min(kArriveGroups, nprep), gi = p % ng;
  const int n_g = nprep / ng + (gi < nprep % ng ? 1 : 0);
  return __hip_atomic_fetch_add(d.arrive + gi * kArriveStride + kPrepArriveWord, 1, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT) == n_g - 1 &&
         __hip_atomic_fetch_add(d.ctl + kCtlPrepArrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ng - 1;
}

// Resets what prep_arrive counted (the committing workgroup, once all have arrived).
__device__ __forceinline__ void prep_arrive_reset(const DevCache& d, int nprep, int tid) {
  const int ng = min(kArriveGroups, nprep);
  if (tid < ng)
    __hip_atomic_store(d.arrive + tid * kArriveStride + kPrepArriveWord, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) __hip_atomic_store(d.ctl + kCtlPrepArrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// plan record kinds (chunk_info[pair][0..7]: kind, unit, t, slot, e, dst, appended, length before)
constexpr int kPlanNone = 0;      // nothing to do (bad sequence id, capacity)
constexpr int kPlanDone = 1;      // the pair's workgroup wrote everything
constexpr int kPlanTables = 2;    // K/V row and slot metadata written; length and ring entry left to the commit
constexpr int kPlanNewPage = 3;   // opens a page: everything at the commit

template <int KV>
__device__ __forceinline__ void prep_store_row(const DevCache& d, int64_t dst, int page, bool new_page, int ppr,
                                               int piece, const uint4& kx, const uint4& vx, bool active) {
  const int page_row_bytes = (KV == DMS_BF16 ? 2 : 1) * ppr * 8;
  float inv_k = 1.0f, inv_v = 1.0f;
  if (KV == DMS_FP8_E4M3) {
    const float mk = piece_row_max(piece_amax(kx, true), ppr);
    const float mv = piece_row_max(piece_amax(vx, true), ppr);
    float sk, sv;
    if (new_page) {
      sk = page_scale_from_amax(mk);
      sv = page_scale_from_amax(mv);
      if (active && piece == 0) {
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
  if (active) {
    store_piece<uint16_t, KV>(d.k_pages, dst, page_row_bytes, piece, kx, inv_k);
    store_piece<uint16_t, KV>(d.v_pages, dst, page_row_bytes, piece, vx, inv_v);
  }
}


// One pair's decision and placement (all threads of the workgroup).  With
// defer_tables the length and ring entry are left to the commit (the fused
// decode step, whose attention workgroups read them).
template <int KV>
__device__ __forceinline__ void prep_pair(const AppendArgs& a, const PrepIn& in, int p, bool defer_tables,
                                          PrepShared& sh) {
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = p / g.Hkv, kh = p % g.Hkv;
  const int kk = a.per_layer ? 0 : kh;
  const int seq = a.seq_ids ? a.seq_ids[row] : row;
  const bool seq_ok = seq >= 0 && seq < g.Bmax;
  const int unit = seq_ok ? seq * g.Hkv + kh : 0;
  const int ppr = g.D / 8;                       // 16-byte pieces of a bf16 row

  // 1. what the slot waits on, and the K/V row
  int t = 0, len = 0, cur = -1;
  if (seq_ok) {
    t = d.pos[seq];
    len = d.lengths[unit];
    cur = d.cur_page[unit];
  }
  uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
  const size_t rowoff = static_cast<size_t>(p) * g.D * 2;
  if (tid < ppr) {
    kx = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.k) + rowoff + 16 * tid);
    vx = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.v) + rowoff + 16 * tid);
  }
  const int64_t ri = static_cast<int64_t>(unit) * g.w + (t % g.w);
  int rv = 0, rrow = -1;
  if (seq_ok && t >= g.w) {
    rv = d.ring[ri];
    rrow = d.ring_row[ri];
  }
  // 2. the logit
  float lg;
  if (in.qneuron) {
    const uint16_t qn = in.q[(static_cast<size_t>(row) * g.Hq + kk * g.g) * g.D + g.D - 1];
    lg = a.alpha * bf16_to_f32(qn) - a.offsets[kk];
  } else {
    // sum(h^2) and sum(gamma * W_k * h) over the row's hidden state
    float ss = 0.0f, dk = 0.0f;
    const uint16_t* h = in.hidden + static_cast<size_t>(row) * g.H;
    const float* w = in.W + static_cast<size_t>(kk) * g.H;
    for (int m = 8 * tid; m < g.H; m += 8 * kPrepThreads) {
      const uint4 hv = *reinterpret_cast<const uint4*>(h + m);
      const float4 g0 = *reinterpret_cast<const float4*>(in.gamma + m);
      const float4 g1 = *reinterpret_cast<const float4*>(in.gamma + m + 4);
      const float4 w0 = *reinterpret_cast<const float4*>(w + m), w1 = *reinterpret_cast<const float4*>(w + m + 4);
      const uint32_t u[4] = {hv.x, hv.y, hv.z, hv.w};
      const float gw[8] = {g0.x * w0.x, g0.y * w0.y, g0.z * w0.z, g0.w * w0.w,
                           g1.x * w1.x, g1.y * w1.y, g1.z * w1.z, g1.w * w1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = __uint_as_float((e & 1) ? (u[e >> 1] & 0xFFFF0000u) : (u[e >> 1] << 16));
        ss = fmaf(x, x, ss);
        dk = fmaf(gw[e], x, dk);
      }
    }
    ss = wave_sum_dpp(ss);
    dk = wave_sum_dpp(dk);
    if (lane == 0) {
      sh.red[wave][0] = ss;
      sh.red[wave][1] = dk;
    }
    __syncthreads();
    ss = (sh.red[0][0] + sh.red[1][0]) + (sh.red[2][0] + sh.red[3][0]);
    dk = (sh.red[0][1] + sh.red[1][1]) + (sh.red[2][1] + sh.red[3][1]);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(g.H) + a.eps);
    float z = r * dk;
    if (a.bias) z += a.bias[kk];
    lg = a.alpha * z - a.offsets[kk];
  }
  const int e = (!a.disable && lg > 0.0f) ? 1 : 0;
  if (tid == 0) {
    a.evict_out[p] = static_cast<uint8_t>(e);
    if (a.logits_out) a.logits_out[p] = lg;
  }

  // 3. the slot: in place, or the next slot of the current page, or a new page
  bool valid = seq_ok, new_page = false;
  int slot = 0, dst = -1, page = -1;
  if (!seq_ok) {
    if (tid == 0) set_status(d.ctl, DMS_DEV_BAD_SEQ);
  } else if (t + 1 > g.max_tokens) {
    if (tid == 0) set_status(d.ctl, DMS_DEV_CAPACITY);
    valid = false;
  } else {
    if (t >= g.w && rv < 0) {
      slot = rv & 0x7FFFFFFF;
      dst = rrow;
      page = dst / g.P;
    } else {
      slot = len;
      if (slot % g.P == 0) {
        new_page = true;
      } else {
        page = cur;
        dst = page * g.P + slot % g.P;
      }
    }
  }
  const int appended = slot == len;
  if (valid && !new_page) {
    if (tid == 0) {
      if (!defer_tables) {
        if (appended) d.lengths[unit] = slot + 1;
        d.ring[ri] = slot | (e << 31);
        d.ring_row[ri] = dst;
      }
      d.slot_meta[dst] = t | (e << 31);
    }
    if (wave == 0) prep_store_row<KV>(d, dst, page, false, ppr, lane % ppr, kx, vx, lane < ppr);
  }

  // 4. plan record
  if (tid == 0) {
    const int kind = !valid ? kPlanNone : new_page ? kPlanNewPage : defer_tables ? kPlanTables : kPlanDone;
    int32_t* pl = d.chunk_info + static_cast<int64_t>(p) * 8;
    const int vals[8] = {kind, unit, t, slot, e, dst, appended, len};
#pragma unroll
    for (int i = 0; i < 8; ++i) __hip_atomic_store(pl + i, vals[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One batch row's pairs in one workgroup (the fused decode step with many
// rows, where one workgroup per pair would not leave the attention room to be
// resident beside it): the linear adapter's sums over the row's hidden state
// are taken once for all the KV heads (each head's products in the same order
// as prep_pair, so the same logits), then wave w places pairs w, w + 4, ...
// exactly as prep_pair does (deferred tables).
template <int KV>
__device__ __forceinline__ void prep_row(const AppendArgs& a, const PrepIn& in, int row, PrepShared& sh) {
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Hkv = g.Hkv;
  const int nk = a.per_layer ? 1 : Hkv;          // distinct logits of the row
  const int seq = a.seq_ids ? a.seq_ids[row] : row;
  const bool seq_ok = seq >= 0 && seq < g.Bmax;
  const int ppr = g.D / 8;
  // 1. the logits
  if (in.qneuron) {
    if (tid < nk) {
      const uint16_t qn = in.q[(static_cast<size_t>(row) * g.Hq + tid * g.g) * g.D + g.D - 1];
      sh.lg[tid] = a.alpha * bf16_to_f32(qn) - a.offsets[tid];
    }
  } else {
    float ss = 0.0f, dk[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) dk[k] = 0.0f;
    const uint16_t* h = in.hidden + static_cast<size_t>(row) * g.H;
    for (int m = 8 * tid; m < g.H; m += 8 * kPrepThreads) {
      const uint4 hv = *reinterpret_cast<const uint4*>(h + m);
      const float4 g0 = *reinterpret_cast<const float4*>(in.gamma + m);
      const float4 g1 = *reinterpret_cast<const float4*>(in.gamma + m + 4);
      const uint32_t u[4] = {hv.x, hv.y, hv.z, hv.w};
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = __uint_as_float((e & 1) ? (u[e >> 1] & 0xFFFF0000u) : (u[e >> 1] << 16));
        ss = fmaf(x[e], x[e], ss);
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k >= nk) break;
        const float* w = in.W + static_cast<size_t>(k) * g.H;
        const float4 w0 = *reinterpret_cast<const float4*>(w + m), w1 = *reinterpret_cast<const float4*>(w + m + 4);
        const float gw[8] = {g0.x * w0.x, g0.y * w0.y, g0.z * w0.z, g0.w * w0.w,
                             g1.x * w1.x, g1.y * w1.y, g1.z * w1.z, g1.w * w1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) dk[k] = fmaf(gw[e], x[e], dk[k]);
      }
    }
    ss = wave_sum_dpp(ss);
    if (lane == 0) sh.rowred[wave][16] = ss;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k >= nk) break;
      const float v = wave_sum_dpp(dk[k]);
      if (lane == 0) sh.rowred[wave][k] = v;
    }
    __syncthreads();
    if (tid < nk) {
      const float s2 = (sh.rowred[0][16] + sh.rowred[1][16]) + (sh.rowred[2][16] + sh.rowred[3][16]);
      const float dd = (sh.rowred[0][tid] + sh.rowred[1][tid]) + (sh.rowred[2][tid] + sh.rowred[3][tid]);
      const float r = 1.0f / sqrtf(s2 / static_cast<float>(g.H) + a.eps);
      float z = r * dd;
      if (a.bias) z += a.bias[tid];
      sh.lg[tid] = a.alpha * z - a.offsets[tid];
    }
  }
  __syncthreads();
  if (!seq_ok) {
    if (tid == 0) set_status(d.ctl, DMS_DEV_BAD_SEQ);
  }
  const int t = seq_ok ? d.pos[seq] : 0;
  // 2. the pairs, one wave each
  for (int kh = wave; kh < Hkv; kh += 4) {
    const int p = row * Hkv + kh;
    const int unit = seq_ok ? seq * Hkv + kh : 0;
    int len = 0, cur = -1;
    if (seq_ok) {
      len = d.lengths[unit];
      cur = d.cur_page[unit];
    }
    uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
    const size_t rowoff = static_cast<size_t>(p) * g.D * 2;
    if (lane < ppr) {
      kx = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.k) + rowoff + 16 * lane);
      vx = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.v) + rowoff + 16 * lane);
    }
    const int64_t ri = static_cast<int64_t>(unit) * g.w + (t % g.w);
    int rv = 0, rrow = -1;
    if (seq_ok && t >= g.w) {
      rv = d.ring[ri];
      rrow = d.ring_row[ri];
    }
    const float lg = sh.lg[a.per_layer ? 0 : kh];
    const int e = (!a.disable && lg > 0.0f) ? 1 : 0;
    if (lane == 0) {
      a.evict_out[p] = static_cast<uint8_t>(e);
      if (a.logits_out) a.logits_out[p] = lg;
    }
    bool valid = seq_ok, new_page = false;
    int slot = 0, dst = -1, page = -1;
    if (seq_ok) {
      if (t + 1 > g.max_tokens) {
        if (lane == 0) set_status(d.ctl, DMS_DEV_CAPACITY);
        valid = false;
      } else if (t >= g.w && rv < 0) {
        slot = rv & 0x7FFFFFFF;
        dst = rrow;
        page = dst / g.P;
      } else {
        slot = len;
        if (slot % g.P == 0) {
          new_page = true;
        } else {
          page = cur;
          dst = page * g.P + slot % g.P;
        }
      }
    }
    const int appended = slot == len;
    if (valid && !new_page) {
      if (lane == 0) d.slot_meta[dst] = t | (e << 31);
      prep_store_row<KV>(d, dst, page, false, ppr, lane % ppr, kx, vx, lane < ppr);
    }
    if (lane == 0) {
      const int kind = !valid ? kPlanNone : new_page ? kPlanNewPage : kPlanTables;
      int32_t* pl = d.chunk_info + static_cast<int64_t>(p) * 8;
      const int vals[8] = {kind, unit, t, slot, e, dst, appended, len};
#pragma unroll
      for (int i = 0; i < 8; ++i) __hip_atomic_store(pl + i, vals[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The commit (all threads of the last workgroup to arrive): tables left by
// the pairs, pages opened in row-major rank order with their K/V rows, the
// positions, the pool top, the query neurons; then the arrival counter reset.
template <int KV>
__device__ __forceinline__ void prep_commit(const AppendArgs& a, const PrepIn& in, int npairs, PrepShared& sh) {
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ppr = g.D / 8;
  if (tid == 0) {
    sh.free_top = d.ctl[kCtlFreeCount];
    sh.used = 0;
  }
  __syncthreads();
  for (int p0 = 0; p0 < npairs; p0 += kPrepThreads) {
    const int q = p0 + tid;
    int kind = kPlanNone, qu = 0, qt = 0, qslot = 0, qe = 0, qdst = 0, qapp = 0;
    if (q < npairs) {
      int32_t* pl = d.chunk_info + static_cast<int64_t>(q) * 8;
      kind = __hip_atomic_load(pl + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      qu = __hip_atomic_load(pl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      qt = __hip_atomic_load(pl + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      qslot = __hip_atomic_load(pl + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      qe = __hip_atomic_load(pl + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      qdst = __hip_atomic_load(pl + 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      qapp = __hip_atomic_load(pl + 6, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int64_t qri = static_cast<int64_t>(qu) * g.w + (qt % g.w);
    if (kind == kPlanTables) {
      if (qapp) d.lengths[qu] = qslot + 1;
      d.ring[qri] = qslot | (qe << 31);
      d.ring_row[qri] = qdst;
    }
    const bool need = kind == kPlanNewPage;
    int wtot;
    const int wr = wave_rank(need, &wtot);
    if (lane == 0) sh.wave_cnt[wave] = wtot;
    if (tid == 0) sh.n = 0;
    __syncthreads();
    int off = 0, tot = 0;
    for (int i = 0; i < 4; ++i) {
      if (i < wave) off += sh.wave_cnt[i];
      tot += sh.wave_cnt[i];
    }
    if (need) {
      const int R = sh.used + off + wr;
      if (R < sh.free_top) {
        const int pg = d.free_stack[sh.free_top - 1 - R];
        const int ndst = pg * g.P + qslot % g.P;
        d.page_table[static_cast<int64_t>(qu) * g.maxp + qslot / g.P] = pg;
        d.cur_page[qu] = pg;
        d.lengths[qu] = qslot + 1;
        d.ring[qri] = qslot | (qe << 31);
        d.ring_row[qri] = ndst;
        d.slot_meta[ndst] = qt | (qe << 31);
        const int at = atomicAdd(&sh.n, 1);
        sh.q[at] = q;
        sh.dst[at] = ndst;
        sh.page[at] = pg;
      } else {
        set_status(d.ctl, DMS_DEV_POOL_EXHAUSTED);
      }
    }
    __syncthreads();
    // rows of the pairs that opened a page: one wave per row
    for (int i = wave; i < sh.n; i += 4) {
      const int q2 = sh.q[i];
      const size_t ro = static_cast<size_t>(q2) * g.D * 2;
      const int piece = lane % ppr;
      const uint4 k2 = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.k) + ro + 16 * piece);
      const uint4 v2 = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.v) + ro + 16 * piece);
      prep_store_row<KV>(d, sh.dst[i], sh.page[i], true, ppr, piece, k2, v2, lane < ppr);
    }
    __syncthreads();
    if (tid == 0) sh.used += tot;
    __syncthreads();
  }
  for (int rr = tid; rr < a.B; rr += kPrepThreads) {
    const int sq = a.seq_ids ? a.seq_ids[rr] : rr;
    if (sq >= 0 && sq < g.Bmax && d.pos[sq] + 1 <= g.max_tokens) d.pos[sq] += 1;
  }
  if (in.qneuron) {
    for (int q = tid; q < npairs; q += kPrepThreads)
      in.q[(static_cast<size_t>(q / g.Hkv) * g.Hq + (q % g.Hkv) * g.g) * g.D + g.D - 1] = 0;
  }
  if (tid == 0) d.ctl[kCtlFreeCount] = sh.free_top - min(sh.used, sh.free_top);
}

}  // namespace dms
