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
// Two kernels:
//  * prefill_attn_mfma_kernel (bf16 activations, bf16 or fp8 pages, head_dim
//    64/128, GQA group 1/2/4, block a multiple of 32): flash-attention on the
//    16x16x32 bf16 matrix cores.  Both products keep the query on the MFMA
//    column:  S^T = K Q^T  and  O^T = V^T P^T,  so the probabilities leave the
//    first product already in the operand layout of the second and the
//    softmax statistics of a column never leave its lane.
//  * prefill_attn_generic_kernel: vector ALU, every dtype and head size.
#include <cmath>
#include <cstdlib>

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
  const float* gate;    // training forward: [B][Hkv][C] gate logits of the keys (cache unused)
  float* lse;           // training forward: [B][Hq][C] natural-log softmax normaliser per query
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


// ---------------------------------------------------------------------------
// Matrix-core kernel.
//
// Workgroup: 8 waves (two per SIMD, so one wave's softmax overlaps the other's
// matrix products), one (sequence, KV head) and a block of query tokens.  Each
// wave owns 2 column tiles of 16 queries (token x query head; the mask depends
// on the token only).  Keys stream through LDS in blocks of 32: the cache
// slots 0..L-1 first (visibility from the slot metadata), then the chunk's own
// keys up to the workgroup's last token.  Each key carries a visibility
// interval [lo, hi) of query positions: lo = its position, hi = position + w
// when its flag is set (delayed eviction), else unbounded.
//
// MFMA 16x16x32 bf16 operand layout (lane l, G4 = l / 16, i = 0..7):
//   A[row l%16][k 8*G4+i], B[k 8*G4+i][col l%16], D[row 4*G4+r][col l%16].
// S^T = K Q^T: A = K rows from LDS, B = Q^T fragments held in registers;
// lane l gets the scores of keys 4*G4+r (and 16+4*G4+r) for query l%16.
// O^T = V^T P^T: B = P^T is exactly those 8 probabilities per lane when the
// key index k of the second product is permuted as
//   k = 8*G4 + i  <->  key (i < 4 ? 4*G4 + i : 16 + 4*G4 + i - 4).
// V stays row-major in LDS like K; its A fragments (4 keys at one head_dim
// column per lane, twice) come from the transposing LDS read
// ds_read_b64_tr_b16: within 16 lanes, lane i receives elements i, 16+i,
// 32+i, 48+i of the 64 the group addresses, so lanes 4r..4r+3 pointing at 16
// consecutive columns of key row r hand lane i the column i of 4 keys.  One
// more product with an all-ones A gives the softmax denominator of the same
// bf16-rounded probabilities in every row of an extra accumulator tile.
//
// LDS rows are 2*D + 32 bytes: with that stride both the K reads (16 bytes
// per lane) and the transposing V reads are free of bank conflicts on gfx950.

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef short pf_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) pf_i16x4 pf_lds_i16x4;
typedef __bf16 pf_bf16x2 __attribute__((ext_vector_type(2)));
typedef float pf_f32x4 __attribute__((ext_vector_type(4)));
typedef float pf_f32x2 __attribute__((ext_vector_type(2)));

constexpr int kPfKB = 32;         // keys per LDS block
constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfNoLimit = 0x7FFFFFFF;
constexpr int kPfMaxPages = 4096;  // page-table entries of a unit held in LDS (larger tables: vector kernel)
constexpr float kPfRescaleLog2 = 8.0f;   // running max is raised only when exceeded by this (log2 units)

template <int D, int G, bool FP8>
struct PfShape {
  static constexpr int HW = G < 2 ? G : 2;    // query heads per wave
  static constexpr int HS = G / HW;           // waves sharing one token group (head split)
  static constexpr int TG = 2 / HW;           // 16-token groups per wave
  static constexpr int NT = TG * HW;          // column tiles per wave (2)
  static constexpr int TOKW = 16 * TG;        // tokens per wave
  static constexpr int TOKB = TOKW * kPfWaves / HS;   // tokens per workgroup
  static constexpr int KS = D / 32;           // k-steps of S^T over head_dim
  static constexpr int DT = D / 16;           // 16-row tiles of O^T
  // LDS tiles of one key block.  bf16 pages arrive by direct global->LDS
  // loads into unpadded rows whose 16-byte chunks are XOR-swizzled per row;
  // fp8 pages are dequantised through registers into rows padded to 2D+32
  // bytes.  Both layouts keep the K reads and the transposing V reads free of
  // bank conflicts on gfx950.
  static constexpr bool DMA = !FP8;
  static constexpr int ROW = DMA ? 2 * D : 2 * D + 32;
  static constexpr int CPR = 2 * D / 16;      // 16-byte chunks per row
  static constexpr int V_OFF = kPfKB * ROW;
  static constexpr int META_OFF = 2 * kPfKB * ROW;   // slot metadata of the block's cache keys
  static constexpr int LO_OFF = META_OFF + 4 * kPfKB;
  static constexpr int HI_OFF = LO_OFF + 4 * kPfKB;
  static constexpr int PEN_OFF = HI_OFF + 4 * kPfKB;  // training forward: gate logit, then penalty / scale
  static constexpr int BUF = PEN_OFF + 4 * kPfKB;
  static constexpr int DC = D / 8;            // 16-byte pieces per bf16 row
  static constexpr int STHREADS = kPfKB * DC; // register path: threads staging one K and one V piece each
  static_assert(NT == 2 && STHREADS <= kPfThreads, "shape");
  static_assert(BUF % 16 == 0 && (!DMA || 1024 % ROW == 0), "LDS layout");
  __device__ static int swz(int r) { return D == 128 ? 2 * (r & 7) : (r & 6); }
  // byte offset of 16-byte chunk c of row r in a tile
  __device__ static int off(int r, int c) { return r * ROW + 16 * (DMA ? (c ^ swz(r)) : c); }
};

// max / sum of lane l and lane l ^ 32 (resp. l ^ 16): v_permlane32_swap and
// v_permlane16_swap return the pair (own, partner) in a lane-independent order.
__device__ __forceinline__ float pf_max_x32(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pf_max_x16(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ uint32_t pf_pack(float lo, float hi) {
  pf_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, pf_bf16x2));
}

// Eight e4m3 codes times a power-of-two page scale -> eight bf16 (exact).
__device__ __forceinline__ uint4 pf_fp8x8_to_bf16(uint32_t w0, uint32_t w1, float sc) {
  const pf_f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
  const pf_f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false), e = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
  return make_uint4(pf_pack(a[0] * sc, a[1] * sc), pf_pack(b[0] * sc, b[1] * sc), pf_pack(c[0] * sc, c[1] * sc),
                    pf_pack(e[0] * sc, e[1] * sc));
}

// Per-call constants of one (sequence, KV head) as staging needs them.
struct PfSrc {
  const int32_t* pt;
  const uint8_t* kchunk;   // chunk key 0 of this KV head (bytes)
  const uint8_t* vchunk;
  const uint8_t* ev;
  int L, s0, nk;
  int64_t chunk_stride;    // bytes between consecutive chunk keys
};

// A 16-byte piece (8 elements from element 8*dc) of key kk's K or V row, as
// loaded; `page` is the block's cache page (uniform), valid when kk < L.
struct PfRaw {
  uint4 w;
  float sc;
  int kind;     // 0: zeros (past the keys), 1: cache page row, 2: chunk row
};

template <int D, bool FP8>
__device__ __forceinline__ PfRaw pf_load(const PrefillArgs& a, const PfSrc& q, int page, int kk, int dc, bool v) {
  PfRaw r;
  r.sc = 1.0f;
  // keys past the end are masked out by their visibility interval; they read
  // the last key's row so every loaded value is finite
  const int kc = min(kk, q.nk - 1);
  const bool cache = kc < q.L;
  r.kind = cache ? 1 : 2;
  const int64_t prow = (static_cast<int64_t>(page) << a.g.Pshift) + (kc & (a.g.P - 1));
  if (FP8) {
    if (cache) {
      const uint8_t* base = (v ? a.d.v_pages : a.d.k_pages) + prow * D;
      const uint2 t = *reinterpret_cast<const uint2*>(base + 8 * dc);
      r.w = make_uint4(t.x, t.y, 0, 0);
      r.sc = a.d.scales[2 * page + (v ? 1 : 0)];
    } else {
      r.w = *reinterpret_cast<const uint4*>((v ? q.vchunk : q.kchunk) + (kc - q.L) * q.chunk_stride + 16 * dc);
    }
  } else {
    const uint8_t* pbase = (v ? a.d.v_pages : a.d.k_pages) + prow * D * 2;
    const uint8_t* cbase = (v ? q.vchunk : q.kchunk) + (kc - q.L) * q.chunk_stride;
    r.w = *reinterpret_cast<const uint4*>((cache ? pbase : cbase) + 16 * dc);
  }
  return r;
}

template <bool FP8>
__device__ __forceinline__ uint4 pf_bf16(const PfRaw& r) {
  if (FP8 && r.kind == 1) return pf_fp8x8_to_bf16(r.w.x, r.w.y, r.sc);
  return r.w;
}

typedef __attribute__((address_space(3))) void pf_lds_void;
typedef __attribute__((address_space(1))) void pf_glb_void;

// TRAIN: the training-mode forward (walkthrough, 训练模式): no cache, the
// chunk is the whole sequence from position 0, every causal key stays, and a
// key j gets the penalty logsigmoid(-y_j) added to its score for queries at
// distance w or more (y = the key's gate logit); writes the per-query
// log-sum-exp as well.
template <int D, int G, bool FP8, bool TRAIN = false>
__global__ __launch_bounds__(kPfThreads) void prefill_attn_mfma_kernel(PrefillArgs a) {
  using S = PfShape<D, G, FP8>;
  static_assert(!TRAIN || !FP8, "the training forward reads bf16 rows");
  // two key-block buffers as separate arrays: with the loop unrolled by two
  // each step's buffers are static, so loads into one are known not to alias
  // reads of the other
  __shared__ __attribute__((aligned(16))) uint8_t sbuf0[S::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t sbuf1[S::BUF];
  __shared__ int s_pt[kPfMaxPages];      // the unit's page table
  __shared__ uint8_t s_ev[kMaxChunk];    // the chunk's evict flags of this KV head
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int l16 = lane & 15, G4 = lane >> 4;

  // Linear workgroup id -> (pair, token block), the heaviest (last) token
  // blocks first; consecutive ids cycle through the pairs.
  const int npairs = a.B * g.Hkv;
  const int ntb = (a.C + S::TOKB - 1) / S::TOKB;
  const int pair = blockIdx.x % npairs;
  const int tb = ntb - 1 - static_cast<int>(blockIdx.x) / npairs;
  const int row = pair / g.Hkv, kh = pair % g.Hkv;
  const int seq = (a.seq_ids && !TRAIN) ? a.seq_ids[row] : row;
  if (!TRAIN && (seq < 0 || seq >= g.Bmax)) {   // uniform over the workgroup: no wave reaches a barrier
    if (tid == 0 && tb == 0 && kh == 0) set_status(d.ctl, DMS_DEV_BAD_SEQ);
    return;
  }
  const int unit = seq * g.Hkv + kh;
  PfSrc src;
  if constexpr (TRAIN) {
    src.pt = nullptr;
    src.L = 0;
    src.s0 = 0;
  } else {
    src.pt = d.page_table + static_cast<int64_t>(unit) * g.maxp;
    src.L = d.lengths[unit];
    src.s0 = d.pos[seq];
  }
  const int tok0 = tb * S::TOKB;
  const int tok_end = min(tok0 + S::TOKB, a.C);
  src.nk = src.L + tok_end;
  src.chunk_stride = static_cast<int64_t>(g.Hkv) * D * 2;
  const size_t chunk0 = (static_cast<size_t>(row) * a.C * g.Hkv + kh) * D * 2;
  src.kchunk = static_cast<const uint8_t*>(a.k) + chunk0;
  src.vchunk = static_cast<const uint8_t*>(a.v) + chunk0;
  src.ev = TRAIN ? nullptr : a.evict + static_cast<int64_t>(pair) * a.C;
  const float* gate = TRAIN ? a.gate + static_cast<int64_t>(pair) * a.C : nullptr;
  const int nblk = (src.nk + kPfKB - 1) / kPfKB;

  // ---- this wave's query columns: tile c = tg * HW + h
  const int hp = wave % S::HS, tp = wave / S::HS;
  const int wtok = tok0 + tp * S::TOKW;
  const int head0 = kh * G + hp * S::HW;
  int qpos[S::TG];
  bool qok[S::TG];
#pragma unroll
  for (int tg = 0; tg < S::TG; ++tg) {
    const int t = wtok + tg * 16 + l16;
    qok[tg] = t < a.C;
    qpos[tg] = qok[tg] ? src.s0 + t : -1;
  }
  // tokens grow with tg: the first group is live whenever any is; groups past
  // the chunk end hold position -1 and must not lower the upper bound
  const int qmin = qpos[0];
  int qmax = qpos[0];
#pragma unroll
  for (int tg = 1; tg < S::TG; ++tg) qmax = max(qmax, qpos[tg]);
  const bool lane_live = qok[0];

  pf_bf16x8 qf[S::NT][S::KS];
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int tg = 0; tg < S::TG; ++tg) {
#pragma unroll
    for (int h = 0; h < S::HW; ++h) {
      const int c = tg * S::HW + h;
      const int t = wtok + tg * 16 + l16;
      const size_t qrow = ((static_cast<size_t>(row) * a.C + t) * g.Hq + head0 + h) * D;
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (qok[tg]) w = *reinterpret_cast<const uint4*>(qbase + qrow + 32 * ks + 8 * G4);
        qf[c][ks] = __builtin_bit_cast(pf_bf16x8, w);
      }
    }
  }

  pf_f32x4 o[S::NT][S::DT], lacc[S::NT];
  float m[S::NT], mb[S::NT];
#pragma unroll
  for (int c = 0; c < S::NT; ++c) {
    m[c] = -INFINITY;
    mb[c] = 0.0f;
    lacc[c] = pf_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) o[c][dt] = pf_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float cs = g.scale_log2;
  const pf_bf16x8 ones = __builtin_bit_cast(pf_bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

  // ---- the unit's page table and the chunk's evict flags, once
  if constexpr (!TRAIN) {
    const int npages = (src.L + g.P - 1) >> g.Pshift;   // <= kPfMaxPages (checked at launch)
    for (int i = tid; i < npages; i += kPfThreads) s_pt[i] = src.pt[i];
    for (int i = tid; i < tok_end; i += kPfThreads) s_ev[i] = src.ev[i];
  }
  __syncthreads();
  // page of a key block (P is a multiple of the block: one page per block)
  auto block_page = [&](int kb) { return kb < src.L ? s_pt[kb >> g.Pshift] : 0; };

  // ---- visibility intervals [lo, hi) of a block's keys, by lanes 0..31 of the
  // last wave; cache keys decode the slot metadata staged at META_OFF
  const bool vis_wave = wave == kPfWaves - 1;
  // (TRAIN: [lo, hi) = [position, position + w): causal from lo, penalised
  // from hi; the gate logit staged at PEN_OFF becomes logsigmoid(-y) / scale,
  // so that adding it to the raw dot product adds logsigmoid(-y) to the
  // scaled score)
  auto vis_write = [&](int blk, uint8_t* b, int meta) {
    if (vis_wave && lane < kPfKB) {
      const int kk = blk * kPfKB + lane;
      int lo, hi;
      if (TRAIN) {
        float* pen = reinterpret_cast<float*>(b + S::PEN_OFF);
        if (kk < src.nk) {
          lo = kk;
          hi = kk + g.w;
          const float y = pen[lane];
          // logsigmoid(-y) = -softplus(y), stable for either sign
          const float ls = -(fmaxf(y, 0.0f) + log1pf(__expf(-fabsf(y))));
          pen[lane] = ls * (1.4426950408889634f / g.scale_log2);
        } else {
          lo = kPfNoLimit;
          hi = 0;
          pen[lane] = 0.0f;
        }
      } else if (kk < src.L) {
        lo = meta & 0x7FFFFFFF;
        hi = meta < 0 ? lo + g.w : kPfNoLimit;
      } else if (kk < src.nk) {
        lo = src.s0 + (kk - src.L);
        hi = s_ev[kk - src.L] ? lo + g.w : kPfNoLimit;
      } else {
        lo = kPfNoLimit;
        hi = 0;
      }
      reinterpret_cast<int*>(b + S::LO_OFF)[lane] = lo;
      reinterpret_cast<int*>(b + S::HI_OFF)[lane] = hi;
    }
  };

  // ---- one key block's products and softmax (LDS buffer b)
  auto compute = [&](const uint8_t* b) {
    const int4 lo0 = *reinterpret_cast<const int4*>(b + S::LO_OFF + 16 * G4);
    const int4 lo1 = *reinterpret_cast<const int4*>(b + S::LO_OFF + 64 + 16 * G4);
    const int4 hi0 = *reinterpret_cast<const int4*>(b + S::HI_OFF + 16 * G4);
    const int4 hi1 = *reinterpret_cast<const int4*>(b + S::HI_OFF + 64 + 16 * G4);
    const int lmin = min(min(min(lo0.x, lo0.y), min(lo0.z, lo0.w)), min(min(lo1.x, lo1.y), min(lo1.z, lo1.w)));
    const int lmax = max(max(max(lo0.x, lo0.y), max(lo0.z, lo0.w)), max(max(lo1.x, lo1.y), max(lo1.z, lo1.w)));
    const int hmin = min(min(min(hi0.x, hi0.y), min(hi0.z, hi0.w)), min(min(hi1.x, hi1.y), min(hi1.z, hi1.w)));
    const int hmax = max(max(max(hi0.x, hi0.y), max(hi0.z, hi0.w)), max(max(hi1.x, hi1.y), max(hi1.z, hi1.w)));
    // (TRAIN: hi only starts the penalty, it hides nothing)
    const bool lane_none = !lane_live || lmin > qmax || (!TRAIN && hmax <= qmin);
    const bool lane_all = !lane_live || (lmax <= qmin && hmin > qmax);
    if (__all(lane_none)) return;
    // S^T = K Q^T
    pf_f32x4 s[2][S::NT];
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const pf_bf16x8 kf = *reinterpret_cast<const pf_bf16x8*>(b + S::off(16 * kt + l16, 4 * ks + G4));
#pragma unroll
        for (int c = 0; c < S::NT; ++c)
          s[kt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf, qf[c][ks], ks == 0 ? pf_f32x4{0.0f, 0.0f, 0.0f, 0.0f} : s[kt][c], 0, 0, 0);
      }
    }
    if (!__all(lane_all)) {
      const int los[8] = {lo0.x, lo0.y, lo0.z, lo0.w, lo1.x, lo1.y, lo1.z, lo1.w};
      const int his[8] = {hi0.x, hi0.y, hi0.z, hi0.w, hi1.x, hi1.y, hi1.z, hi1.w};
      if constexpr (TRAIN) {
        const float4 pa = *reinterpret_cast<const float4*>(b + S::PEN_OFF + 16 * G4);
        const float4 pb = *reinterpret_cast<const float4*>(b + S::PEN_OFF + 64 + 16 * G4);
        const float pens[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
        // every pair causal and past the window (most blocks of a long
        // sequence): the penalty alone, without per-element tests
        const bool lane_pen = !lane_live || (lmax <= qmin && hmax <= qmin);
        if (__all(lane_pen)) {
#pragma unroll
          for (int c = 0; c < S::NT; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e >> 2][c][e & 3] += pens[e];
        } else {
#pragma unroll
          for (int c = 0; c < S::NT; ++c) {
            const int qp = qpos[c / S::HW];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = s[e >> 2][c][e & 3] + (qp >= his[e] ? pens[e] : 0.0f);
              s[e >> 2][c][e & 3] = los[e] <= qp ? v : -INFINITY;
            }
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < S::NT; ++c) {
          const int qp = qpos[c / S::HW];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool vis = los[e] <= qp && qp < his[e];
            s[e >> 2][c][e & 3] = vis ? s[e >> 2][c][e & 3] : -INFINITY;
          }
        }
      }
    }
    // running max per column, raised lazily (probabilities stay below 2^8)
    float mx[S::NT];
    bool need = false;
#pragma unroll
    for (int c = 0; c < S::NT; ++c) {
      float x = fmaxf(fmaxf(fmaxf(s[0][c][0], s[0][c][1]), fmaxf(s[0][c][2], s[0][c][3])),
                      fmaxf(fmaxf(s[1][c][0], s[1][c][1]), fmaxf(s[1][c][2], s[1][c][3])));
      x = pf_max_x32(x);
      x = pf_max_x16(x);
      mx[c] = x;
      need |= x * cs > m[c] * cs + kPfRescaleLog2;
    }
    if (__any(need)) {
#pragma unroll
      for (int c = 0; c < S::NT; ++c) {
        if (mx[c] * cs > m[c] * cs + kPfRescaleLog2) {
          const float alpha = __builtin_amdgcn_exp2f((m[c] - mx[c]) * cs);   // 0 from -inf
          m[c] = mx[c];
          mb[c] = mx[c] * cs;
          lacc[c] *= alpha;
#pragma unroll
          for (int dt = 0; dt < S::DT; ++dt) o[c][dt] *= alpha;
        }
      }
    }
    // P^T (bf16) and O^T += V^T P^T, denominator += 1^T P^T
    pf_bf16x8 pk[S::NT];
#pragma unroll
    for (int c = 0; c < S::NT; ++c) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(s[e >> 2][c][e & 3], cs, -mb[c]));
      const uint4 w = make_uint4(pf_pack(p[0], p[1]), pf_pack(p[2], p[3]), pf_pack(p[4], p[5]), pf_pack(p[6], p[7]));
      pk[c] = __builtin_bit_cast(pf_bf16x8, w);
      lacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pk[c], lacc[c], 0, 0, 0);
    }
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
      // keys 4*G4 + 0..3 and 16 + 4*G4 + 0..3 at column 16*dt + l16
      const int r0 = 4 * G4 + (l16 >> 2), ch = 2 * dt + ((l16 & 3) >> 1), half = 8 * (l16 & 1);
      const uint8_t* vb = b + S::V_OFF;
      const pf_i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pf_lds_i16x4*)(vb + S::off(r0, ch) + half));
      const pf_i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pf_lds_i16x4*)(vb + S::off(r0 + 16, ch) + half));
      const pf_bf16x8 vf = __builtin_bit_cast(pf_bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int c = 0; c < S::NT; ++c) o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pk[c], o[c][dt], 0, 0, 0);
    }
  };

  if constexpr (S::DMA) {
    // ---- bf16 pages: direct global->LDS loads.  Lane i of a wave-wide load
    // writes bytes [16 i, 16 i + 16) of a 1 KB stretch (whole rows); it reads
    // the chunk that the row's swizzle places there.  Keys past the end read
    // the last key's row (finite values; their interval hides them).
    auto row_src = [&](int page, int kk, bool v) {
      const int kc = min(kk, src.nk - 1);
      const uint8_t* pr = (v ? d.v_pages : d.k_pages) +
                          ((static_cast<int64_t>(page) << g.Pshift) + (kc & (g.P - 1))) * (D * 2);
      const uint8_t* cr = (v ? src.vchunk : src.kchunk) + static_cast<int64_t>(kc - src.L) * src.chunk_stride;
      return kc < src.L ? pr : cr;
    };
    auto dma_issue = [&](int blk, uint8_t* b) {
      const int kb = blk * kPfKB;
      const int page = block_page(kb);
      constexpr int RPW = 1024 / S::ROW;   // rows per wave-wide load
      if constexpr (D == 128) {
        const int r = wave * RPW + lane / S::CPR, c = (lane % S::CPR) ^ S::swz(r);
        __builtin_amdgcn_global_load_lds((const pf_glb_void*)(row_src(page, kb + r, false) + 16 * c),
                                         (pf_lds_void*)(b + wave * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const pf_glb_void*)(row_src(page, kb + r, true) + 16 * c),
                                         (pf_lds_void*)(b + S::V_OFF + wave * 1024), 16, 0, 0);
      } else {
        const int w4 = wave & 3;
        const bool isv = wave >= 4;
        const int r = w4 * RPW + lane / S::CPR, c = (lane % S::CPR) ^ S::swz(r);
        __builtin_amdgcn_global_load_lds((const pf_glb_void*)(row_src(page, kb + r, isv) + 16 * c),
                                         (pf_lds_void*)(b + (isv ? S::V_OFF : 0) + w4 * 1024), 16, 0, 0);
      }
      if (TRAIN && vis_wave && lane < kPfKB) {
        __builtin_amdgcn_global_load_lds((const pf_glb_void*)(gate + min(kb + lane, src.nk - 1)),
                                         (pf_lds_void*)(b + S::PEN_OFF), 4, 0, 0);
      }
      if (!TRAIN && vis_wave && kb < src.L && lane < kPfKB) {
        const int kc = min(kb + lane, src.L - 1);   // same page as kb
        __builtin_amdgcn_global_load_lds(
            (const pf_glb_void*)(d.slot_meta + (static_cast<int64_t>(page) << g.Pshift) + (kc & (g.P - 1))),
            (pf_lds_void*)(b + S::META_OFF), 4, 0, 0);
      }
    };
    auto vis_from_lds = [&](int blk, uint8_t* b) {
      const int meta = vis_wave && lane < kPfKB ? reinterpret_cast<const int*>(b + S::META_OFF)[lane] : 0;
      vis_write(blk, b, meta);
    };

    dma_issue(0, sbuf0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    vis_from_lds(0, sbuf0);
    __syncthreads();
    // block blk in sbuf0 while blk+1 loads into sbuf1, then the reverse; each
    // step ends with this wave's loads complete and one barrier
    for (int blk = 0; blk < nblk; blk += 2) {
      if (blk + 1 < nblk) dma_issue(blk + 1, sbuf1);
      compute(sbuf0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (blk + 1 < nblk) vis_from_lds(blk + 1, sbuf1);
      __syncthreads();
      if (blk + 1 >= nblk) break;
      if (blk + 2 < nblk) dma_issue(blk + 2, sbuf0);
      compute(sbuf1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (blk + 2 < nblk) vis_from_lds(blk + 2, sbuf0);
      __syncthreads();
    }
  } else {
    // ---- fp8 pages: loads into registers two blocks ahead of the LDS
    // writes; staging runs unconditionally (blocks past the end load clamped
    // rows and land in a buffer nobody reads again), so every path issues and
    // consumes the same loads
    const int skey = tid / S::DC, sdc = tid % S::DC;
    struct Stage {
      PfRaw k, v;
      int meta;     // slot metadata of the key's cache row (visibility wave)
    };
    Stage st0, st1;
    auto stage_load = [&](int blk, Stage& sg) {
      const int kb = blk * kPfKB;
      const int page = block_page(kb);
      if (tid < S::STHREADS) {
        const int kk = kb + skey;
        sg.k = pf_load<D, FP8>(a, src, page, kk, sdc, false);
        sg.v = pf_load<D, FP8>(a, src, page, kk, sdc, true);
      }
      if (vis_wave) {
        const int kk = kb + (lane & 31);
        sg.meta = d.slot_meta[kk < src.L ? (static_cast<int64_t>(page) << g.Pshift) + (kk & (g.P - 1)) : 0];
      }
    };
    auto stage_write = [&](uint8_t* b, int blk, const Stage& sg) {
      if (tid < S::STHREADS) {
        *reinterpret_cast<uint4*>(b + S::off(skey, sdc)) = pf_bf16<FP8>(sg.k);
        *reinterpret_cast<uint4*>(b + S::V_OFF + S::off(skey, sdc)) = pf_bf16<FP8>(sg.v);
      }
      vis_write(blk, b, sg.meta);
    };
    stage_load(0, st0);
    stage_write(sbuf0, 0, st0);
    stage_load(1, st1);
    __syncthreads();
    for (int blk = 0; blk < nblk; blk += 2) {
      stage_load(blk + 2, st0);
      compute(sbuf0);
      stage_write(sbuf1, blk + 1, st1);
      __syncthreads();
      if (blk + 1 >= nblk) break;
      stage_load(blk + 3, st1);
      compute(sbuf1);
      stage_write(sbuf0, blk + 2, st0);
      __syncthreads();
    }
  }

  // ---- normalise and store: lane holds d = 16 dt + 4 G4 + r of its column
  uint16_t* obase = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int tg = 0; tg < S::TG; ++tg) {
    if (!qok[tg]) continue;
    const int t = wtok + tg * 16 + l16;
#pragma unroll
    for (int h = 0; h < S::HW; ++h) {
      const int c = tg * S::HW + h;
      const float inv = 1.0f / lacc[c][0];
      if (TRAIN && G4 == 0)   // natural log of sum_j exp(scaled score_j)
        a.lse[(static_cast<size_t>(row) * g.Hq + head0 + h) * a.C + t] = (mb[c] + __log2f(lacc[c][0])) * 0.6931471805599453f;
      uint16_t* orow = obase + ((static_cast<size_t>(row) * a.C + t) * g.Hq + head0 + h) * D + 4 * G4;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) {
        const pf_f32x4 v = o[c][dt];
        *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(pf_pack(v[0] * inv, v[1] * inv), pf_pack(v[2] * inv, v[3] * inv));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined matrix-core kernel (bf16 pages and the training forward).
//
// Same workgroup shape, operand layouts and LDS row swizzle as the kernel
// above; the work per key block is reordered so that both the matrix cores
// and the vector ALU stay busy inside every wave:
//  * K and V of a block live in separate LDS rings of four buffers.  Step j
//    issues the direct global->LDS loads of K for block j+4 and V for block
//    j+3, and waits only for the loads issued two steps earlier, so every
//    load has two steps to land.
//  * Step j computes S of block j+1 (K from LDS) while the same wave turns
//    the scores of block j into probabilities (exp2), then P.V of block j
//    while it takes the maxima of block j+1; the running maximum is raised
//    after P.V (lazily, as above).
//  * Visibility enters the score product as its accumulator's initial value:
//    0 for a visible key, -inf for a hidden one (training: the key's
//    penalty once the query is w or more positions past it).  A block whose
//    keys are all visible to every query of the workgroup (the common case
//    for cached keys) starts from 0 without any per-key test; the lane that
//    stages the block's intervals decides that with one ballot.
// The ring buffers are separate arrays and the block loop is unrolled by
// four, so each step's buffers are static and the compiler can tell that
// the loads in flight do not alias the LDS reads of the step.
constexpr int kPpRing = 4;

template <int D, int G, bool TRAIN>
struct PpShape {
  using S = PfShape<D, G, false>;
  static constexpr int KROWS = kPfKB * S::ROW;
  static constexpr int META = KROWS;            // 32 ints: slot metadata (cache keys)
  static constexpr int LO = META + 4 * kPfKB;   // 32 ints
  static constexpr int HI = LO + 4 * kPfKB;     // 32 ints
  static constexpr int PEN = HI + 4 * kPfKB;    // 32 floats (training: gate logit, then penalty / scale)
  static constexpr int FLAG = PEN + 4 * kPfKB;  // 1 int: 1 every key visible to the whole block of queries,
                                                //        2 (training) every key penalised for all of them
  static constexpr int KBUF = FLAG + 16;
  static constexpr int VBUF = KROWS;
};

template <int D, int G, bool TRAIN>
__global__ __launch_bounds__(kPfThreads) void prefill_attn_pipe_kernel(PrefillArgs a) {
  using S = PfShape<D, G, false>;
  using P = PpShape<D, G, TRAIN>;
  constexpr int TG = S::TG, NT = S::NT, HW = S::HW, KS = S::KS, DT = S::DT;
  __shared__ __attribute__((aligned(16))) uint8_t kb0[P::KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t kb1[P::KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t kb2[P::KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t kb3[P::KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t vb0[P::VBUF];
  __shared__ __attribute__((aligned(16))) uint8_t vb1[P::VBUF];
  __shared__ __attribute__((aligned(16))) uint8_t vb2[P::VBUF];
  __shared__ __attribute__((aligned(16))) uint8_t vb3[P::VBUF];
  __shared__ int s_pt[TRAIN ? 1 : kPfMaxPages];
  __shared__ uint8_t s_ev[TRAIN ? 1 : kMaxChunk];
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, G4 = lane >> 4;

  // workgroup -> (pair, token block): heaviest token blocks first
  const int npairs = a.B * g.Hkv;
  const int ntb = (a.C + S::TOKB - 1) / S::TOKB;
  const int pair = blockIdx.x % npairs;
  const int tb = ntb - 1 - static_cast<int>(blockIdx.x) / npairs;
  const int row = pair / g.Hkv, kh = pair % g.Hkv;
  const int seq = (a.seq_ids && !TRAIN) ? a.seq_ids[row] : row;
  if (!TRAIN && (seq < 0 || seq >= g.Bmax)) {
    if (tid == 0 && tb == 0 && kh == 0) set_status(d.ctl, DMS_DEV_BAD_SEQ);
    return;
  }
  const int unit = seq * g.Hkv + kh;
  const int L = TRAIN ? 0 : d.lengths[unit];
  const int s0 = TRAIN ? 0 : d.pos[seq];
  const int tok0 = tb * S::TOKB;
  const int tok_end = min(tok0 + S::TOKB, a.C);
  const int nk = L + tok_end;
  const int nblk = (nk + kPfKB - 1) / kPfKB;
  const int64_t stride = static_cast<int64_t>(g.Hkv) * D * 2;   // bytes between chunk keys
  const size_t chunk0 = (static_cast<size_t>(row) * a.C * g.Hkv + kh) * D * 2;
  const uint8_t* kchunk = static_cast<const uint8_t*>(a.k) + chunk0;
  const uint8_t* vchunk = static_cast<const uint8_t*>(a.v) + chunk0;
  const float* gate = TRAIN ? a.gate + static_cast<int64_t>(pair) * a.C : nullptr;
  // query positions of the whole workgroup (the all-visible test)
  const int qlo_wg = s0 + tok0, qhi_wg = s0 + tok_end - 1;

  // ---- this wave's query columns
  const int hp = wave % S::HS, tp = wave / S::HS;
  const int wtok = tok0 + tp * S::TOKW;
  const int head0 = kh * G + hp * HW;
  int qpos[TG];
  bool qok[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int t = wtok + tg * 16 + l16;
    qok[tg] = t < a.C;
    qpos[tg] = qok[tg] ? s0 + t : -1;
  }
  pf_bf16x8 qf[NT][KS];
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const int c = tg * HW + h;
      const int t = wtok + tg * 16 + l16;
      const size_t qrow = ((static_cast<size_t>(row) * a.C + t) * g.Hq + head0 + h) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (qok[tg]) w = *reinterpret_cast<const uint4*>(qbase + qrow + 32 * ks + 8 * G4);
        qf[c][ks] = __builtin_bit_cast(pf_bf16x8, w);
      }
    }
  }

  pf_f32x4 o[NT][DT], lacc[NT];
  float m[NT], mb[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    m[c] = -INFINITY;
    mb[c] = 0.0f;
    lacc[c] = pf_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[c][dt] = pf_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float cs = g.scale_log2;
  const pf_bf16x8 ones = __builtin_bit_cast(pf_bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

  if constexpr (!TRAIN) {
    const int npages = (L + g.P - 1) >> g.Pshift;   // <= kPfMaxPages (checked at launch)
    const int32_t* pt = d.page_table + static_cast<int64_t>(unit) * g.maxp;
    const uint8_t* ev = a.evict + static_cast<int64_t>(pair) * a.C;
    for (int i = tid; i < npages; i += kPfThreads) s_pt[i] = pt[i];
    for (int i = tid; i < tok_end; i += kPfThreads) s_ev[i] = ev[i];
  }
  __syncthreads();

  // ---- direct global->LDS loads of one tensor (K or V) of one key block.
  // D = 128: every wave loads 4 rows of K and 4 rows of V; D = 64: waves
  // 0-3 load K (8 rows each), waves 4-7 V.  Lane i writes bytes
  // [16 i, 16 i + 16) of the wave's 1 KB stretch: row rl, the chunk that the
  // row's swizzle places there.  Rows past the keys read the last key's row.
  constexpr int RPW = 1024 / S::ROW;
  constexpr int RB = 2 * D;
  const int rl = (D == 128 ? wave : (wave & 3)) * RPW + lane / S::CPR;
  const int cl = (lane % S::CPR) ^ S::swz(rl);
  const int loff = (D == 128 ? wave : (wave & 3)) * 1024;
  const uint32_t off_page = static_cast<uint32_t>(rl * RB + 16 * cl);
  const uint32_t off_chunk = static_cast<uint32_t>(rl * stride + 16 * cl);
  const bool vis_wave = wave == kPfWaves - 1;
  auto block_page = [&](int kb) { return (!TRAIN && kb < L) ? s_pt[kb >> g.Pshift] : 0; };
  auto dma_rows = [&](int blk, bool v, uint8_t* buf) {
    const int kb = blk * kPfKB;
    const uint8_t* pages = v ? d.v_pages : d.k_pages;
    const uint8_t* chunk = v ? vchunk : kchunk;
    const uint8_t* src;
    if (!TRAIN && kb + kPfKB <= L) {
      const uint8_t* base = pages + ((static_cast<int64_t>(block_page(kb)) << g.Pshift) + (kb & (g.P - 1))) * RB;
      src = base + off_page;
    } else if (kb >= L && kb + kPfKB <= nk) {
      src = chunk + static_cast<int64_t>(kb - L) * stride + off_chunk;
    } else {
      const int kc = min(kb + rl, nk - 1);
      if (!TRAIN && kc < L)
        src = pages + ((static_cast<int64_t>(block_page(kb)) << g.Pshift) + (kc & (g.P - 1))) * RB + 16 * cl;
      else
        src = chunk + static_cast<int64_t>(kc - L) * stride + 16 * cl;
    }
    __builtin_amdgcn_global_load_lds((const pf_glb_void*)src, (pf_lds_void*)(buf + loff), 16, 0, 0);
  };
  // the staging wave's extra load per block: slot metadata (cache keys) or
  // the gate logits (training); one load per block in either case, so every
  // wave issues a fixed number of loads per step
  auto dma_meta = [&](int blk, uint8_t* kbuf) {
    if (vis_wave && lane < kPfKB) {
      const int kb = blk * kPfKB;
      if constexpr (TRAIN) {
        __builtin_amdgcn_global_load_lds((const pf_glb_void*)(gate + min(kb + lane, nk - 1)),
                                         (pf_lds_void*)(kbuf + P::PEN), 4, 0, 0);
      } else {
        const int kc = min(kb + lane, L - 1);
        const int64_t mi = kb < L ? (static_cast<int64_t>(block_page(kb)) << g.Pshift) + (kc & (g.P - 1)) : 0;
        __builtin_amdgcn_global_load_lds((const pf_glb_void*)(d.slot_meta + mi), (pf_lds_void*)(kbuf + P::META), 4,
                                         0, 0);
      }
    }
  };
  auto issue_k = [&](int blk, uint8_t* kbuf) {
    if (D == 128 || wave < 4) dma_rows(blk, false, kbuf);
    dma_meta(blk, kbuf);
  };
  auto issue_v = [&](int blk, uint8_t* vbuf) {
    if (D == 128 || wave >= 4) dma_rows(blk, true, vbuf);
  };
  // loads one step issues per wave
  constexpr int LD_STEP = D == 128 ? 2 : 1;
  auto wait_two_steps_back = [&]() {
    // the loads of the two latest steps may stay in flight
    if (vis_wave) {
      if constexpr (D == 128) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      if constexpr (D == 128) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    }
  };
  static_assert(LD_STEP == (D == 128 ? 2 : 1), "load count");

  // A workgroup barrier that orders LDS only: __syncthreads() would also
  // wait for every global->LDS load in flight (its fence covers global
  // memory), which the ring leaves in flight on purpose; the loads a step
  // needs are waited for explicitly (wait_two_steps_back) before it.
  auto lds_barrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // ---- visibility intervals [lo, hi) of a landed block's keys and the
  // block flag (staging wave, lanes 0..31)
  auto vis_write = [&](int blk, uint8_t* kbuf) {
    if (vis_wave) {
      const int kk = blk * kPfKB + (lane & 31);
      int lo, hi;
      if constexpr (TRAIN) {
        float* pen = reinterpret_cast<float*>(kbuf + P::PEN);
        float pv = 0.0f;
        if (kk < nk) {
          lo = kk;
          hi = kk + g.w;
          const float y = lane < kPfKB ? pen[lane] : 0.0f;
          // logsigmoid(-y) = -softplus(y), stable for either sign
          const float ls = -(fmaxf(y, 0.0f) + log1pf(__expf(-fabsf(y))));
          pv = ls * (1.4426950408889634f / g.scale_log2);
        } else {
          lo = kPfNoLimit;
          hi = 0;
        }
        if (lane < kPfKB) pen[lane] = pv;
      } else {
        const int meta = lane < kPfKB ? reinterpret_cast<const int*>(kbuf + P::META)[lane] : 0;
        if (kk < L) {
          lo = meta & 0x7FFFFFFF;
          hi = meta < 0 ? lo + g.w : kPfNoLimit;
        } else if (kk < nk) {
          lo = s0 + (kk - L);
          hi = s_ev[kk - L] ? lo + g.w : kPfNoLimit;
        } else {
          lo = kPfNoLimit;
          hi = 0;
        }
      }
      const uint64_t half = 0xFFFFFFFFull;
      const bool all_vis = lo <= qlo_wg && hi > qhi_wg;
      const bool all_pen = TRAIN && lo <= qlo_wg && hi <= qlo_wg;
      const uint64_t bv = __builtin_amdgcn_ballot_w64(all_vis) & half;
      const uint64_t bp = __builtin_amdgcn_ballot_w64(all_pen) & half;
      if (lane < kPfKB) {
        reinterpret_cast<int*>(kbuf + P::LO)[lane] = lo;
        reinterpret_cast<int*>(kbuf + P::HI)[lane] = hi;
      }
      if (lane == 0) *reinterpret_cast<int*>(kbuf + P::FLAG) = bv == half ? 1 : (bp == half ? 2 : 0);
    }
  };

  // ---- the score accumulators' initial values for a block: lane (G4, l16)
  // holds keys 4 G4 + i (kt 0) and 16 + 4 G4 + i (kt 1)
  auto bias_of = [&](const uint8_t* kbuf, pf_f32x4 (&bias)[TG][2]) {
    const int flag = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(kbuf + P::FLAG));
    if (flag == 1) {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) bias[tg][0] = bias[tg][1] = pf_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      return;
    }
    pf_f32x4 pen[2] = {pf_f32x4{0.0f, 0.0f, 0.0f, 0.0f}, pf_f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
    if constexpr (TRAIN) {
      pen[0] = *reinterpret_cast<const pf_f32x4*>(kbuf + P::PEN + 16 * G4);
      pen[1] = *reinterpret_cast<const pf_f32x4*>(kbuf + P::PEN + 64 + 16 * G4);
      if (flag == 2) {
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          bias[tg][0] = pen[0];
          bias[tg][1] = pen[1];
        }
        return;
      }
    }
    const int4 lo0 = *reinterpret_cast<const int4*>(kbuf + P::LO + 16 * G4);
    const int4 lo1 = *reinterpret_cast<const int4*>(kbuf + P::LO + 64 + 16 * G4);
    const int4 hi0 = *reinterpret_cast<const int4*>(kbuf + P::HI + 16 * G4);
    const int4 hi1 = *reinterpret_cast<const int4*>(kbuf + P::HI + 64 + 16 * G4);
    const int los[8] = {lo0.x, lo0.y, lo0.z, lo0.w, lo1.x, lo1.y, lo1.z, lo1.w};
    const int his[8] = {hi0.x, hi0.y, hi0.z, hi0.w, hi1.x, hi1.y, hi1.z, hi1.w};
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int qp = qpos[tg];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float b;
        if constexpr (TRAIN) b = los[e] <= qp ? (qp >= his[e] ? pen[e >> 2][e & 3] : 0.0f) : -INFINITY;
        else b = (los[e] <= qp && qp < his[e]) ? 0.0f : -INFINITY;
        bias[tg][e >> 2][e & 3] = b;
      }
    }
  };

  // S^T = K Q^T of one block from its bias
  auto scores = [&](const uint8_t* kbuf, const pf_f32x4 (&bias)[TG][2], pf_f32x4 (&s)[2][NT]) {
    pf_bf16x8 kf[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        kf[ks][kt] = *reinterpret_cast<const pf_bf16x8*>(kbuf + S::off(16 * kt + l16, 4 * ks + G4));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c = 0; c < NT; ++c)
          s[kt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][kt], qf[c][ks], ks == 0 ? bias[c / HW][kt] : s[kt][c],
                                                             0, 0, 0);
  };
  // block maxima; true where the running maximum must be raised
  auto maxima = [&](const pf_f32x4 (&s)[2][NT], float (&mx)[NT]) {
    bool need = false;
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      float x = fmaxf(fmaxf(fmaxf(s[0][c][0], s[0][c][1]), fmaxf(s[0][c][2], s[0][c][3])),
                      fmaxf(fmaxf(s[1][c][0], s[1][c][1]), fmaxf(s[1][c][2], s[1][c][3])));
      x = pf_max_x32(x);
      x = pf_max_x16(x);
      mx[c] = x;
      need |= x * cs > m[c] * cs + kPfRescaleLog2;
    }
    return need;
  };
  auto raise = [&](const float (&mx)[NT]) {
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      if (mx[c] * cs > m[c] * cs + kPfRescaleLog2) {
        const float alpha = __builtin_amdgcn_exp2f((m[c] - mx[c]) * cs);   // 0 from -inf
        m[c] = mx[c];
        mb[c] = mx[c] * cs;
        lacc[c] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[c][dt] *= alpha;
      }
    }
  };
  // probabilities of a block (bf16, the second product's operand) and the
  // denominator
  auto probs = [&](const pf_f32x4 (&s)[2][NT], pf_bf16x8 (&pk)[NT]) {
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(s[e >> 2][c][e & 3], cs, -mb[c]));
      const uint4 w = make_uint4(pf_pack(p[0], p[1]), pf_pack(p[2], p[3]), pf_pack(p[4], p[5]), pf_pack(p[6], p[7]));
      pk[c] = __builtin_bit_cast(pf_bf16x8, w);
      lacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pk[c], lacc[c], 0, 0, 0);
    }
  };
  // O^T += V^T P^T of a block
  auto pv = [&](const uint8_t* vbuf, const pf_bf16x8 (&pk)[NT]) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int r0 = 4 * G4 + (l16 >> 2), ch = 2 * dt + ((l16 & 3) >> 1), half = 8 * (l16 & 1);
      const pf_i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pf_lds_i16x4*)(vbuf + S::off(r0, ch) + half));
      const pf_i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pf_lds_i16x4*)(vbuf + S::off(r0 + 16, ch) + half));
      const pf_bf16x8 vf = __builtin_bit_cast(pf_bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int c = 0; c < NT; ++c) o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pk[c], o[c][dt], 0, 0, 0);
    }
  };

  // ---- prologue: K 0, K 1, V 0 landed with their intervals, S of block 0
  // and its maxima; then the loads of the two steps before step 0
  issue_k(0, kb0);
  issue_v(0, vb0);
  issue_k(1, kb1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  vis_write(0, kb0);
  vis_write(1, kb1);
  __syncthreads();
  issue_k(2, kb2);
  issue_v(1, vb1);
  issue_k(3, kb3);
  issue_v(2, vb2);
  pf_f32x4 sa[2][NT], sb[2][NT];
  {
    pf_f32x4 bias[TG][2];
    bias_of(kb0, bias);
    scores(kb0, bias, sa);
    float mx[NT];
    if (__any(maxima(sa, mx))) raise(mx);
  }
  __syncthreads();   // kb0 is step 0's load target

  // step j: loads of K j+4 into K j's buffer and V j+3 into V j-1's; S of
  // block j+1 beside the probabilities of block j; P.V of block j beside the
  // maxima of block j+1; the running maximum; then the loads of two steps
  // back, block j+2's intervals, and the barrier
  auto step = [&](int j, uint8_t* ku, uint8_t* kd, uint8_t* kl, uint8_t* vu, uint8_t* vd, pf_f32x4 (&sc)[2][NT],
                  pf_f32x4 (&sn)[2][NT]) {
    issue_k(j + 4, kd);
    issue_v(j + 3, vd);
    pf_f32x4 bias[TG][2];
    bias_of(ku, bias);
    pf_bf16x8 pk[NT];
    float mx[NT];
    scores(ku, bias, sn);
    probs(sc, pk);
    pv(vu, pk);
    const bool need = maxima(sn, mx);
    // the K fragment reads, the score products (each beside exp2 /
    // conversion work), the V fragment reads (into the K fragments'
    // registers), the denominators, then P.V beside the maxima
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS * NT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
#pragma unroll
    for (int i = 0; i < 2 * DT; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NT + DT * NT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (__any(need)) raise(mx);
    wait_two_steps_back();
    vis_write(j + 2, kl);
    lds_barrier();
  };
  for (int j = 0; j < nblk; j += 4) {
    step(j, kb1, kb0, kb2, vb0, vb3, sa, sb);
    if (j + 1 >= nblk) break;
    step(j + 1, kb2, kb1, kb3, vb1, vb0, sb, sa);
    if (j + 2 >= nblk) break;
    step(j + 2, kb3, kb2, kb0, vb2, vb1, sa, sb);
    if (j + 3 >= nblk) break;
    step(j + 3, kb0, kb3, kb1, vb3, vb2, sb, sa);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load outlives the workgroup

  // ---- normalise and store
  uint16_t* obase = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    if (!qok[tg]) continue;
    const int t = wtok + tg * 16 + l16;
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const int c = tg * HW + h;
      const float inv = 1.0f / lacc[c][0];
      if (TRAIN && G4 == 0)
        a.lse[(static_cast<size_t>(row) * g.Hq + head0 + h) * a.C + t] = (mb[c] + __log2f(lacc[c][0])) * 0.6931471805599453f;
      uint16_t* orow = obase + ((static_cast<size_t>(row) * a.C + t) * g.Hq + head0 + h) * D + 4 * G4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const pf_f32x4 v = o[c][dt];
        *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(pf_pack(v[0] * inv, v[1] * inv), pf_pack(v[2] * inv, v[3] * inv));
      }
    }
  }
}

// DMS_PREFILL_PIPE=0 keeps bf16 pages and the training forward on the
// kernel without the software pipeline.
static bool pf_pipe_enabled() {
  const char* e = std::getenv("DMS_PREFILL_PIPE");
  return !e || std::atoi(e) != 0;
}

template <int D, int G, bool FP8>
static int launch_mfma_dgf(const PrefillArgs& a, hipStream_t st) {
  using S = PfShape<D, G, FP8>;
  const int ntb = (a.C + S::TOKB - 1) / S::TOKB;
  const dim3 grid(ntb * a.B * a.g.Hkv), block(kPfThreads);
  if (!FP8 && pf_pipe_enabled())
    hipLaunchKernelGGL((prefill_attn_pipe_kernel<D, G, false>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((prefill_attn_mfma_kernel<D, G, FP8>), grid, block, 0, st, a);
  return DMS_OK;
}

template <int D, bool FP8>
static int launch_mfma_d(const PrefillArgs& a, hipStream_t st) {
  switch (a.g.g) {
    case 1: return launch_mfma_dgf<D, 1, FP8>(a, st);
    case 2: return launch_mfma_dgf<D, 2, FP8>(a, st);
    case 4: return launch_mfma_dgf<D, 4, FP8>(a, st);
    default: return fail(DMS_ERR_UNSUPPORTED, "group size");
  }
}

static bool mfma_ok(const Geo& g) {
  return (g.kv_dtype == DMS_BF16 || g.kv_dtype == DMS_FP8_E4M3) && (g.D == 64 || g.D == 128) &&
         (g.g == 1 || g.g == 2 || g.g == 4) && g.Pshift >= 5 && g.maxp <= kPfMaxPages;
}

static int launch_mfma(const PrefillArgs& a, hipStream_t st) {
  const bool fp8 = a.g.kv_dtype == DMS_FP8_E4M3;
  if (a.g.D == 128) return fp8 ? launch_mfma_d<128, true>(a, st) : launch_mfma_d<128, false>(a, st);
  return fp8 ? launch_mfma_d<64, true>(a, st) : launch_mfma_d<64, false>(a, st);
}

template <int D, int G>
static void launch_train_dg(const PrefillArgs& a, hipStream_t st) {
  using S = PfShape<D, G, false>;
  const int ntb = (a.C + S::TOKB - 1) / S::TOKB;
  if (pf_pipe_enabled())
    hipLaunchKernelGGL((prefill_attn_pipe_kernel<D, G, true>), dim3(ntb * a.B * a.g.Hkv), dim3(kPfThreads), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_attn_mfma_kernel<D, G, false, true>), dim3(ntb * a.B * a.g.Hkv), dim3(kPfThreads), 0,
                       st, a);
}

template <int D>
static int launch_train_d(const PrefillArgs& a, hipStream_t st) {
  switch (a.g.g) {
    case 1: launch_train_dg<D, 1>(a, st); return DMS_OK;
    case 2: launch_train_dg<D, 2>(a, st); return DMS_OK;
    case 4: launch_train_dg<D, 4>(a, st); return DMS_OK;
    default: return fail(DMS_ERR_UNSUPPORTED, "group size (1, 2 or 4)");
  }
}

}  // namespace dms

using namespace dms;

extern "C" int dms_train_attn_fwd(int B, int T, int num_q_heads, int num_kv_heads, int head_dim, int window,
                                  float softmax_scale, const void* q, const void* k, const void* v,
                                  const float* gate_logits, void* out, float* lse, void* stream) {
  if (!q || !k || !v || !gate_logits || !out || !lse) return fail(DMS_ERR_ARG, "q, k, v, gate_logits, out and lse are required");
  if (B <= 0 || T <= 0) return fail(DMS_ERR_ARG, "B and T must be positive");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(DMS_ERR_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (head_dim != 64 && head_dim != 128) return fail(DMS_ERR_UNSUPPORTED, "head_dim (64 or 128)");
  if (window <= 0) return fail(DMS_ERR_ARG, "window must be positive");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
       reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(gate_logits)) % 16 != 0)
    return fail(DMS_ERR_ARG, "q, k, v, out and gate_logits must be 16-byte aligned");
  Geo g{};
  g.Bmax = B;
  g.Hq = num_q_heads;
  g.Hkv = num_kv_heads;
  g.D = head_dim;
  g.g = num_q_heads / num_kv_heads;
  g.w = window;
  g.kv_dtype = DMS_BF16;
  g.Pshift = -1;
  const float sc = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  g.scale_log2 = sc * 1.4426950408889634f;
  PrefillArgs a{};
  a.g = g;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.B = B;
  a.C = T;
  a.gate = gate_logits;
  a.lse = lse;
  hipStream_t st = as_stream(stream);
  const int s = head_dim == 128 ? launch_train_d<128>(a, st) : launch_train_d<64>(a, st);
  if (s) return s;
  return check_hip(hipGetLastError(), "dms_train_attn_fwd launch");
}

extern "C" int dms_prefill_attn(dms_cache* cache, const int32_t* seq_ids, const void* q, const void* k,
                                const void* v, const uint8_t* evict, void* out, int B, int C, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  if (!q || !k || !v || !evict || !out) return fail(DMS_ERR_ARG, "q, k, v, evict and out are required");
  const Geo& g = cache->geo;
  if (B <= 0 || C <= 0) return fail(DMS_ERR_ARG, "B and C must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  if (C > g.max_chunk) return fail(DMS_ERR_CAPACITY, "C above max_chunk");
  PrefillArgs a{cache->dev, g, seq_ids, q, k, v, evict, out, B, C, nullptr, nullptr};
  hipStream_t st = as_stream(stream);
  int s;
  if (mfma_ok(g) && !cache->force_generic) {
    s = launch_mfma(a, st);
  } else {
    switch (g.kv_dtype) {
      case DMS_F32: s = launch_generic<float, DMS_F32>(a, st); break;
      case DMS_BF16: s = launch_generic<uint16_t, DMS_BF16>(a, st); break;
      case DMS_FP8_E4M3: s = launch_generic<uint16_t, DMS_FP8_E4M3>(a, st); break;
      default: return fail(DMS_ERR_UNSUPPORTED, "kv dtype");
    }
  }
  if (s) return s;
  return check_hip(hipGetLastError(), "dms_prefill_attn launch");
}
