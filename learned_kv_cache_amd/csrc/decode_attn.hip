// dms_decode_attn: GQA decode attention over the ragged per-head paged cache.
//
// "基于 DMS 的 KV Cache 压缩实战" walkthrough, 推理模式: inference attention runs
// over the paged per-head cache whose per-head lengths differ.  After the
// current token is appended, the live slots of a head are exactly the keys the
// token may see (delayed eviction overwrote every key that left the window
// marked), so the kernel needs no mask.  The FastDMS post (subsystem table)
// replaces attention scoring with split-K grouped decode attention over
// variable-length per-head live spans; this is that idea laid out for CDNA4:
//
// * Work balance: with few (row, KV head) units each unit gets whole
//   workgroups in proportion to its live slots (no workgroup spans two
//   units); with many, the concatenated live slots are cut into one
//   contiguous range per workgroup and a range spanning a unit boundary
//   emits one partial per unit.  Either way every workgroup streams about the
//   same number of bytes however ragged the heads are.
// * One workgroup serves all g query heads of a KV head, so K/V are read once.
// * Each lane loads 16 contiguous bytes of a K row and of a V row; LPR lanes
//   cover one row, a wave covers 64/LPR rows per pass, NP passes per chunk,
//   chunks double-buffered.
// * Online softmax per wave in base 2; waves merge through LDS; the last
//   workgroup of a split unit merges the unit's partial records.
#include <algorithm>
#include <cstdlib>
#include <mutex>

#include <memory>
#include <vector>
#include "dms_internal.h"
#include "decode_prep.h"

namespace dms {

struct DecodeArgs {
  DevCache d;
  Geo g;
  const int32_t* seq_ids;
  const void* q;
  void* out;
  int B;
  int lanes_per_row;   // fast kernel row layout (8 or 16 lanes per bf16 row of 128)
  float* partials;     // caller's workspace: partial (o, m, l) records of split units
  int mfma;            // bf16 pages: the matrix-core variant of the fast kernel
};

template <int KV> struct KvTraits;
template <> struct KvTraits<DMS_F32> { static constexpr int bytes = 4; };
template <> struct KvTraits<DMS_BF16> { static constexpr int bytes = 2; };
template <> struct KvTraits<DMS_FP8_E4M3> { static constexpr int bytes = 1; };

// 16 bytes of a row -> EPL floats.
template <int KV>
__device__ __forceinline__ void unpack16(const uint4& raw, float* f) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  if (KV == DMS_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else if (KV == DMS_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) f[4 * i + j] = e4m3_to_f32((w[i] >> (8 * j)) & 0xFFu);
    }
  }
}

// Block-wide (256 threads) exclusive scan; returns this thread's exclusive
// prefix and writes the block total to *total.
__device__ __forceinline__ int block_scan_256(int x, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < wave) off += s_tmp[i];
    tot += s_tmp[i];
  }
  __syncthreads();
  *total = tot;
  return off + incl - x;
}

// Unit prefix tables shared by the attention and combine kernels:
// s_start[u] = first concatenated slot of unit u (s_start[units] = W);
// s_pbase[u] = first partial record of unit u; c = slots per workgroup.
struct UnitTables {
  int W;
  int c;
};

template <int ROWS_WG>
__device__ UnitTables build_unit_tables(const DecodeArgs& a, int* s_start, int* s_pbase, int* s_tmp, int grid) {
  const Geo& g = a.g;
  const int units = a.B * g.Hkv;
  const int per = (units + 255) / 256;           // units per thread (contiguous)
  const int u0 = threadIdx.x * per;
  int len[8];
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int u = u0 + i;
    int L = 0;
    if (u < units) {
      const int row = u / g.Hkv, kh = u % g.Hkv;
      const int seq = a.seq_ids ? a.seq_ids[row] : row;
      if (seq >= 0 && seq < g.Bmax) L = a.d.lengths[seq * g.Hkv + kh];
      else if (blockIdx.x == 0 && kh == 0) set_status(a.d.ctl, DMS_DEV_BAD_SEQ);
    }
    len[i] = L;
    sum += L;
  }
  int W;
  int run = block_scan_256(sum, s_tmp, &W);
  for (int i = 0; i < per; ++i) {
    const int u = u0 + i;
    if (u < units) s_start[u] = run;
    run += len[i];
  }
  if (threadIdx.x == 0) s_start[units] = W;
  const int c = max((W + grid - 1) / grid, ROWS_WG);
  __syncthreads();
  int nsum = 0;
  int nu[8];
  for (int i = 0; i < per; ++i) {
    const int u = u0 + i;
    int n = 0;
    if (u < units && len[i] > 0) n = (s_start[u] + len[i] - 1) / c - s_start[u] / c + 1;
    nu[i] = n;
    nsum += n;
  }
  int tot;
  int pr = block_scan_256(nsum, s_tmp, &tot);
  for (int i = 0; i < per; ++i) {
    const int u = u0 + i;
    if (u < units) {
      s_pbase[u] = pr;
      if (blockIdx.x == 0) {
        a.d.unit_info[4 * u] = pr;
        a.d.unit_info[4 * u + 1] = nu[i];
      }
    }
    pr += nu[i];
  }
  __syncthreads();
  return UnitTables{W, c};
}

template <typename ACT, int KV, int D, int G, int NP>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeArgs a) {
  constexpr int KB = KvTraits<KV>::bytes;
  constexpr int EPL = 16 / KB;                 // elements per lane per row
  constexpr int LPR = D / EPL;                 // lanes per row
  constexpr int RPW = 64 / LPR;                // rows per wave per pass
  constexpr int ROWS_WAVE = RPW * NP;
  constexpr int ROWS_WG = 4 * ROWS_WAVE;
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row must map onto a wave");

  __shared__ int s_start[kMaxUnits + 1];
  __shared__ int s_pbase[kMaxUnits];
  __shared__ int s_tmp[4];
  __shared__ float s_o[4][G][D];
  __shared__ float s_m[4][G], s_l[4][G];

  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lane_row = lane / LPR, lane_col = lane % LPR;
  const int units = a.B * g.Hkv;
  const UnitTables tb = build_unit_tables<ROWS_WG>(a, s_start, s_pbase, s_tmp, gridDim.x);
  const int c = tb.c;
  int a0 = blockIdx.x * c;
  const int a1 = min(a0 + c, tb.W);
  if (a0 >= a1) return;
  // unit holding slot a0: the last u with s_start[u] <= a0 (empty units share starts)
  int lo_u = 0, hi_u = units - 1;
  while (lo_u < hi_u) {
    const int mid = (lo_u + hi_u + 1) >> 1;
    if (s_start[mid] <= a0) lo_u = mid; else hi_u = mid - 1;
  }
  int u = lo_u;
  const ACT* qbase = static_cast<const ACT*>(a.q);
  ACT* obase = static_cast<ACT*>(a.out);

  while (a0 < a1) {
    const int ustart = s_start[u];
    const int seg_end = min(a1, s_start[u + 1]);
    const int lo = a0 - ustart, hi = seg_end - ustart;
    const int row = u / g.Hkv, kh = u % g.Hkv;
    const int seq = a.seq_ids ? a.seq_ids[row] : row;
    const int32_t* pt = d.page_table + (static_cast<int64_t>(seq) * g.Hkv + kh) * g.maxp;

    float qf[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        qf[h][e] = load_act<ACT>(qbase, (static_cast<size_t>(row) * g.Hq + kh * G + h) * D + lane_col * EPL + e) *
                   g.scale_log2;
    }
    float m[G], l[G], o[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
    }

    for (int sb = lo; sb < hi; sb += ROWS_WG) {
      const int base = sb + wave * ROWS_WAVE;
      uint4 kr[NP], vr[NP];
      float sk[NP], sv[NP];
      bool ok[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int r = base + p * RPW + lane_row;
        ok[p] = r < hi;
        sk[p] = 1.0f;
        sv[p] = 1.0f;
        if (ok[p]) {
          const int page = pt[r / g.P];
          const int64_t roff = static_cast<int64_t>(page) * g.P + r % g.P;
          kr[p] = *reinterpret_cast<const uint4*>(d.k_pages + (roff * D + lane_col * EPL) * KB);
          vr[p] = *reinterpret_cast<const uint4*>(d.v_pages + (roff * D + lane_col * EPL) * KB);
          if (KV == DMS_FP8_E4M3) {
            sk[p] = d.scales[2 * page];
            sv[p] = d.scales[2 * page + 1];
          }
        } else {
          kr[p] = make_uint4(0, 0, 0, 0);
          vr[p] = make_uint4(0, 0, 0, 0);
        }
      }
      float s[NP][G];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        float kf[EPL];
        unpack16<KV>(kr[p], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float acc = 0.0f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc = fmaf(qf[h][e], kf[e], acc);
#pragma unroll
          for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
          s[p][h] = ok[p] ? acc * sk[p] : -INFINITY;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = s[0][h];
#pragma unroll
        for (int p = 1; p < NP; ++p) mx = fmaxf(mx, s[p][h]);
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const float m_new = fmaxf(m[h], mx);
        if (m_new == -INFINITY) continue;            // no live row seen yet (wave-uniform)
        const float alpha = exp2f(m[h] - m_new);     // m[h] = -inf gives 0
        m[h] = m_new;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const float pe = ok[p] ? exp2f(s[p][h] - m_new) : 0.0f;
          l[h] += pe;
          float vf[EPL];
          unpack16<KV>(vr[p], vf);
          const float w = pe * sv[p];
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(w, vf[e], o[h][e]);
        }
      }
    }
    // merge row groups inside the wave, then the four waves through LDS
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) {
        l[h] += __shfl_xor(l[h], off);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] += __shfl_xor(o[h][e], off);
      }
    }
    if (lane_row == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_o[wave][h][lane_col * EPL + e] = o[h][e];
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
    __syncthreads();
    const int n_u = (s_start[u] + (s_start[u + 1] - s_start[u]) - 1) / c - s_start[u] / c + 1;
    for (int idx = tid; idx < G * D; idx += 256) {
      const int h = idx / D, dd = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
      float ov = 0.0f, lv = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (s_m[w][h] == -INFINITY) continue;
          const float f = exp2f(s_m[w][h] - M);
          ov += f * s_o[w][h][dd];
          lv += f * s_l[w][h];
        }
      }
      if (n_u == 1) {
        store_act<ACT>(obase, (static_cast<size_t>(row) * g.Hq + kh * G + h) * D + dd, lv > 0.0f ? ov / lv : 0.0f);
      } else {
        const int rec = s_pbase[u] + (blockIdx.x - s_start[u] / c);
        float* pr = a.partials + (static_cast<int64_t>(rec) * G + h) * (D + 2);
        pr[dd] = ov;
        if (dd == 0) {
          pr[D] = M;
          pr[D + 1] = lv;
        }
      }
    }
    __syncthreads();
    a0 = seg_end;
    ++u;
    while (u < units && s_start[u + 1] <= a0) ++u;   // skip empty units
  }
}

// Merges the partials of units split over several workgroups; zero-fills
// units without live slots.
template <typename ACT, int D, int G>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const Geo& g = a.g;
  const int u = blockIdx.x;
  const int pb = a.d.unit_info[4 * u];
  const int n = a.d.unit_info[4 * u + 1];
  if (n == 1) return;
  const int row = u / g.Hkv, kh = u % g.Hkv;
  ACT* obase = static_cast<ACT*>(a.out);
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, dd = idx % D;
    float res = 0.0f;
    if (n > 1) {
      float M = -INFINITY;
      for (int i = 0; i < n; ++i) M = fmaxf(M, a.partials[(static_cast<int64_t>(pb + i) * G + h) * (D + 2) + D]);
      float ov = 0.0f, lv = 0.0f;
      for (int i = 0; i < n; ++i) {
        const float* pr = a.partials + (static_cast<int64_t>(pb + i) * G + h) * (D + 2);
        if (pr[D] == -INFINITY) continue;
        const float f = exp2f(pr[D] - M);
        ov += f * pr[dd];
        lv += f * pr[D + 1];
      }
      res = lv > 0.0f ? ov / lv : 0.0f;
    }
    store_act<ACT>(obase, (static_cast<size_t>(row) * g.Hq + kh * G + h) * D + dd, res);
  }
}

// ---------------------------------------------------------------------------
// Fast path for bf16 and fp8 pages (D = 64 or 128).
//
// Each lane owns 16 bytes of a row (8 bf16 or 16 fp8 elements), LPR lanes a
// row, RG = 64 / LPR rows per wave and pass, 4 waves per workgroup.  The
// loads of a chunk (NP passes) are issued before the previous chunk's
// arithmetic, so a wave keeps two chunks of K and V in flight.  Scores use
// the packed bf16 dot product (fp8 codes are widened to bf16 exactly); the
// row sum runs over LPR lanes with DPP; probabilities are rounded to bf16 for
// the P.V dot products, accumulation is fp32.  A unit split over workgroups
// leaves one partial record per workgroup and segment (records 2w and 2w+1:
// a workgroup's first and second segment), written with device-scope stores
// (coherent across XCDs without an L2 write-back, unlike a device-scope
// release fence); the workgroup that completes the unit's arrival count
// merges them.

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR lanes of a row (LPR in {4, 8, 16}); every lane gets the sum.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_mov<0xB1>(x);                      // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);                      // quad_perm [2,3,0,1]
  if (LPR >= 8) x += dpp_mov<0x141>(x);       // row_half_mirror
  if (LPR >= 16) x += dpp_mov<0x140>(x);      // row_mirror
  return x;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// four fp8 codes -> two bf16 pairs (exact)
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Max over all row groups of the wave (x uniform within each group), returned to every lane.
template <int LPR>
__device__ __forceinline__ float cross_rows_max(float x) {
  return lane63(rows_max_to_last(fold_groups_max<LPR>(x)));
}

// K/V rows of NP passes held in registers (one 16-byte piece or more per lane per row).
template <int NP, int NV>
struct KvChunk {
  uint4 k[NP][NV];
  uint4 v[NP][NV];
  float sk[NP], sv[NP];    // fp8 page scales of each pass's rows
};

// Issues the loads of passes [pass0, pass0 + NP) of a segment (rows at or
// past `hi` load a stand-in row, masked by compute_chunk).
// STEP: row `vrow` of the unit is the current token, read from the input rows
// kin/vin (this lane's bytes) instead of a page (fp8 pages: compute_chunk
// substitutes its quantised codes).
template <int D, int NP, bool FP8, int LPR, bool STEP = false>
__device__ __forceinline__ void load_chunk(KvChunk<NP, (D * (FP8 ? 1 : 2)) / LPR / 16>& c, const uint8_t* __restrict__ kp,
                                           const uint8_t* __restrict__ vp, const float* __restrict__ scales, int pt_reg,
                                           int first_page, int lo, int pass0,
                                           int hi, int wave, int lane_row, int lane_col, int psh, int pmask,
                                           int vrow = -1, const uint8_t* kin = nullptr, const uint8_t* vin = nullptr) {
  constexpr int RB = D * (FP8 ? 1 : 2);
  constexpr int BPL = RB / LPR;
  constexpr int NV = BPL / 16;
  constexpr int RG = 64 / LPR;
  constexpr int RPP = 4 * RG;
  // page of the block's first row (live, so its bytes are finite)
  const int pg_lo = __builtin_amdgcn_readlane(pt_reg, (lo >> psh) - first_page);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = lo + (pass0 + p) * RPP + wave * RG + lane_row;
    const bool ok = r < hi;
    // a wave's RG rows of a pass span at most two pages: read both entries
    // from the lanes holding them (uniform lane indices, no LDS crossbar)
    const int rf = lo + (pass0 + p) * RPP + wave * RG;
    const int pf = __builtin_amdgcn_readlane(pt_reg, min((rf >> psh) - first_page, 63));
    const int pl = __builtin_amdgcn_readlane(pt_reg, min(((rf + RG - 1) >> psh) - first_page, 63));
    // Every lane loads: a row past the end rereads the block's first row
    // (STEP: the input row) and is masked in the compute.  Loads under a
    // branch would make the compiler wait for this chunk's loads before
    // computing the previous one.
    // (fp8: the current token's row and the rows past the end are
    // substituted at compute time; the current token's page may not exist
    // yet — a block can start at that row, leaving no live row and page id -1
    // in pg_lo — so pool page 0 stands in for the address then)
    const bool stand = !ok || (STEP && FP8 && r == vrow);
    const int pg = stand ? ((STEP && FP8) ? max(pg_lo, 0) : pg_lo) : (((r >> psh) == (rf >> psh)) ? pf : pl);
    const int rr = stand ? lo : r;
    if (FP8) {
      // issued with the rows (a load issued later would be waited for with them)
      c.sk[p] = scales[2 * pg];
      c.sv[p] = scales[2 * pg + 1];
    }
    const uint32_t off = (static_cast<uint32_t>(pg) * static_cast<uint32_t>(pmask + 1) +
                          static_cast<uint32_t>(rr & pmask)) * static_cast<uint32_t>(RB) +
                         static_cast<uint32_t>(lane_col * BPL);
    const bool cur = STEP && !FP8 && (r == vrow || !ok);
    const uint8_t* kb = cur ? kin : kp + off;
    const uint8_t* vb = cur ? vin : vp + off;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      c.k[p][j] = *reinterpret_cast<const uint4*>(kb + 16 * j);
      c.v[p][j] = *reinterpret_cast<const uint4*>(vb + 16 * j);
    }
  }
}

// Lazy-rescale threshold of the decode online softmax (log2 units).
constexpr float kDecRescaleLog2 = 8.0f;

// Online-softmax update with the rows of one chunk.
// STEP: slot `skip` of the unit (the key the current token overwrites) is masked.
template <int D, int G, int NP, bool FP8, int LPR, bool STEP = false>
__device__ __forceinline__ void compute_chunk(const KvChunk<NP, (D * (FP8 ? 1 : 2)) / LPR / 16>& c, int lo,
                                              int pass0, int hi, int wave,
                                              int lane_row, float scale_log2,
                                              const uint32_t (&qv)[G][(D * (FP8 ? 1 : 2)) / LPR / 16 * (16 / (FP8 ? 1 : 2)) / 2],
                                              float (&m)[G], float (&l)[G],
                                              float (&o)[G][(D * (FP8 ? 1 : 2)) / LPR / 16 * (16 / (FP8 ? 1 : 2))],
                                              int skip = -1, int vrow = -1, const uint4* vk = nullptr,
                                              const uint4* vv = nullptr, float vsk = 1.0f, float vsv = 1.0f) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int RB = D * EB;
  constexpr int BPL = RB / LPR;
  constexpr int NV = BPL / 16;
  constexpr int EPL = BPL / EB;
  constexpr int QW = EPL / 2;
  constexpr int RG = 64 / LPR;
  constexpr int RPP = 4 * RG;
  bool ok[NP];
  float sk[NP], sv[NP];
  // STEP with fp8 pages: the current token's row (row vrow) takes the codes
  // and scales it will have once stored (vk, vv, vsk, vsv)
  KvChunk<NP, NV> cc;
  if constexpr (STEP && FP8) cc = c;
  const KvChunk<NP, NV>& cu = (STEP && FP8) ? cc : c;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = lo + (pass0 + p) * RPP + wave * RG + lane_row;
    ok[p] = r < hi && (!STEP || r != skip);
    if constexpr (STEP && FP8) {
      // (rows past the end take the same codes: finite, and masked)
      const bool vr = r == vrow || r >= hi;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        cc.k[p][j] = vr ? vk[j] : c.k[p][j];
        cc.v[p][j] = vr ? vv[j] : c.v[p][j];
      }
      cc.sk[p] = vr ? vsk : c.sk[p];
      cc.sv[p] = vr ? vsv : c.sv[p];
    }
    sk[p] = scale_log2;
    sv[p] = 1.0f;
    if (FP8) {
      sk[p] *= cu.sk[p];
      sv[p] = cu.sv[p];
    }
  }
  float s[NP][G];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t kw[QW];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint32_t raw[4] = {cu.k[p][j].x, cu.k[p][j].y, cu.k[p][j].z, cu.k[p][j].w};
      if (FP8) {
#pragma unroll
        for (int t = 0; t < 4; ++t) fp8x4_to_bf16(raw[t], kw[8 * j + 2 * t], kw[8 * j + 2 * t + 1]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) kw[4 * j + t] = raw[t];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < QW; ++j) acc = dot2(qv[h][j], kw[j], acc);
      acc = row_sum<LPR>(acc) * sk[p];
      s[p][h] = ok[p] ? acc : -INFINITY;
    }
  }
  float pe[NP][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = s[0][h];
#pragma unroll
    for (int p = 1; p < NP; ++p) mx = fmaxf(mx, s[p][h]);
    mx = cross_rows_max<LPR>(mx);
    // Lazy rescale: the reference max m moves only when a score passes it by
    // more than 2^kDecRescaleLog2 (wave-uniform branch), so the weights
    // exp2(s - m) stay below 2^kDecRescaleLog2, exact enough in fp32 and as
    // packed bf16, and most chunks skip the rescale.  The first real score
    // always moves m off -inf (alpha 0 on zero state).
    if (__builtin_amdgcn_readfirstlane(__float_as_int(mx)) != __float_as_int(-INFINITY) &&
        __builtin_amdgcn_readfirstlane(mx > m[h] + kDecRescaleLog2)) {
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);   // m = -inf gives 0
      m[h] = mx;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
    }
    // no real score yet: subtract nothing (every weight is exp2(-inf) = 0)
    const float msub = (m[h] == -INFINITY) ? 0.0f : m[h];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      pe[p][h] = __builtin_amdgcn_exp2f(s[p][h] - msub);   // -inf gives 0
      l[h] += pe[p][h];
    }
  }
#pragma unroll
  for (int p = 0; p < NP; p += 2) {
    uint32_t va[QW], vb[QW];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint32_t ra[4] = {cu.v[p][j].x, cu.v[p][j].y, cu.v[p][j].z, cu.v[p][j].w};
      const uint32_t rc[4] = {cu.v[p + 1][j].x, cu.v[p + 1][j].y, cu.v[p + 1][j].z, cu.v[p + 1][j].w};
      if (FP8) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          fp8x4_to_bf16(ra[t], va[8 * j + 2 * t], va[8 * j + 2 * t + 1]);
          fp8x4_to_bf16(rc[t], vb[8 * j + 2 * t], vb[8 * j + 2 * t + 1]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          va[4 * j + t] = ra[t];
          vb[4 * j + t] = rc[t];
        }
      }
    }
    uint32_t pk[G];
#pragma unroll
    for (int h = 0; h < G; ++h) pk[h] = pack_bf16(pe[p][h] * sv[p], pe[p + 1][h] * sv[p + 1]);
#pragma unroll
    for (int j = 0; j < QW; ++j) {
      const uint32_t lo2 = __builtin_amdgcn_perm(vb[j], va[j], 0x05040100u);   // (row p, row p+1) of element 2j
      const uint32_t hi2 = __builtin_amdgcn_perm(vb[j], va[j], 0x07060302u);   // element 2j+1
#pragma unroll
      for (int h = 0; h < G; ++h) {
        o[h][2 * j] = dot2(pk[h], lo2, o[h][2 * j]);
        o[h][2 * j + 1] = dot2(pk[h], hi2, o[h][2 * j + 1]);
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Matrix-core variant (bf16 pages, D = 64 or 128, pages of at least 16 rows).
//
// A wave takes 16-row tiles of its segment, aligned to 16 rows of the unit so
// that a tile lies in one page.  The tile's scores for the group's G query
// heads come from v_mfma_f32_16x16x32_bf16 with the 16 keys as rows (A: lane
// (g, n) = (lane / 16, lane % 16) holds the 8 elements 32s + 8g.. of key n's
// row, loaded from the page) and the heads as columns (B: the same elements of
// query head n, zero from head G on); lane (g, n) is left the scores of keys
// 4g..4g+3 for head n.  The max over the tile's keys is a reduction over the
// four 16-lane rows.  The P.V products run on the vector ALU over coalesced V
// loads (whole rows per load): lane (g, s, c) holds 16-byte piece c of the V
// rows of keys of its row group g, takes head h's probabilities from lane
// (g, h) by a row broadcast, and accumulates o[h][8c..8c+8] with packed bf16
// dot products over key pairs.  Per 16 keys that is D / 32 matrix products
// and about (G + 2) * 16 vector instructions, against G * D / 4 packed dot
// products and the per-row reductions of the lane-per-row-piece kernel.

typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));

// max / sum of lane l and lane l ^ 32 (resp. l ^ 16): the swap builtins
// return the pair (own, partner) in a lane-independent order.
__device__ __forceinline__ float mf_max_x32(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float mf_max_x16(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float mf_sum_x32(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float mf_sum_x16(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// lane h of each 16-lane row, to every lane of the row (row_newbcast:h)
template <int H>
__device__ __forceinline__ uint32_t mf_row_bcast(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x150 + H, 0xF, 0xF, false));
}

template <int D>
struct MfTile {
  static constexpr int KS = D / 32;                // k-steps of the score product
  static constexpr int NVI = D == 128 ? 4 : 2;     // V loads per tile
  uint4 k[KS];
  uint4 v[NVI];
};

// Issues the loads of tile t of a page block (clamped to its last tile, nt
// tiles from row t0): K in the matrix-core layout, V as whole rows.  Rows past
// `hi` read the tile's first row instead (finite: a live row or, STEP, the
// current token's input row) and are masked; STEP: row `vrow` is the current
// token, read from the input rows kin0 / vin0.
template <int D, bool STEP>
__device__ __forceinline__ void mf_load(MfTile<D>& b, int t, int nt, int t0, int pb, int pt_reg,
                                        const uint8_t* __restrict__ kp, const uint8_t* __restrict__ vp, int hi,
                                        int psh, int pmask, int vrow, const uint8_t* kin0, const uint8_t* vin0,
                                        int lane) {
  constexpr int RB = D * 2, VL = D / 8, RPG = 16 / VL;
  const int tb = t0 + 16 * min(t, nt - 1);
  const int page = __builtin_amdgcn_readlane(pt_reg, (tb >> psh) - pb);
  const uint32_t prow = static_cast<uint32_t>(page) * static_cast<uint32_t>(pmask + 1);
  const int g4 = lane >> 4, n16 = lane & 15;
  const bool tb_in = STEP && tb == vrow;
  {
    const int r = tb + n16;
    const bool past = r >= hi;
    const bool in = STEP && (past ? tb_in : r == vrow);
    const int rr = past ? tb : r;
    const uint8_t* base = in ? kin0 : kp + (prow + static_cast<uint32_t>(rr & pmask)) * static_cast<uint32_t>(RB);
#pragma unroll
    for (int s = 0; s < MfTile<D>::KS; ++s) b.k[s] = *reinterpret_cast<const uint4*>(base + (32 * s + 8 * g4) * 2);
  }
  const int vs = (lane & 15) / VL, vc = lane % VL;
#pragma unroll
  for (int j = 0; j < MfTile<D>::NVI; ++j) {
    const int r = tb + 4 * g4 + RPG * j + vs;
    const bool past = r >= hi;
    const bool in = STEP && (past ? tb_in : r == vrow);
    const int rr = past ? tb : r;
    const uint8_t* base = in ? vin0 : vp + (prow + static_cast<uint32_t>(rr & pmask)) * static_cast<uint32_t>(RB);
    b.v[j] = *reinterpret_cast<const uint4*>(base + 16 * vc);
  }
}

// o[8] += P (bf16 pair: keys a, b) . (V rows a, b), 8 elements
__device__ __forceinline__ void mf_pv_pair(const uint4& va, const uint4& vb, uint32_t P, float* o) {
  const uint32_t x[4] = {va.x, va.y, va.z, va.w};
  const uint32_t y[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo2 = __builtin_amdgcn_perm(y[w], x[w], 0x05040100u);
    const uint32_t hi2 = __builtin_amdgcn_perm(y[w], x[w], 0x07060302u);
    o[2 * w] = dot2(P, lo2, o[2 * w]);
    o[2 * w + 1] = dot2(P, hi2, o[2 * w + 1]);
  }
}

template <int D, int G, int H>
__device__ __forceinline__ void mf_pv_head(const MfTile<D>& b, uint32_t pa, uint32_t pb, bool vs1, float (&o)[G][8]) {
  if constexpr (H < G) {
    const uint32_t Pa = mf_row_bcast<H>(pa), Pb = mf_row_bcast<H>(pb);
    if constexpr (D == 128) {
      mf_pv_pair(b.v[0], b.v[1], Pa, o[H]);
      mf_pv_pair(b.v[2], b.v[3], Pb, o[H]);
    } else {
      mf_pv_pair(b.v[0], b.v[1], vs1 ? Pb : Pa, o[H]);
    }
    mf_pv_head<D, G, H + 1>(b, pa, pb, vs1, o);
  }
}

// Online-softmax update with tile t: m (running max, base 2) and lsum are
// lane (g, n)'s for head n (lsum over the keys of its row group); o[h][e] is
// lane (g, s, c)'s partial for element 8c + e of head h.
template <int D, int G, bool STEP>
__device__ __forceinline__ void mf_compute(const MfTile<D>& b, int t, int t0, int lo, int hi, int skip,
                                           float scale_log2, const uint4 (&qb)[D / 32], float& m, float& lsum,
                                           float (&o)[G][8], int lane) {
  const int g4 = lane >> 4, n16 = lane & 15;
  const int tb = t0 + 16 * t;
  mf_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < MfTile<D>::KS; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, b.k[s]),
                                                  __builtin_bit_cast(mf_bf16x8, qb[s]), acc, 0, 0, 0);
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tb + 4 * g4 + i;
    const bool ok = n16 < G && r >= lo && r < hi && (!STEP || r != skip);
    sc[i] = ok ? acc[i] * scale_log2 : -INFINITY;
  }
  float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  tmax = mf_max_x16(mf_max_x32(tmax));
  // lazy rescale (see compute_chunk); every lane of head n moves together
  const bool need = tmax > m + kDecRescaleLog2;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(m - tmax) : 1.0f;   // m = -inf gives 0
    if (need) m = tmax;
    lsum *= alpha;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ah = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= ah;
    }
  }
  const float msub = (m == -INFINITY) ? 0.0f : m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - msub);   // -inf gives 0
  lsum += (p[0] + p[1]) + (p[2] + p[3]);
  // key pairs of the P.V products: (0, 1), (2, 3) for D = 128 (a lane's V rows
  // are keys 4g..4g+3); (0, 2), (1, 3) for D = 64 (keys 4g + s, 4g + 2 + s)
  const uint32_t pa = D == 128 ? pack_bf16(p[0], p[1]) : pack_bf16(p[0], p[2]);
  const uint32_t pb = D == 128 ? pack_bf16(p[2], p[3]) : pack_bf16(p[1], p[3]);
  mf_pv_head<D, G, 0>(b, pa, pb, (lane & 15) >= 8, o);
}

// Combines the partial records (m, l, o) of one unit's workgroups w0..w1 into
// its bf16 output [G][D] (256 threads); the records are read with
// device-scope atomic loads (written by workgroups on other XCDs).  The first workgroup's record is its
// second segment when `odd`.  All loads of a batch of records (16, or 8
// when a thread combines more than two outputs) are issued before any of
// them is used.
template <int D, int G>
__device__ __forceinline__ void merge_unit_records(float* partials, int w0, int w1, int odd, uint16_t* out) {
  constexpr int PER = (G * D + 255) / 256;
  const int n = w1 - w0 + 1;
  float M[PER], O[PER], L[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    M[i] = -INFINITY;
    O[i] = 0.0f;
    L[i] = 0.0f;
  }
  constexpr int MB = PER <= 2 ? 16 : 8;   // records per batch of loads
  for (int b0 = 0; b0 < n; b0 += MB) {
    float mv[MB][PER], lv[MB][PER], ov[MB][PER];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int w = w0 + b0 + j;
      const int rec = (b0 + j == 0 && odd) ? 2 * w + 1 : 2 * w;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int h = idx / D, dd = idx % D;
        if (b0 + j < n && idx < G * D) {
          float* pr = partials + (static_cast<int64_t>(rec) * G + h) * (D + 2);
          mv[j][i] = __hip_atomic_load(pr + D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          lv[j][i] = __hip_atomic_load(pr + D + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ov[j][i] = __hip_atomic_load(pr + dd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          mv[j][i] = -INFINITY;
          lv[j][i] = 0.0f;
          ov[j][i] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float mb = M[i];
#pragma unroll
      for (int j = 0; j < MB; ++j) mb = fmaxf(mb, mv[j][i]);
      if (mb == -INFINITY) continue;
      const float f0 = exp2f(M[i] - mb);
      O[i] *= f0;
      L[i] *= f0;
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const float f = exp2f(mv[j][i] - mb);
        O[i] = fmaf(f, ov[j][i], O[i]);
        L[i] = fmaf(f, lv[j][i], L[i]);
      }
      M[i] = mb;
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = threadIdx.x + 256 * i;
    if (idx < G * D) out[idx] = f32_to_bf16(L[i] > 0.0f ? O[i] / L[i] : 0.0f);
  }
}

// Inputs of the fused decode step that the attention role reads.
struct StepArgs {
  const uint8_t* k;        // [B][Hkv][D] bf16 rows of the current token
  const uint8_t* v;
  int npairs;              // (row, KV head) pairs of the call (B * Hkv)
  int nprep;               // workgroups of the prepare role, placed first in the grid: one per pair, or
                           // (per_row) one per batch row
  int per_row;
  int groups;              // arrival groups of the attention workgroups (min(kArriveGroups, their count))
  int agrid;               // attention workgroups
  int qneuron;             // the decision neuron (last element of each group's first query head) reads as zero
  int spin_limit;          // polls of the commit's wait before it gives up (0: give up at once)
};

// Up to this many units (and at most half as many as workgroups) each unit
// gets whole workgroups of its own.
constexpr int kAlignedUnits = 512;
// ... at most this many: the merge of a unit's records then takes one batch
// of loads (a few units with short contexts would otherwise spread over
// dozens of workgroups whose merge costs more than their streaming saves).
constexpr int kMaxSplit = 16;

template <int G, int D, bool STEP>
struct FastLds {
  int start[kMaxUnits + 1];
  int wstart[kAlignedUnits + 1];       // unit-aligned split: first workgroup of each unit
  int ext[STEP ? kMaxUnits : 1];    // STEP: -1 no current token, else 1 + the slot it overwrites (0: appended)
  int tmp[4];
  union {
    float o[4][4][G][D];               // [wave][DPP row][head][dim]
    PrepShared prep;                   // the commit (before any use of o)
  };
  float ml[4][4][G][2];                // m (row 0 only) and l per row
};

// Live slots (and, STEP, the current token's placement) of unit u.
template <bool STEP>
__device__ __forceinline__ int unit_slots(const DecodeArgs& a, int u, int wg, int* ext) {
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int row = u / g.Hkv, kh = u % g.Hkv;
  const int seq = a.seq_ids ? a.seq_ids[row] : row;
  *ext = -1;
  if (seq < 0 || seq >= g.Bmax) {
    if (wg == 0 && kh == 0) set_status(d.ctl, DMS_DEV_BAD_SEQ);
    return 0;
  }
  const int unit = seq * g.Hkv + kh;
  int L = d.lengths[unit];
  if (STEP) {
    // the current token: in place over the slot of position t - w when that
    // token was marked, else appended as slot L (the prepare role's choice)
    const int t = d.pos[seq];
    if (t + 1 <= g.max_tokens) {
      int skip = -1;
      if (t >= g.w) {
        const int rv = d.ring[static_cast<int64_t>(unit) * g.w + t % g.w];
        if (rv < 0) skip = rv & 0x7FFFFFFF;
      }
      *ext = skip + 1;
      L += 1;
    }
  }
  return L;
}

// Tiles in flight per wave in the matrix-core decode (a ring of buffers); 3
// or 4 also fit two waves per SIMD (221, 254 registers) but measured slower.
constexpr int kMfTiles = 2;

// One wave's share of a segment (rows [lo, hi) of unit (row, kh)) on the
// matrix cores: the wave takes tiles wave, wave + 4, ... of each page block,
// keeps kMfTiles tiles in flight, and leaves its (m, l, o) in entry 0 of the
// workgroup's LDS rows (m, l of head h from lane h, o from the lanes of row
// group 0).
template <int D, int G, bool STEP>
__device__ __forceinline__ void mf_segment(const DecodeArgs& a, const StepArgs* sa, FastLds<G, D, STEP>& lds,
                                           bool use_plan, int p_np, int p_page, const int32_t* pt, int row, int kh,
                                           int lo, int hi, int vrow, int skip, int wave, int lane) {
  constexpr int KS = D / 32, VL = D / 8;
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int psh = g.Pshift, pmask = g.P - 1;
  const int g4 = lane >> 4, n16 = lane & 15;
  // query rows as the B operand: lane (g, n) holds elements 32s + 8g.. of head n
  uint4 qb[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<size_t>(row) * g.Hq + kh * G + min(n16, G - 1)) * D + 8 * g4;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qb[s] = n16 < G ? *reinterpret_cast<const uint4*>(qp + 32 * s) : make_uint4(0, 0, 0, 0);
    // the decision neuron (element D - 1 of the group's first head) plays no
    // part in attention (the commit zeroes it in memory)
    if (STEP && sa->qneuron && n16 == 0 && g4 == 3) qb[KS - 1].w &= 0xFFFFu;
  }
  const uint8_t* kin0 = nullptr;
  const uint8_t* vin0 = nullptr;
  if constexpr (STEP) {
    const size_t ro = (static_cast<size_t>(row) * g.Hkv + kh) * (D * 2);
    kin0 = sa->k + ro;
    vin0 = sa->v + ro;
  }
  float m = -INFINITY, lsum = 0.0f;
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;
  for (int pb = lo >> psh; pb <= (hi - 1) >> psh; pb += 64) {
    const int plast = min((hi - 1) >> psh, pb + 63);
    const bool from_plan = use_plan && p_np > 0;
    const int pt_reg = from_plan ? (lane < p_np ? p_page : 0) : (pb + lane <= plast) ? pt[pb + lane] : 0;
    const int blo = max(lo, pb << psh), bhi = min(hi, (plast + 1) << psh);
    const int t0 = blo & ~15;
    const int nt = (bhi - t0 + 15) >> 4;
    // loads one tile ahead, unconditionally (past the block's end they reread
    // its last tile), in written order (see the lane-per-row-piece kernel)
    constexpr int NB = kMfTiles;
    MfTile<D> ring[NB];
    auto load = [&](MfTile<D>& b, int t) {
      mf_load<D, STEP>(b, t, nt, t0, pb, pt_reg, d.k_pages, d.v_pages, hi, psh, pmask, vrow, kin0, vin0, lane);
    };
    auto compute = [&](const MfTile<D>& b, int t) {
      mf_compute<D, G, STEP>(b, t, t0, lo, hi, skip, g.scale_log2, qb, m, lsum, o, lane);
    };
#pragma unroll
    for (int k = 0; k < NB - 1; ++k) load(ring[k], wave + 4 * k);
    for (int t = wave; t < nt; t += 4 * NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        load(ring[(k + NB - 1) % NB], t + 4 * (k + NB - 1));
        __builtin_amdgcn_sched_barrier(0);
        if (t + 4 * k < nt) compute(ring[k], t + 4 * k);
      }
    }
  }
  // sums over the row groups (and, D = 64, the two rows of a group)
  lsum = mf_sum_x16(mf_sum_x32(lsum));
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = mf_sum_x16(mf_sum_x32(o[h][e]));
      if (VL == 8) x += dpp_f<0x128, 0xF>(x, 0.0f);   // row_ror:8
      o[h][e] = x;
    }
  if (lane < VL) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) lds.o[wave][0][h][8 * lane + e] = o[h][e];
  }
  if (lane < G) {
    lds.ml[wave][0][lane][0] = m;
    lds.ml[wave][0][lane][1] = lsum;
  }
}

// Matrix-core variant for fp8 pages (D = 128, dms_decode_attn).  The same
// tiles and lane roles as the bf16 variant, with the contraction index of the
// score product permuted: lane (g, n) loads the 32 contiguous codes
// 32g..32g+31 of key n's row (two 16-byte loads) and uses codes 32g + 8s..
// at k-step s, widened exactly to bf16; the query operand takes the same
// elements.  V rows are 128 bytes: lane (g, s, c) holds codes 16c..16c+15 of
// the rows of keys 4g + s and 4g + 2 + s.  A tile lies in one page, so the
// page's K scale multiplies the tile's scores and its V scale the
// probabilities of the P.V products (l sums the unscaled ones).
struct Mf8Tile {
  uint4 k[2];
  uint4 v[2];
  float sk, sv;
};

__device__ __forceinline__ void mf8_load(Mf8Tile& b, int t, int nt, int t0, int pb, int pt_reg,
                                         const uint8_t* __restrict__ kp, const uint8_t* __restrict__ vp,
                                         const float* __restrict__ scales, int hi, int psh, int pmask, int lane) {
  constexpr int RB = 128;
  const int tb = t0 + 16 * min(t, nt - 1);
  const int page = __builtin_amdgcn_readlane(pt_reg, (tb >> psh) - pb);
  const uint32_t prow = static_cast<uint32_t>(page) * static_cast<uint32_t>(pmask + 1);
  const int g4 = lane >> 4, n16 = lane & 15;
  b.sk = scales[2 * page];
  b.sv = scales[2 * page + 1];
  {
    const int r = tb + n16;
    const int rr = r >= hi ? tb : r;
    const uint8_t* base = kp + (prow + static_cast<uint32_t>(rr & pmask)) * static_cast<uint32_t>(RB) + 32 * g4;
    b.k[0] = *reinterpret_cast<const uint4*>(base);
    b.k[1] = *reinterpret_cast<const uint4*>(base + 16);
  }
  const int vs = (lane & 15) >> 3, vc = lane & 7;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = tb + 4 * g4 + 2 * j + vs;
    const int rr = r >= hi ? tb : r;
    b.v[j] = *reinterpret_cast<const uint4*>(vp + (prow + static_cast<uint32_t>(rr & pmask)) *
                                                      static_cast<uint32_t>(RB) + 16 * vc);
  }
}

// o[16] += P (bf16 pair: keys a, b) . (fp8 V rows a, b, 16 codes each, widened exactly)
__device__ __forceinline__ void mf8_pv_pair(const uint4& va, const uint4& vb, uint32_t P, float* o) {
  const uint32_t x[4] = {va.x, va.y, va.z, va.w};
  const uint32_t y[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t xl, xh, yl, yh;                      // codes 4w..4w+3 as two bf16 pairs
    fp8x4_to_bf16(x[w], xl, xh);
    fp8x4_to_bf16(y[w], yl, yh);
    const uint32_t xs[2] = {xl, xh}, ys[2] = {yl, yh};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t lo2 = __builtin_amdgcn_perm(ys[q], xs[q], 0x05040100u);
      const uint32_t hi2 = __builtin_amdgcn_perm(ys[q], xs[q], 0x07060302u);
      o[4 * w + 2 * q] = dot2(P, lo2, o[4 * w + 2 * q]);
      o[4 * w + 2 * q + 1] = dot2(P, hi2, o[4 * w + 2 * q + 1]);
    }
  }
}

template <int G, int H>
__device__ __forceinline__ void mf8_pv_head(const Mf8Tile& b, uint32_t pa, uint32_t pb, bool vs1, float (&o)[G][16]) {
  if constexpr (H < G) {
    const uint32_t Pa = mf_row_bcast<H>(pa), Pb = mf_row_bcast<H>(pb);
    mf8_pv_pair(b.v[0], b.v[1], vs1 ? Pb : Pa, o[H]);
    mf8_pv_head<G, H + 1>(b, pa, pb, vs1, o);
  }
}

template <int G>
__device__ __forceinline__ void mf8_compute(const Mf8Tile& b, int t, int t0, int lo, int hi, float scale_log2,
                                            const uint4 (&qb)[4], float& m, float& lsum, float (&o)[G][16],
                                            int lane) {
  const int g4 = lane >> 4, n16 = lane & 15;
  const int tb = t0 + 16 * t;
  mf_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t kw[8] = {b.k[0].x, b.k[0].y, b.k[0].z, b.k[0].w, b.k[1].x, b.k[1].y, b.k[1].z, b.k[1].w};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t a0, a1, a2, a3;
    fp8x4_to_bf16(kw[2 * s], a0, a1);
    fp8x4_to_bf16(kw[2 * s + 1], a2, a3);
    const uint4 a = make_uint4(a0, a1, a2, a3);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, a),
                                                  __builtin_bit_cast(mf_bf16x8, qb[s]), acc, 0, 0, 0);
  }
  const float sc_k = scale_log2 * b.sk;
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tb + 4 * g4 + i;
    const bool ok = n16 < G && r >= lo && r < hi;
    sc[i] = ok ? acc[i] * sc_k : -INFINITY;
  }
  float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  tmax = mf_max_x16(mf_max_x32(tmax));
  const bool need = tmax > m + kDecRescaleLog2;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(m - tmax) : 1.0f;
    if (need) m = tmax;
    lsum *= alpha;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ah = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
#pragma unroll
      for (int e = 0; e < 16; ++e) o[h][e] *= ah;
    }
  }
  const float msub = (m == -INFINITY) ? 0.0f : m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - msub);
  lsum += (p[0] + p[1]) + (p[2] + p[3]);
  // V rows of a lane: keys 4g + s and 4g + 2 + s
  const uint32_t pa = pack_bf16(p[0] * b.sv, p[2] * b.sv);
  const uint32_t pb = pack_bf16(p[1] * b.sv, p[3] * b.sv);
  mf8_pv_head<G, 0>(b, pa, pb, (lane & 15) >= 8, o);
}

template <int G>
__device__ __forceinline__ void mf8_segment(const DecodeArgs& a, FastLds<G, 128, false>& lds, const int32_t* pt,
                                            int row, int kh, int lo, int hi, int wave, int lane) {
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int psh = g.Pshift, pmask = g.P - 1;
  const int g4 = lane >> 4, n16 = lane & 15;
  // query operand: lane (g, n) holds elements 32g + 8s.. of head n at k-step s
  uint4 qb[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<size_t>(row) * g.Hq + kh * G + min(n16, G - 1)) * 128 + 32 * g4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qb[s] = n16 < G ? *reinterpret_cast<const uint4*>(qp + 8 * s) : make_uint4(0, 0, 0, 0);
  }
  float m = -INFINITY, lsum = 0.0f;
  float o[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[h][e] = 0.0f;
  for (int pb = lo >> psh; pb <= (hi - 1) >> psh; pb += 64) {
    const int plast = min((hi - 1) >> psh, pb + 63);
    const int pt_reg = (pb + lane <= plast) ? pt[pb + lane] : 0;
    const int blo = max(lo, pb << psh), bhi = min(hi, (plast + 1) << psh);
    const int t0 = blo & ~15;
    const int nt = (bhi - t0 + 15) >> 4;
    Mf8Tile ta, tb;
    auto load = [&](Mf8Tile& b, int t) {
      mf8_load(b, t, nt, t0, pb, pt_reg, d.k_pages, d.v_pages, d.scales, hi, psh, pmask, lane);
    };
    auto compute = [&](const Mf8Tile& b, int t) { mf8_compute<G>(b, t, t0, lo, hi, g.scale_log2, qb, m, lsum, o, lane); };
    load(ta, wave);
    for (int t = wave; t < nt; t += 8) {
      __builtin_amdgcn_sched_barrier(0);
      load(tb, t + 4);
      __builtin_amdgcn_sched_barrier(0);
      compute(ta, t);
      __builtin_amdgcn_sched_barrier(0);
      load(ta, t + 8);
      __builtin_amdgcn_sched_barrier(0);
      if (t + 4 < nt) compute(tb, t + 4);
    }
  }
  // sums over the row groups and the two rows of a group
  lsum = mf_sum_x16(mf_sum_x32(lsum));
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[h][e] = mf_sum_x16(mf_sum_x32(o[h][e]));
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[h][e] += dpp_f<0x128, 0xF>(o[h][e], 0.0f);   // row_ror:8
  if (lane < 8) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) lds.o[wave][0][h][16 * lane + e] = o[h][e];
  }
  if (lane < G) {
    lds.ml[wave][0][lane][0] = m;
    lds.ml[wave][0][lane][1] = lsum;
  }
}

// The decode plan (fused step): the kernel variant a plan was split for, and
// where its rows and records start.
template <int D, int G, bool FP8, int LPR, bool MF>
__device__ __forceinline__ constexpr int plan_variant() {
  return D | (G << 8) | ((FP8 ? 1 : 0) << 12) | ((MF ? 1 : 0) << 13) | (LPR << 16) | (1 << 24);
}
__device__ __forceinline__ int32_t* plan_rows(const DevCache& d) { return d.plan + kPlanHeader; }
__device__ __forceinline__ int32_t* plan_records(const DevCache& d, const Geo& g) {
  return d.plan + kPlanHeader + ((g.Bmax + 63) & ~63);
}
// record words
constexpr int kRecUnit = 0, kRecLo = 1, kRecHi = 2, kRecRows = 3, kRecExt = 4, kRecW0 = 5, kRecW1 = 6,
              kRecScalePage = 7, kRecNpages = 8, kRecPages = 9;
constexpr int kRecMaxPages = kPlanRec - kRecPages;

// The attention of dms_decode_attn (workgroup wg of `grid`).  STEP: the
// attention of the fused decode step, run before the current token is in the
// cache: each unit's rows are its live slots plus one more, the current
// token, read from the input rows; the slot the token overwrites in place is
// masked.  The same keys as after the append.  Once a workgroup has read the
// lengths, positions and ring entries it works from, it counts itself on its
// arrival group; the prepare role's commit waits for all of them.
template <int D, int G, int NP, bool FP8, int LPR, bool STEP, bool MF = false>
__device__ __forceinline__ void decode_attn_fast_body(const DecodeArgs& a, const StepArgs* sa, int wg, int grid,
                                                      FastLds<G, D, STEP>& lds) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int RB = D * EB;
  constexpr int BPL = RB / LPR;
  constexpr int EPL = BPL / EB;
  constexpr int QW = EPL / 2;
  constexpr int RG = 64 / LPR;
  // rows per workgroup pass: the floor of a workgroup's share in the split
  constexpr int RPP = MF ? 64 : 4 * RG;
  static_assert(!MF || !FP8 || (!STEP && D == 128), "matrix-core fp8: dms_decode_attn with head_dim 128");
  constexpr int NV = BPL / 16;
  static_assert(NP % 2 == 0, "passes are paired for the P.V dot products");
  static_assert(BPL % 16 == 0, "a lane loads whole 16-byte pieces");

  int* s_start = lds.start;
  int* s_tmp = lds.tmp;
  int* s_wstart = lds.wstart;
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lane_row = lane / LPR, lane_col = lane % LPR;
  const int units = a.B * g.Hkv;

  // STEP: the plan the previous step's commit left, when it was made for this
  // kernel, grid, batch and row-to-sequence mapping and nothing has changed
  // the cache since (every other call that does clears it).  It gives this
  // workgroup's unit, row range, page ids and the next token's placement in
  // one load, in place of the length, position and ring reads, the scans
  // and the page-table read.
  bool use_plan = false;
  int p_u = 0, p_lo = 0, p_hi = 0, p_rows = 0, p_ext = -1, p_w0 = 0, p_w1 = 0, p_spage = -1, p_np = -1, p_page = 0;
  if constexpr (STEP) {
    if (grid <= kPlanMaxWgs) {
      const int32_t* P = d.plan;
      const int32_t* rec = plan_records(d, g) + static_cast<int64_t>(wg) * kPlanRec;
      const int rv = rec[lane & (kPlanRec - 1)];
      p_page = rec[kRecPages + min(lane, kRecMaxPages - 1)];
      const int nrec = P[kPlanNrec];
      int bad = !(P[kPlanValid] == 1 && P[kPlanB] == a.B && P[kPlanGrid] == grid &&
                  P[kPlanSeqNull] == (a.seq_ids == nullptr ? 1 : 0) &&
                  P[kPlanVariant] == plan_variant<D, G, FP8, LPR, MF>());
      for (int r = tid; r < a.B; r += 256)
        if ((a.seq_ids ? a.seq_ids[r] : r) != plan_rows(d)[r]) bad = 1;
      use_plan = !__syncthreads_or(bad);
      if (use_plan) {
        p_u = __builtin_amdgcn_readlane(rv, kRecUnit);
        p_lo = __builtin_amdgcn_readlane(rv, kRecLo);
        p_hi = __builtin_amdgcn_readlane(rv, kRecHi);
        p_rows = __builtin_amdgcn_readlane(rv, kRecRows);
        p_ext = __builtin_amdgcn_readlane(rv, kRecExt);
        p_w0 = __builtin_amdgcn_readlane(rv, kRecW0);
        p_w1 = __builtin_amdgcn_readlane(rv, kRecW1);
        p_spage = __builtin_amdgcn_readlane(rv, kRecScalePage);
        p_np = __builtin_amdgcn_readlane(rv, kRecNpages);
        // every plan word this workgroup uses has arrived (the commit
        // rewrites the plan once all have arrived), and nothing it reads
        // later can change: arrive
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        if (tid == 0)
          __hip_atomic_fetch_add(d.arrive + (wg % sa->groups) * kArriveStride, 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        if (wg >= nrec) return;
      }
    }
  }

  int W = 0, c = 0;
  bool aligned = true;
  int a0, a1, u;
  if (use_plan) {
    u = p_u;
    a0 = p_lo;
    a1 = p_hi;
  } else {
  // -- unit prefix (live slots of every (row, KV head), concatenated) --------
  if (units <= 64) {
    if (wave == 0) {
      int L = 0, ext = -1;
      if (lane < units) L = unit_slots<STEP>(a, lane, wg, &ext);
      int incl = L;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      if (lane < units) {
        s_start[lane] = incl - L;
        if (STEP) lds.ext[lane] = ext;
      }
      if (lane == 63) s_start[units] = incl;
    }
    __syncthreads();
  } else {
    const int per = (units + 255) / 256;
    const int u0 = tid * per;
    int len[8];
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int u = u0 + i;
      int L = 0, ext = -1;
      if (u < units) {
        L = unit_slots<STEP>(a, u, wg, &ext);
        if (STEP) lds.ext[u] = ext;
      }
      len[i] = L;
      sum += L;
    }
    int W;
    int run = block_scan_256(sum, s_tmp, &W);
    for (int i = 0; i < per; ++i) {
      const int u = u0 + i;
      if (u < units) s_start[u] = run;
      run += len[i];
    }
    if (tid == 0) s_start[units] = W;
    __syncthreads();
  }
  if constexpr (STEP) {
    // every read of state the commit changes has returned (the values are in
    // LDS): arrive, without waiting for the add to complete
    if (tid == 0)
      __hip_atomic_fetch_add(d.arrive + (wg % sa->groups) * kArriveStride, 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  W = s_start[units];
  c = max((W + grid - 1) / grid, RPP);
  // Few units: each unit gets workgroups of its own, ceil(slots / ca) of
  // them for a cap of ca = ceil(W / (grid - units)) slots per workgroup (at
  // most one per RPP rows and kMaxSplit in all), so no workgroup spans two
  // units (a second segment would repeat the setup and the merge);
  // sum(ceil(slots / ca)) <= W / ca + units <= grid.  Otherwise the
  // concatenated slots are cut into equal ranges.
  aligned = units <= kAlignedUnits && 2 * units <= grid;
  if (aligned) {
    const int ca = max(1, (W + (grid - units) - 1) / (grid - units));
    const int u0 = tid * 2;
    int nw[2], sum = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = u0 + i;
      int n = 0;
      if (u < units) {
        const int wu = s_start[u + 1] - s_start[u];
        if (wu > 0) n = min(min((wu + ca - 1) / ca, max(1, wu / RPP)), kMaxSplit);
      }
      nw[i] = n;
      sum += n;
    }
    int tot;
    int run = block_scan_256(sum, s_tmp, &tot);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (u0 + i < units) s_wstart[u0 + i] = run;
      run += nw[i];
    }
    if (tid == 0) s_wstart[units] = tot;
    __syncthreads();
  }

  // heads without live slots have no workgroup: the last workgroup writes
  // their zeros (a thread per unit; it is the one most often left without
  // slots of its own, and no merge waits for it)
  if (wg == grid - 1) {
    uint4* ob = static_cast<uint4*>(a.out);
    for (int uu = tid; uu < units; uu += 256) {
      if (s_start[uu + 1] != s_start[uu]) continue;
      const int row = uu / g.Hkv, kh = uu % g.Hkv;
      uint4* dst = ob + (static_cast<size_t>(row) * g.Hq + kh * G) * D / 8;
      for (int i = 0; i < G * D / 8; ++i) dst[i] = make_uint4(0, 0, 0, 0);
    }
  }

  if (aligned) {
    if (wg >= s_wstart[units]) return;
    // the unit owning workgroup wg: the last u with s_wstart[u] <= wg (units without slots share starts)
    int lo_u = 0, hi_u = units - 1;
    while (lo_u < hi_u) {
      const int mid = (lo_u + hi_u + 1) >> 1;
      if (s_wstart[mid] <= wg) lo_u = mid; else hi_u = mid - 1;
    }
    u = lo_u;
    const int k = wg - s_wstart[u], n = s_wstart[u + 1] - s_wstart[u];
    const int wu = s_start[u + 1] - s_start[u];
    a0 = s_start[u] + static_cast<int>(static_cast<int64_t>(k) * wu / n);
    a1 = s_start[u] + static_cast<int>(static_cast<int64_t>(k + 1) * wu / n);
  } else {
    a0 = wg * c;
    a1 = min(a0 + c, W);
    if (a0 >= a1) return;
    // unit holding slot a0: the last u with s_start[u] <= a0 (empty units share starts)
    int lo_u = 0, hi_u = units - 1;
    while (lo_u < hi_u) {
      const int mid = (lo_u + hi_u + 1) >> 1;
      if (s_start[mid] <= a0) lo_u = mid; else hi_u = mid - 1;
    }
    u = lo_u;
  }
  }
  bool first_seg = true;
  uint16_t* obase = static_cast<uint16_t*>(a.out);
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
  const int psh = g.Pshift, pmask = g.P - 1;

  while (a0 < a1) {
    const int ustart = use_plan ? 0 : s_start[u], uend = use_plan ? p_rows : s_start[u + 1];
    const int seg_end = min(a1, uend);
    const int lo = a0 - ustart, hi = seg_end - ustart;
    const int row = u / g.Hkv, kh = u % g.Hkv;
    const int seq = a.seq_ids ? a.seq_ids[row] : row;
    const int32_t* pt = d.page_table + (static_cast<int64_t>(seq) * g.Hkv + kh) * g.maxp;
    int vrow = -1, skip = -1;
    const uint8_t* kin = nullptr;
    const uint8_t* vin = nullptr;
    if constexpr (STEP) {
      const int ext = use_plan ? p_ext : lds.ext[u];
      if (ext >= 0) {
        vrow = uend - ustart - 1;
        skip = ext - 1;
      }
      // (the input rows are bf16: 2 bytes per element whatever the pages hold)
      const size_t ro = (static_cast<size_t>(row) * g.Hkv + kh) * (D * 2) + lane_col * (BPL * 2 / EB);
      kin = sa->k + ro;
      vin = sa->v + ro;
    }
    // fp8 pages: the current token's codes and scales as the append stores
    // them — in place or in the current page with that page's scales, in a
    // new page with scales from the row's own largest magnitudes
    uint4 vk[NV], vv[NV];
    float vsk = 1.0f, vsv = 1.0f;
    if constexpr (STEP && FP8) {
      static_assert(NV == 1 && BPL == 16, "fp8 step: 16 codes (32 input bytes) per lane");
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        vk[j] = make_uint4(0, 0, 0, 0);
        vv[j] = make_uint4(0, 0, 0, 0);
      }
      if (vrow >= 0) {
        const uint4 k0 = *reinterpret_cast<const uint4*>(kin), k1 = *reinterpret_cast<const uint4*>(kin + 16);
        const uint4 v0 = *reinterpret_cast<const uint4*>(vin), v1 = *reinterpret_cast<const uint4*>(vin + 16);
        const float mk = piece_row_max(fmaxf(piece_amax(k0, true), piece_amax(k1, true)), LPR);
        const float mv = piece_row_max(fmaxf(piece_amax(v0, true), piece_amax(v1, true)), LPR);
        const int L = uend - ustart - 1;
        if (skip < 0 && (L & pmask) == 0) {
          vsk = page_scale_from_amax(mk);
          vsv = page_scale_from_amax(mv);
        } else {
          const int page = use_plan ? p_spage
                                    : skip >= 0 ? pt[skip >> psh] : d.cur_page[static_cast<int64_t>(seq) * g.Hkv + kh];
          vsk = d.scales[2 * page];
          vsv = d.scales[2 * page + 1];
        }
        const float ik = 1.0f / vsk, iv = 1.0f / vsv;
        auto codes = [](const uint4& a, const uint4& b, float inv) {
          const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          uint32_t out[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t bits = w[2 * q + (e >> 1)];
              const float x = __uint_as_float((e & 1) ? (bits & 0xFFFF0000u) : (bits << 16));
              word |= static_cast<uint32_t>(f32_to_e4m3(x * inv)) << (8 * e);
            }
            out[q] = word;
          }
          return make_uint4(out[0], out[1], out[2], out[3]);
        };
        vk[0] = codes(k0, k1, ik);
        vv[0] = codes(v0, v1, iv);
      }
    }

    if constexpr (MF && FP8) {
      mf8_segment<G>(a, lds, pt, row, kh, lo, hi, wave, lane);
    } else if constexpr (MF) {
      mf_segment<D, G, STEP>(a, sa, lds, use_plan, p_np, p_page, pt, row, kh, lo, hi, vrow, skip, wave, lane);
    } else {
    uint32_t qv[G][QW];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint16_t* qp = qbase + (static_cast<size_t>(row) * g.Hq + kh * G + h) * D + lane_col * EPL;
#pragma unroll
      for (int j = 0; j < QW; j += 4) {
        const uint4 t4 = *reinterpret_cast<const uint4*>(qp + 2 * j);
        qv[h][j] = t4.x;
        qv[h][j + 1] = t4.y;
        qv[h][j + 2] = t4.z;
        qv[h][j + 3] = t4.w;
      }
    }
    // the decision neuron plays no part in attention (the commit zeroes it in memory)
    if (STEP && sa->qneuron && lane_col == LPR - 1) qv[0][QW - 1] &= 0xFFFFu;
    float m[G], l[G], o[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
    }
    // pages of the segment, up to 64 at a time (lane i holds page first + i);
    // chunks of NP passes are double-buffered: the loads of chunk i+1 are in
    // flight while chunk i is computed
    for (int pb = lo >> psh; pb <= (hi - 1) >> psh; pb += 64) {
      const int plast = min((hi - 1) >> psh, pb + 63);
      const bool from_plan = use_plan && p_np > 0;       // the range's pages (at most kRecMaxPages) are in the record
      const int pt_reg = from_plan ? (lane < p_np ? p_page : 0) : (pb + lane <= plast) ? pt[pb + lane] : 0;
      const int blo = max(lo, pb << psh), bhi = min(hi, (plast + 1) << psh);
      const int npass = (bhi - blo + RPP - 1) / RPP;
      // The next chunk's loads are issued before the current chunk's compute,
      // unconditionally and with no exit between them and their use (past
      // the end they reread a stand-in row, and a trailing chunk past the end
      // is computed fully masked): a load under a branch, or one that an exit
      // leaves unused, is waited for or moved down to its use by the compiler.
      // The scheduling barriers keep the written order: the counter of
      // outstanding loads drains in issue order, so a chunk issued ahead of
      // the one being waited for would be waited for too.
      KvChunk<NP, NV> ca, cb;
      auto load = [&](KvChunk<NP, NV>& ch, int pass0) {
        load_chunk<D, NP, FP8, LPR, STEP>(ch, d.k_pages, d.v_pages, d.scales, pt_reg, pb, blo, pass0, bhi, wave,
                                          lane_row, lane_col, psh, pmask, vrow, kin, vin);
      };
      auto compute = [&](const KvChunk<NP, NV>& ch, int pass0) {
        compute_chunk<D, G, NP, FP8, LPR, STEP>(ch, blo, pass0, bhi, wave, lane_row, g.scale_log2, qv, m, l, o, skip,
                                                vrow, vk, vv, vsk, vsv);
      };
      load(ca, 0);
      for (int p0 = 0; p0 < npass; p0 += 2 * NP) {
        __builtin_amdgcn_sched_barrier(0);
        load(cb, p0 + NP);
        __builtin_amdgcn_sched_barrier(0);
        compute(ca, p0);
        __builtin_amdgcn_sched_barrier(0);
        load(ca, p0 + 2 * NP);
        __builtin_amdgcn_sched_barrier(0);
        compute(cb, p0 + NP);
      }
    }
    // per-column sums over the wave's rows go through LDS: lanes of the first
    // 16-lane row group fold the other groups of their DPP row first
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] = fold_groups_sum<LPR>(l[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = fold_groups_sum<LPR>(o[h][e]);
    }
    const int drow = lane >> 4;                   // DPP row 0..3
    if ((lane & 15) < LPR) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) lds.o[wave][drow][h][lane_col * EPL + e] = o[h][e];
      }
      if (lane_col == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) lds.ml[wave][drow][h][1] = l[h];
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) lds.ml[wave][0][h][0] = m[h];
    }
    }
    __syncthreads();
    // the unit's workgroups w0..w1 (concatenated split: w0's record is its
    // second one when the unit starts inside w0's range)
    const int w0 = use_plan ? p_w0 : aligned ? s_wstart[u] : ustart / c;
    const int w1 = use_plan ? p_w1 : aligned ? s_wstart[u + 1] - 1 : (uend - 1) / c;
    const int odd = (!aligned && ustart != w0 * c) ? 1 : 0;
    const bool split = w1 > w0;
    const int rec = 2 * wg + (first_seg ? 0 : 1);
    for (int idx = tid; idx < G * D; idx += 256) {
      const int h = idx / D, dd = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, lds.ml[w][0][h][0]);
      float ov = 0.0f, lv = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float f = exp2f(lds.ml[w][0][h][0] - M);     // -inf gives 0
          if constexpr (MF) {
            // (one entry per wave)
            ov += f * lds.o[w][0][h][dd];
            lv += f * lds.ml[w][0][h][1];
          } else {
            ov += f * (lds.o[w][0][h][dd] + lds.o[w][1][h][dd] + lds.o[w][2][h][dd] + lds.o[w][3][h][dd]);
            lv += f * (lds.ml[w][0][h][1] + lds.ml[w][1][h][1] + lds.ml[w][2][h][1] + lds.ml[w][3][h][1]);
          }
        }
      }
      if (!split) {
        obase[(static_cast<size_t>(row) * g.Hq + kh * G + h) * D + dd] = f32_to_bf16(lv > 0.0f ? ov / lv : 0.0f);
      } else {
        // device-coherent stores (no L2 write-back of the XCD needed)
        float* pr = a.partials + (static_cast<int64_t>(rec) * G + h) * (D + 2);
        __hip_atomic_store(pr + dd, ov, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (dd == 0) {
          __hip_atomic_store(pr + D, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(pr + D + 1, lv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if (split) {
      // The last workgroup of the unit to finish combines its records.  The
      // records are written and read with device-scope (coherent across XCDs)
      // atomic stores and loads, so no fence has to write back or invalidate
      // an L2: each wave waits for its record stores to complete, then one
      // thread counts the arrival; the workgroup that brings the count to the
      // unit's number of workgroups merges and resets the counter for the
      // next call.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      int32_t* cnt = d.unit_info + 4 * u + 3;
      if (tid == 0) s_tmp[0] = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == w1 - w0;
      __syncthreads();
      if (s_tmp[0]) {
        merge_unit_records<D, G>(a.partials, w0, w1, odd, obase + (static_cast<size_t>(row) * g.Hq + kh * G) * D);
        if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (use_plan) break;
    first_seg = false;
    a0 = seg_end;
    ++u;
    while (u < units && s_start[u + 1] <= a0) ++u;
  }
}


template <int D, int G, int NP, bool FP8, int LPR, bool MF = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((MF && G <= 4) ? 2 : 1)))
void decode_attn_fast_kernel(DecodeArgs a) {
  __shared__ FastLds<G, D, false> lds;
  decode_attn_fast_body<D, G, NP, FP8, LPR, false, MF>(a, nullptr, blockIdx.x, gridDim.x, lds);
}

// The next step's plan, built by the committing workgroup once its commit's
// stores are complete: for each pair of this call, its rows at the next step
// (live slots after the commit plus the next token) and the next token's
// placement (in place over the slot of position t + 1 - w when that token was
// marked, else appended), split over the attention workgroups by the rule the
// attention uses, one record per workgroup.  Only when the next step can use
// it: every pair placed with room for one more token, no device error, units
// split one per workgroup, at most kPlanMaxWgs workgroups; else the plan is
// marked invalid.  Sequence ids of one call are distinct, so no unit has two
// pairs.
template <int D, int G, bool FP8, int LPR, bool MF>
__device__ void plan_build(const DecodeArgs& a, const StepArgs& sa, FastLds<G, D, true>& lds) {
  constexpr int RPP = MF ? 64 : 4 * (64 / LPR);     // as the attention's split
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x;
  const int units = sa.npairs, grid = sa.agrid;
  const int psh = g.Pshift, pmask = g.P - 1;
  int* s_start = lds.start;
  int* s_wstart = lds.wstart;
  int* s_tmp = lds.tmp;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const bool shape_ok = units <= kAlignedUnits && 2 * units <= grid && grid <= kPlanMaxWgs;
  int bad = shape_ok ? 0 : 1;
  if (tid == 0 && __hip_atomic_load(d.ctl + kCtlStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) bad = 1;
  // rows of the next step per pair (two per thread, as the attention's split scan)
  int rows[2] = {0, 0};
  if (shape_ok) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = 2 * tid + i;
      if (p >= units) continue;
      const int32_t* pl = d.chunk_info + static_cast<int64_t>(p) * 8;
      const int kind = __hip_atomic_load(pl + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int unit = __hip_atomic_load(pl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int t = __hip_atomic_load(pl + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int slot = __hip_atomic_load(pl + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int app = __hip_atomic_load(pl + 6, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int len = __hip_atomic_load(pl + 7, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int t1 = t + 1;
      if (kind == kPlanNone || t1 + 1 > g.max_tokens) bad = 1;
      int ext = 0;
      if (t1 >= g.w) {
        // position t + 1 - w: its ring entry predates this call
        const int rv = d.ring[static_cast<int64_t>(unit) * g.w + t1 % g.w];
        if (rv < 0) ext = (rv & 0x7FFFFFFF) + 1;
      }
      lds.ext[p] = ext;
      rows[i] = (app ? slot + 1 : len) + 1;
    }
  }
  if (__syncthreads_or(bad)) {
    if (tid == 0) plan_invalidate(d);
    return;
  }
  int W;
  int run = block_scan_256(rows[0] + rows[1], s_tmp, &W);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (2 * tid + i < units) s_start[2 * tid + i] = run;
    run += rows[i];
  }
  if (tid == 0) s_start[units] = W;
  __syncthreads();
  const int ca = max(1, (W + (grid - units) - 1) / (grid - units));
  int nw[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int wu = rows[i];
    if (2 * tid + i < units && wu > 0) nw[i] = min(min((wu + ca - 1) / ca, max(1, wu / RPP)), kMaxSplit);
  }
  int tot;
  run = block_scan_256(nw[0] + nw[1], s_tmp, &tot);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (2 * tid + i < units) s_wstart[2 * tid + i] = run;
    run += nw[i];
  }
  if (tid == 0) s_wstart[units] = tot;
  __syncthreads();
  int32_t* recs = plan_records(d, g);
  for (int j = tid; j < tot; j += 256) {
    int lo_u = 0, hi_u = units - 1;
    while (lo_u < hi_u) {
      const int mid = (lo_u + hi_u + 1) >> 1;
      if (s_wstart[mid] <= j) lo_u = mid; else hi_u = mid - 1;
    }
    const int u = lo_u;
    const int k = j - s_wstart[u], n = s_wstart[u + 1] - s_wstart[u];
    const int wu = s_start[u + 1] - s_start[u];
    const int lo = static_cast<int>(static_cast<int64_t>(k) * wu / n);
    const int hi = static_cast<int>(static_cast<int64_t>(k + 1) * wu / n);
    const int unit = __hip_atomic_load(d.chunk_info + static_cast<int64_t>(u) * 8 + 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    const int32_t* pt = d.page_table + static_cast<int64_t>(unit) * g.maxp;
    const int ext = lds.ext[u];
    int spage = -1;
    if (FP8) {
      // the page whose scales the next token takes (-1: it opens a page)
      if (ext > 0) spage = __hip_atomic_load(pt + ((ext - 1) >> psh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else if (((wu - 1) & pmask) != 0)
        spage = __hip_atomic_load(d.cur_page + unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int p0 = lo >> psh;
    int np = ((hi - 1) >> psh) - p0 + 1;
    if (np > kRecMaxPages) np = -1;
    int32_t* r = recs + static_cast<int64_t>(j) * kPlanRec;
    r[kRecUnit] = u;
    r[kRecLo] = lo;
    r[kRecHi] = hi;
    r[kRecRows] = wu;
    r[kRecExt] = ext;
    r[kRecW0] = s_wstart[u];
    r[kRecW1] = s_wstart[u + 1] - 1;
    r[kRecScalePage] = spage;
    r[kRecNpages] = np;
    for (int i = 0; i < np; ++i)
      r[kRecPages + i] = __hip_atomic_load(pt + p0 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int rr = tid; rr < a.B; rr += 256) plan_rows(d)[rr] = a.seq_ids ? a.seq_ids[rr] : rr;
  if (tid == 0) {
    d.plan[kPlanB] = a.B;
    d.plan[kPlanGrid] = grid;
    d.plan[kPlanSeqNull] = a.seq_ids == nullptr ? 1 : 0;
    d.plan[kPlanVariant] = plan_variant<D, G, FP8, LPR, MF>();
    d.plan[kPlanNrec] = tot;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) d.plan[kPlanValid] = 1;
}

// dms_decode_step: workgroups [0, npairs) prepare the current token of one
// (row, KV head) pair each (decision, placement, plan record); the others run
// the attention (STEP).  The last pair to finish waits until every attention
// workgroup has arrived (read the tables it works from), then commits.
// (the matrix-core variant for groups of up to 4 heads is built for 2 waves
// per SIMD, i.e. two workgroups per CU: the one-launch step needs its prepare
// and attention workgroups resident together, and the launch shape asks for
// exactly two per CU; at 3 the register cap leaves one tile fewer in flight)
// Workgroup wg of one step (the body of the kernel below, and of each layer
// of the persistent kernel after it).
template <int D, int G, int NP, bool FP8, int LPR, bool MF>
__device__ __forceinline__ void step_body(const DecodeArgs& a, const AppendArgs& ap, const PrepIn& pin,
                                          const StepArgs& sa, int wg, FastLds<G, D, true>& lds) {
  constexpr int KV = FP8 ? DMS_FP8_E4M3 : DMS_BF16;
  if (wg < sa.nprep) {
    PrepShared& sh = lds.prep;
    if (sa.per_row) prep_row<KV>(ap, pin, wg, sh);
    else prep_pair<KV>(ap, pin, wg, true, sh);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) sh.last = prep_arrive(ap.d, wg, sa.nprep);
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(sh.last)) return;
    // the last pair commits once every attention workgroup has arrived: lane
    // i of wave 0 polls group i (bounded; all of them are normally resident
    // and arrive within their first microseconds)
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
      bool ok = true;
      if (lane < sa.groups) {
        const int want = sa.agrid / sa.groups + (lane < sa.agrid % sa.groups ? 1 : 0);
        const int32_t* gc = ap.d.arrive + lane * kArriveStride;
        for (int it = 0;; ++it) {
          if (it >= sa.spin_limit) {
            ok = false;
            break;
          }
          if (__hip_atomic_load(gc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) break;
          __builtin_amdgcn_s_sleep(2);
        }
      }
      const bool all = __all(ok);
      if (lane == 0) sh.n = all ? 1 : 0;
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(sh.n)) {
      // no commit: the tables are as before the call (the pairs wrote only
      // their K/V rows and slot metadata); the arrival counters are reset by
      // dms_cache_clear_status, once every workgroup of this launch is done
      if (threadIdx.x == 0) set_status(ap.d.ctl, DMS_DEV_STEP_SYNC);
      return;
    }
    prep_commit<KV>(ap, pin, sa.npairs, sh);
    plan_build<D, G, FP8, LPR, MF>(a, sa, lds);
    if (threadIdx.x < sa.groups)
      __hip_atomic_store(ap.d.arrive + threadIdx.x * kArriveStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prep_arrive_reset(ap.d, sa.nprep, threadIdx.x);
    return;
  }
  decode_attn_fast_body<D, G, NP, FP8, LPR, true, MF>(a, &sa, wg - sa.nprep, sa.agrid, lds);
}

template <int D, int G, int NP, bool FP8, int LPR, bool MF = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((MF && G <= 4) ? 2 : 1)))
void decode_step_kernel(DecodeArgs a, AppendArgs ap, PrepIn pin, StepArgs sa) {
  __shared__ FastLds<G, D, true> lds;
  step_body<D, G, NP, FP8, LPR, MF>(a, ap, pin, sa, blockIdx.x, lds);
}

// The decode step of every layer of a model in one launch (dms_step_layers_run).
// Layer l is the step above on layer l's cache, with layer l's inputs and
// outputs; a grid-wide barrier between layers lets layer l+1 start only once
// every attention workgroup of layer l has written its outputs (in a model,
// layer l+1's inputs are computed from them), which also frees the shared
// workspace's partial records for the next layer.  The prepare role of a
// layer's last pair commits that layer while the others go on.  All
// workgroups are resident (checked at launch); each wait is bounded.
struct LayerDesc {
  DecodeArgs a;                 // seq_ids, B and partials are the call's
  AppendArgs ap;                // seq_ids and B are the call's
  PrepIn pin;
  const uint8_t* k;             // [B][Hkv][D] rows of the current token
  const uint8_t* v;
};
struct LayersRun {
  const int32_t* seq_ids;
  int B;
  float* partials;              // caller's workspace, shared by the layers
  StepArgs sa;                  // k and v are each layer's
  int32_t* bar;                 // kBarInts counters (layout below), zero between launches
  int n_layers;
  int nwg;
};

// The layer barrier's counters, each on a 256-byte line of its own: the
// attention workgroups arrive in kBarGroups groups (attention index mod the
// group count); the last of a group adds to the count of complete groups, and
// the last group's last workgroup raises every group's release flag to the
// number of layers passed.  Every workgroup polls the flag of its own group,
// so no line takes more than a group's adds or polls (one counter taking
// every add while every workgroup polled it cost 14 us per layer).
constexpr int kBarGroups = 32;
constexpr int kBarStride = 64;
constexpr int kBarTop = kBarGroups * kBarStride;
constexpr int kBarFlag0 = kBarTop + kBarStride;
constexpr int kBarEnd = kBarFlag0 + kBarGroups * kBarStride;
constexpr int kBarInts = kBarEnd + kBarStride;

template <int D, int G, int NP, bool FP8, int LPR, bool MF = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((MF && G <= 4) ? 2 : 1)))
void decode_layers_kernel(const LayerDesc* __restrict__ desc, LayersRun r) {
  __shared__ FastLds<G, D, true> lds;
  const int wg = blockIdx.x;
  const bool attn = wg >= r.sa.nprep;
  const int ng = min(kBarGroups, r.sa.agrid);
  for (int l = 0; l < r.n_layers; ++l) {
    DecodeArgs a = desc[l].a;
    a.seq_ids = r.seq_ids;
    a.B = r.B;
    a.partials = r.partials;
    AppendArgs ap = desc[l].ap;
    ap.seq_ids = r.seq_ids;
    ap.B = r.B;
    const PrepIn pin = desc[l].pin;
    StepArgs sa = r.sa;
    sa.k = desc[l].k;
    sa.v = desc[l].v;
    step_body<D, G, NP, FP8, LPR, MF>(a, ap, pin, sa, wg, lds);
    if (l + 1 == r.n_layers) break;
    // layer barrier: attention workgroups arrive once their outputs (and,
    // for a unit's last one, the merge) are written: every thread's stores
    // acknowledged, then relaxed atomics.  No fence: nothing after the
    // barrier reads what layer l wrote (the shared workspace's records are
    // only overwritten, and their readers consumed them before arriving),
    // and an agent-scope fence writes back the XCD's L2 on every workgroup
    // (measured: a layer step of 73-79 us instead of 12-20).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      if (attn) {
        const int ai = wg - sa.nprep, gi = ai % ng;
        const int n_g = sa.agrid / ng + (gi < sa.agrid % ng ? 1 : 0);
        if (__hip_atomic_fetch_add(r.bar + gi * kBarStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (l + 1) * n_g - 1 &&
            __hip_atomic_fetch_add(r.bar + kBarTop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (l + 1) * ng - 1) {
          for (int k = 0; k < ng; ++k)
            __hip_atomic_store(r.bar + kBarFlag0 + k * kBarStride, l + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      const int32_t* flag = r.bar + kBarFlag0 + (wg % ng) * kBarStride;
      for (int it = 0;; ++it) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) > l) break;
        if (it >= sa.spin_limit) {
          set_status(a.d.ctl, DMS_DEV_STEP_SYNC);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
  }
  // every workgroup is past its last wait: the last one to finish clears the
  // counters for the next launch
  __syncthreads();
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(r.bar + kBarEnd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == r.nwg - 1) {
    for (int k = 0; k < kBarInts; k += kBarStride)
      __hip_atomic_store(r.bar + k, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int D, int G, bool FP8, int NP>
static void launch_fast_np(const DecodeArgs& a, int grid, hipStream_t st) {
  // default: one 16-byte piece per lane (LPR = row bytes / 16, at most 16);
  // DMS_DECODE_LPR=8 selects 32 bytes per lane for 256-byte rows
  constexpr int RB = D * (FP8 ? 1 : 2);
  constexpr int LPR1 = RB / 16 >= 16 ? 16 : RB / 16;
  if constexpr (RB / 16 >= 16) {
    if (a.lanes_per_row == 8) {
      hipLaunchKernelGGL((decode_attn_fast_kernel<D, G, NP, FP8, 8>), dim3(grid), dim3(256), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((decode_attn_fast_kernel<D, G, NP, FP8, LPR1>), dim3(grid), dim3(256), 0, st, a);
}

template <int D, int G, bool FP8>
static int launch_fast_dg(const DecodeArgs& a, int grid, int np, hipStream_t st) {
  if constexpr (!FP8) {
    if (a.mfma) {
      constexpr int LPR1 = D * 2 / 16 >= 16 ? 16 : D * 2 / 16;
      hipLaunchKernelGGL((decode_attn_fast_kernel<D, G, 2, false, LPR1, true>), dim3(grid), dim3(256), 0, st, a);
      return DMS_OK;
    }
  } else if constexpr (D == 128) {
    if (a.mfma) {
      hipLaunchKernelGGL((decode_attn_fast_kernel<128, G, 2, true, 8, true>), dim3(grid), dim3(256), 0, st, a);
      return DMS_OK;
    }
  }
  switch (np) {
    case 2: launch_fast_np<D, G, FP8, 2>(a, grid, st); break;
    case 4: launch_fast_np<D, G, FP8, 4>(a, grid, st); break;
    case 6: launch_fast_np<D, G, FP8, 6>(a, grid, st); break;
    default: launch_fast_np<D, G, FP8, 8>(a, grid, st); break;
  }
  return DMS_OK;
}

template <int D, bool FP8>
static int launch_fast_d(const DecodeArgs& a, int grid, int np, hipStream_t st) {
  switch (a.g.g) {
    case 1: return launch_fast_dg<D, 1, FP8>(a, grid, np, st);
    case 2: return launch_fast_dg<D, 2, FP8>(a, grid, np, st);
    case 4: return launch_fast_dg<D, 4, FP8>(a, grid, np, st);
    case 8: return launch_fast_dg<D, 8, FP8>(a, grid, np, st);
    default: return fail(DMS_ERR_UNSUPPORTED, "group size");
  }
}

template <typename ACT, int KV, int D, int G>
static int launch_decode_dg(const DecodeArgs& a, int grid, hipStream_t st) {
  constexpr int NP = 4;
  hipLaunchKernelGGL((decode_attn_kernel<ACT, KV, D, G, NP>), dim3(grid), dim3(256), 0, st, a);
  hipLaunchKernelGGL((decode_combine_kernel<ACT, D, G>), dim3(a.B * a.g.Hkv), dim3(256), 0, st, a);
  return DMS_OK;
}

template <typename ACT, int KV, int D>
static int launch_decode_d(const DecodeArgs& a, int grid, hipStream_t st) {
  switch (a.g.g) {
    case 1: return launch_decode_dg<ACT, KV, D, 1>(a, grid, st);
    case 2: return launch_decode_dg<ACT, KV, D, 2>(a, grid, st);
    case 4: return launch_decode_dg<ACT, KV, D, 4>(a, grid, st);
    case 8: return launch_decode_dg<ACT, KV, D, 8>(a, grid, st);
    default: return fail(DMS_ERR_UNSUPPORTED, "group size");
  }
}

template <typename ACT, int KV>
static int launch_decode(const DecodeArgs& a, int grid, hipStream_t st) {
  switch (a.g.D) {
    case 32: return launch_decode_d<ACT, KV, 32>(a, grid, st);
    case 64: return launch_decode_d<ACT, KV, 64>(a, grid, st);
    case 128: return launch_decode_d<ACT, KV, 128>(a, grid, st);
    default: return fail(DMS_ERR_UNSUPPORTED, "head_dim");
  }
}

// The one-launch step kernel of a cache's shape: fp8 rows of D bytes take
// 16 bytes (16 codes) per lane; bf16 rows 16 lanes per row of 128 (8 on request).
using StepKernel = void (*)(DecodeArgs, AppendArgs, PrepIn, StepArgs);

template <int D, int G>
static StepKernel step_kernel_dg(const Geo& g, int lanes_per_row, bool mfma) {
  if (g.kv_dtype == DMS_FP8_E4M3) return decode_step_kernel<D, G, 2, true, D / 16>;
  constexpr int RB = D * 2;
  constexpr int LPR1 = RB / 16 >= 16 ? 16 : RB / 16;
  if (mfma) return decode_step_kernel<D, G, 2, false, LPR1, true>;
  if constexpr (RB / 16 >= 16) {
    if (lanes_per_row == 8) return decode_step_kernel<D, G, 2, false, 8>;
  }
  return decode_step_kernel<D, G, 2, false, LPR1>;
}

template <int D>
static StepKernel step_kernel_d(const Geo& g, int lanes_per_row, bool mfma) {
  switch (g.g) {
    case 1: return step_kernel_dg<D, 1>(g, lanes_per_row, mfma);
    case 2: return step_kernel_dg<D, 2>(g, lanes_per_row, mfma);
    case 4: return step_kernel_dg<D, 4>(g, lanes_per_row, mfma);
    case 8: return step_kernel_dg<D, 8>(g, lanes_per_row, mfma);
    default: return nullptr;
  }
}

static StepKernel step_kernel(const Geo& g, int lanes_per_row, bool mfma) {
  return g.D == 128 ? step_kernel_d<128>(g, lanes_per_row, mfma) : step_kernel_d<64>(g, lanes_per_row, mfma);
}

// The fast decode attention applies: bf16/fp8 pages, D 64/128, power-of-two
// pages holding at least the 64 / lanes-per-row rows a wave reads per pass
// (so they span at most two pages), page bytes addressable in 32 bits.
static bool fast_decode_ok(const dms_cache* cache, int* lpr_out) {
  const Geo& g = cache->geo;
  const int row_bytes = g.D * (g.kv_dtype == DMS_FP8_E4M3 ? 1 : 2);
  const int lpr = row_bytes / 16 >= 16 ? (cache->decode_lpr == 8 ? 8 : 16) : row_bytes / 16;
  if (lpr_out) *lpr_out = lpr;
  return (g.kv_dtype == DMS_BF16 || g.kv_dtype == DMS_FP8_E4M3) && (g.D == 64 || g.D == 128) && g.Pshift >= 0 &&
         (1 << g.Pshift) >= 64 / lpr && cache->layout.v_pages - cache->layout.k_pages < (1ull << 32) &&
         !cache->force_generic;
}

// The matrix-core variant applies to the fast kernel's bf16 pages of at least
// 16 rows (a 16-row tile lies in one page); DMS_DECODE_MFMA=0 turns it off.
static bool mfma_decode_ok(const dms_cache* cache) {
  const Geo& g = cache->geo;
  return cache->decode_mfma != 0 && g.kv_dtype == DMS_BF16 && g.Pshift >= 4 && fast_decode_ok(cache, nullptr);
}
// dms_decode_attn also takes it for fp8 pages of head_dim 128 (the one-launch
// step keeps fp8 pages on the lane-per-row-piece kernel).
static bool mfma_attn_ok(const dms_cache* cache) {
  const Geo& g = cache->geo;
  return mfma_decode_ok(cache) || (cache->decode_mfma != 0 && g.kv_dtype == DMS_FP8_E4M3 && g.D == 128 &&
                                   g.Pshift >= 4 && fast_decode_ok(cache, nullptr));
}

// ---- decode attention without an allocation ------------------------------
// For callers that cannot allocate (code under HIP graph capture, serving
// loops that must not call hipMalloc): dms_decode_attn_noalloc runs the same
// kernels with their partial records in this file-scope device array, of
// which each GPU holds its own copy for the life of the process.  Nothing in
// it has to start at zero (every record is written before it is read within
// a call).  Its device address is looked up once per device and kept; host
// code passes that address, never the array's name.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxScratchDevices];

// The scratch array's address on device `dev` (which must be current).
static int noalloc_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(DMS_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const int s = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (s) return s;
    if (!p) return fail(DMS_ERR_HIP, "hipGetSymbolAddress(scratch) returned no address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DMS_OK;
}

}  // namespace dms

using namespace dms;

// Checks the caller's decode workspace against what a call of B rows needs.
static int check_workspace(const dms_cache* cache, int B, const void* workspace, size_t ws_bytes) {
  const Geo& g = cache->geo;
  const size_t need = decode_workspace_bytes(decode_grid_for(cache), B * g.Hkv, g.g, g.D);
  if (!workspace || ws_bytes < need)
    return fail(DMS_ERR_CAPACITY, "decode workspace missing or smaller than dms_decode_workspace_bytes (" +
                                      std::to_string(need) + " bytes)");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(DMS_ERR_ARG, "decode workspace must be 256-byte aligned");
  return DMS_OK;
}

extern "C" int dms_decode_attn(dms_cache* cache, const int32_t* seq_ids, const void* q, void* out, int B,
                               void* workspace, size_t ws_bytes, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  if (!q || !out) return fail(DMS_ERR_ARG, "q and out are required");
  const Geo& g = cache->geo;
  if (B <= 0) return fail(DMS_ERR_ARG, "B must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  int s = check_workspace(cache, B, workspace, ws_bytes);
  if (s) return s;
  DecodeArgs a{cache->dev, g, seq_ids, q, out, B, cache->decode_lpr, static_cast<float*>(workspace),
               mfma_attn_ok(cache) ? cache->decode_mfma : 0};
  const int grid = decode_grid_call(cache, B * g.Hkv);
  hipStream_t st = as_stream(stream);
  // the fast kernels read q and write out in 16-byte pieces
  const bool aligned16 = (reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) % 16 == 0;
  if (fast_decode_ok(cache, nullptr) && aligned16) {
    const bool fp8 = g.kv_dtype == DMS_FP8_E4M3;
    const int np = cache->decode_np > 0 ? cache->decode_np : 2;
    if (g.D == 128) s = fp8 ? launch_fast_d<128, true>(a, grid, np, st) : launch_fast_d<128, false>(a, grid, np, st);
    else s = fp8 ? launch_fast_d<64, true>(a, grid, np, st) : launch_fast_d<64, false>(a, grid, np, st);
  } else {
    switch (g.kv_dtype) {
      case DMS_F32: s = launch_decode<float, DMS_F32>(a, grid, st); break;
      case DMS_BF16: s = launch_decode<uint16_t, DMS_BF16>(a, grid, st); break;
      case DMS_FP8_E4M3: s = launch_decode<uint16_t, DMS_FP8_E4M3>(a, grid, st); break;
      default: return fail(DMS_ERR_UNSUPPORTED, "kv dtype");
    }
  }
  if (s) return s;
  return check_hip(hipGetLastError(), "dms_decode_attn launch");
}

extern "C" int dms_decode_step(dms_cache* cache, const int32_t* seq_ids, const void* hidden, const float* rms_gamma,
                               const float* W, const float* bias, const float* offsets, void* q_inout, const void* k,
                               const void* v, void* out, int B, float* logits_out, uint8_t* evict_out,
                               void* workspace, size_t ws_bytes, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  const dms_config& c = cache->cfg;
  const Geo& g = cache->geo;
  if (!q_inout || !out || !k || !v || !offsets || !evict_out)
    return fail(DMS_ERR_ARG, "q_inout, out, k, v, offsets and evict_out are required");
  if (B <= 0) return fail(DMS_ERR_ARG, "B must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  if (int s = check_workspace(cache, B, workspace, ws_bytes)) return s;
  const bool linear = c.decide_mode == DMS_DECIDE_LINEAR;
  if (linear && (!hidden || !rms_gamma || !W)) return fail(DMS_ERR_ARG, "hidden, rms_gamma and W are required");
  uintptr_t al = reinterpret_cast<uintptr_t>(q_inout) | reinterpret_cast<uintptr_t>(k) |
                 reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if (linear)
    al |= reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(rms_gamma) |
          reinterpret_cast<uintptr_t>(W);
  const int npairs = B * g.Hkv;
  // the attention workgroups fill what the prepare workgroups leave of the
  // decode grid (two workgroups per CU by default), so that no CU holds a
  // third workgroup beside two attention ones
  const int dgrid = decode_grid_call(cache, npairs);
  auto attn_grid = [&](int nprep) { return std::max(dgrid / 2, dgrid - nprep); };
  int nprep = npairs;
  bool per_row = false;
  int agrid = attn_grid(nprep);
  bool fused = cache->step_fuse != 0 && fast_decode_ok(cache, nullptr) && al % 16 == 0 &&
               (!linear || c.hidden % 8 == 0) && npairs <= kMaxUnits;
  StepKernel kern = fused ? step_kernel(g, cache->decode_lpr, mfma_decode_ok(cache)) : nullptr;
  if (!kern) fused = false;
  if (fused && cache->step_fuse < 0) {
    // One launch only when every workgroup can be resident at once: else the
    // attention workgroups wait for whole prepare workgroups to leave, and
    // the two calls in turn are faster.
    if (cache->step_blocks_per_cu < 0) {
      int n = 0;
      if (check_hip(hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kern), 256, 0),
                    "step kernel occupancy"))
        return DMS_ERR_HIP;
      cache->step_blocks_per_cu = n;
    }
  }
  // DMS_DECODE_STEP_ROWS=1 (read at every call): one prepare workgroup per
  // batch row instead of one per pair.  It lets a large batch run in one
  // launch, but with the attention a grid of pairs smaller; for fp8 pages at
  // 64 rows the two calls in turn are faster, so it is not the default.
  if (const char* e = std::getenv("DMS_DECODE_STEP_ROWS")) per_row = std::atoi(e) != 0 && g.Hkv > 1;
  if (per_row) {
    nprep = B;
    agrid = attn_grid(B);
  }
  if (fused && cache->step_fuse < 0) fused = nprep + agrid <= cache->step_blocks_per_cu * cache->num_cus;
  hipStream_t st = as_stream(stream);
  if (!fused) {
    // other shapes, or a step too large for one resident launch: the two calls in turn
    int s = dms_decode_prepare(cache, seq_ids, hidden, rms_gamma, W, bias, offsets, q_inout, k, v, B, logits_out,
                               evict_out, stream);
    if (s) return s;
    return dms_decode_attn(cache, seq_ids, q_inout, out, B, workspace, ws_bytes, stream);
  }
  DecodeArgs a{cache->dev, g, seq_ids, q_inout, out, B, cache->decode_lpr, static_cast<float*>(workspace),
               mfma_decode_ok(cache) ? cache->decode_mfma : 0};
  AppendArgs ap{};
  ap.d = cache->dev;
  ap.g = g;
  ap.seq_ids = seq_ids;
  ap.k = k;
  ap.v = v;
  ap.evict = nullptr;
  ap.B = B;
  ap.T = 1;
  ap.bias = bias;
  ap.offsets = offsets;
  ap.alpha = c.alpha_scale;
  ap.eps = c.rms_eps;
  ap.per_layer = c.alpha_per == DMS_ALPHA_PER_LAYER;
  ap.disable = c.disable_eviction != 0;
  ap.logits_out = logits_out;
  ap.evict_out = evict_out;
  PrepIn pin{static_cast<const uint16_t*>(hidden), rms_gamma, W, static_cast<uint16_t*>(q_inout), linear ? 0 : 1};
  const int groups = std::min(kArriveGroups, agrid);
  // DMS_STEP_SPIN_LIMIT (read at every call): the commit's bounded wait, in
  // polls; 0 makes it give up at once (a host-side way to exercise the
  // DMS_DEV_STEP_SYNC path with every kernel exiting normally)
  int spin = kArriveSpinLimit;
  if (const char* e = std::getenv("DMS_STEP_SPIN_LIMIT")) spin = std::max(0, std::atoi(e));
  StepArgs sa{static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), npairs, nprep, per_row ? 1 : 0, groups, agrid,
              linear ? 0 : 1, spin};
  hipLaunchKernelGGL(kern, dim3(nprep + agrid), dim3(256), 0, st, a, ap, pin, sa);
  return check_hip(hipGetLastError(), "dms_decode_step launch");
}

namespace dms {

// The persistent kernel of a cache's shape (the variants of step_kernel).
using LayersKernel = void (*)(const LayerDesc*, LayersRun);

template <int D, int G>
static LayersKernel layers_kernel_dg(const Geo& g, int lanes_per_row, bool mfma) {
  if (g.kv_dtype == DMS_FP8_E4M3) return decode_layers_kernel<D, G, 2, true, D / 16>;
  constexpr int RB = D * 2;
  constexpr int LPR1 = RB / 16 >= 16 ? 16 : RB / 16;
  if (mfma) return decode_layers_kernel<D, G, 2, false, LPR1, true>;
  if constexpr (RB / 16 >= 16) {
    if (lanes_per_row == 8) return decode_layers_kernel<D, G, 2, false, 8>;
  }
  return decode_layers_kernel<D, G, 2, false, LPR1>;
}

template <int D>
static LayersKernel layers_kernel_d(const Geo& g, int lanes_per_row, bool mfma) {
  switch (g.g) {
    case 1: return layers_kernel_dg<D, 1>(g, lanes_per_row, mfma);
    case 2: return layers_kernel_dg<D, 2>(g, lanes_per_row, mfma);
    case 4: return layers_kernel_dg<D, 4>(g, lanes_per_row, mfma);
    case 8: return layers_kernel_dg<D, 8>(g, lanes_per_row, mfma);
    default: return nullptr;
  }
}

}  // namespace dms

struct dms_step_layers {
  std::vector<dms_cache*> caches;
  std::vector<dms_layer_io> io;
  int device = -1;
  dms::LayersKernel kern = nullptr;   // null: the layers run as one dms_decode_step each
  int blocks_per_cu = 0;
  dms::LayerDesc* desc = nullptr;     // [n_layers] device
  int32_t* bar = nullptr;             // [kBarInts] device, zero between launches
};

namespace dms {

static bool same_shape(const dms_cache* a, const dms_cache* b) {
  const Geo &x = a->geo, &y = b->geo;
  return x.Bmax == y.Bmax && x.Hq == y.Hq && x.Hkv == y.Hkv && x.D == y.D && x.H == y.H && x.w == y.w &&
         x.P == y.P && x.kv_dtype == y.kv_dtype && a->cfg.decide_mode == b->cfg.decide_mode &&
         a->device == b->device && a->decode_lpr == b->decode_lpr && a->decode_mfma == b->decode_mfma &&
         a->decode_grid == b->decode_grid && a->step_fuse == b->step_fuse;
}

static int layers_fallback(dms_step_layers* p, const int32_t* seq_ids, int B, void* ws, size_t ws_bytes, void* stream) {
  for (size_t l = 0; l < p->caches.size(); ++l) {
    const dms_layer_io& o = p->io[l];
    int s = dms_decode_step(p->caches[l], seq_ids, o.hidden, o.rms_gamma, o.W, o.bias, o.offsets, o.q_inout, o.k, o.v,
                            o.out, B, o.logits_out, o.evict_out, ws, ws_bytes, stream);
    if (s) return s;
  }
  return DMS_OK;
}

}  // namespace dms

extern "C" int dms_step_layers_create(dms_cache* const* caches, const dms_layer_io* io, int n_layers,
                                      dms_step_layers** out) {
  if (!out) return fail(DMS_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!caches || !io) return fail(DMS_ERR_ARG, "caches and io are required");
  if (n_layers <= 0 || n_layers > kMaxStepLayers)
    return fail(DMS_ERR_ARG, "n_layers must be in 1.." + std::to_string(kMaxStepLayers));
  for (int l = 0; l < n_layers; ++l) {
    if (!caches[l]) return fail(DMS_ERR_ARG, "cache " + std::to_string(l) + " is NULL");
    if (!same_shape(caches[0], caches[l]))
      return fail(DMS_ERR_ARG, "cache " + std::to_string(l) + " differs from cache 0 in shape, mode or device");
    for (int j = 0; j < l; ++j)
      if (caches[j] == caches[l]) return fail(DMS_ERR_ARG, "a cache appears twice");
    const dms_layer_io& o = io[l];
    if (!o.q_inout || !o.out || !o.k || !o.v || !o.offsets || !o.evict_out)
      return fail(DMS_ERR_ARG, "layer " + std::to_string(l) + ": q_inout, out, k, v, offsets and evict_out are required");
    if (caches[0]->cfg.decide_mode == DMS_DECIDE_LINEAR && (!o.hidden || !o.rms_gamma || !o.W))
      return fail(DMS_ERR_ARG, "layer " + std::to_string(l) + ": hidden, rms_gamma and W are required");
  }
  dms_cache* c0 = caches[0];
  const Geo& g = c0->geo;
  const bool linear = c0->cfg.decide_mode == DMS_DECIDE_LINEAR;
  // one launch needs the one-launch step's conditions in every layer
  bool fused = c0->step_fuse != 0 && fast_decode_ok(c0, nullptr) && (!linear || c0->cfg.hidden % 8 == 0);
  for (int l = 0; l < n_layers && fused; ++l) {
    const dms_layer_io& o = io[l];
    uintptr_t al = reinterpret_cast<uintptr_t>(o.q_inout) | reinterpret_cast<uintptr_t>(o.k) |
                   reinterpret_cast<uintptr_t>(o.v) | reinterpret_cast<uintptr_t>(o.out);
    if (linear)
      al |= reinterpret_cast<uintptr_t>(o.hidden) | reinterpret_cast<uintptr_t>(o.rms_gamma) |
            reinterpret_cast<uintptr_t>(o.W);
    if (al % 16) fused = false;
  }
  std::unique_ptr<dms_step_layers> p(new dms_step_layers());
  p->caches.assign(caches, caches + n_layers);
  p->io.assign(io, io + n_layers);
  p->device = c0->device;
  if (fused) {
    p->kern = g.D == 128 ? layers_kernel_d<128>(g, c0->decode_lpr, mfma_decode_ok(c0))
                         : layers_kernel_d<64>(g, c0->decode_lpr, mfma_decode_ok(c0));
  }
  if (p->kern) {
    int dev = -1;
    if (int s = check_hip(hipGetDevice(&dev), "hipGetDevice")) return s;
    if (dev != c0->device) return fail(DMS_ERR_ARG, "the caches' device must be the current device");
    if (int s = check_hip(hipOccupancyMaxActiveBlocksPerMultiprocessor(&p->blocks_per_cu,
                                                                        reinterpret_cast<const void*>(p->kern), 256, 0),
                          "layers kernel occupancy"))
      return s;
    std::vector<LayerDesc> h(n_layers);
    for (int l = 0; l < n_layers; ++l) {
      const dms_cache* c = caches[l];
      const dms_layer_io& o = io[l];
      LayerDesc& L = h[l];
      L.a = DecodeArgs{c->dev, c->geo, nullptr, o.q_inout, o.out, 0, c->decode_lpr, nullptr,
                       mfma_decode_ok(c) ? c->decode_mfma : 0};
      L.ap = AppendArgs{};
      L.ap.d = c->dev;
      L.ap.g = c->geo;
      L.ap.k = o.k;
      L.ap.v = o.v;
      L.ap.T = 1;
      L.ap.bias = o.bias;
      L.ap.offsets = o.offsets;
      L.ap.alpha = c->cfg.alpha_scale;
      L.ap.eps = c->cfg.rms_eps;
      L.ap.per_layer = c->cfg.alpha_per == DMS_ALPHA_PER_LAYER;
      L.ap.disable = c->cfg.disable_eviction != 0;
      L.ap.logits_out = o.logits_out;
      L.ap.evict_out = o.evict_out;
      L.pin = PrepIn{static_cast<const uint16_t*>(o.hidden), o.rms_gamma, o.W, static_cast<uint16_t*>(o.q_inout),
                     linear ? 0 : 1};
      L.k = static_cast<const uint8_t*>(o.k);
      L.v = static_cast<const uint8_t*>(o.v);
    }
    void* d = nullptr;
    const size_t bar_off = (sizeof(LayerDesc) * n_layers + 255) / 256 * 256;
    const size_t bar_bytes = sizeof(int32_t) * kBarInts;
    if (int s = check_hip(hipMalloc(&d, bar_off + bar_bytes), "hipMalloc (layer descriptors)")) return s;
    p->desc = static_cast<LayerDesc*>(d);
    p->bar = reinterpret_cast<int32_t*>(static_cast<char*>(d) + bar_off);
    int s = check_hip(hipMemcpy(p->desc, h.data(), sizeof(LayerDesc) * n_layers, hipMemcpyHostToDevice),
                      "hipMemcpy (layer descriptors)");
    if (!s) s = check_hip(hipMemset(p->bar, 0, bar_bytes), "hipMemset (layer barrier)");
    if (s) {
      hipFree(d);
      return s;
    }
  }
  *out = p.release();
  return DMS_OK;
}

extern "C" int dms_step_layers_run(dms_step_layers* p, const int32_t* seq_ids, int B, void* workspace,
                                   size_t ws_bytes, void* stream) {
  if (!p) return fail(DMS_ERR_ARG, "layers is NULL");
  dms_cache* c0 = p->caches[0];
  const Geo& g = c0->geo;
  if (B <= 0) return fail(DMS_ERR_ARG, "B must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  if (int s = check_workspace(c0, B, workspace, ws_bytes)) return s;
  const int npairs = B * g.Hkv;
  // the full grid: with one workgroup per CU the layer barrier's waits grew
  // (24.3 against 21.5 us per Qwen3-8B layer step at B 8)
  const int dgrid = decode_grid_for(c0);
  const int agrid = std::max(dgrid / 2, dgrid - npairs);
  const int nwg = npairs + agrid;
  if (!p->kern || npairs > kMaxUnits || nwg > p->blocks_per_cu * c0->num_cus)
    return layers_fallback(p, seq_ids, B, workspace, ws_bytes, stream);
  int spin = kArriveSpinLimit;
  if (const char* e = std::getenv("DMS_STEP_SPIN_LIMIT")) spin = std::max(0, std::atoi(e));
  LayersRun r{};
  r.seq_ids = seq_ids;
  r.B = B;
  r.partials = static_cast<float*>(workspace);
  r.sa = StepArgs{nullptr, nullptr, npairs, npairs, 0, std::min(kArriveGroups, agrid), agrid,
                  c0->cfg.decide_mode == DMS_DECIDE_LINEAR ? 0 : 1, spin};
  r.bar = p->bar;
  r.n_layers = static_cast<int>(p->caches.size());
  r.nwg = nwg;
  hipLaunchKernelGGL(p->kern, dim3(nwg), dim3(256), 0, as_stream(stream), p->desc, r);
  return check_hip(hipGetLastError(), "dms_step_layers_run launch");
}

extern "C" int dms_step_layers_one_launch(const dms_step_layers* p, int B, int32_t* one_launch) {
  if (!p || !one_launch) return fail(DMS_ERR_ARG, "layers and one_launch are required");
  const dms_cache* c0 = p->caches[0];
  const int npairs = B * c0->geo.Hkv;
  const int dgrid = decode_grid_for(c0);
  const int nwg = npairs + std::max(dgrid / 2, dgrid - npairs);
  *one_launch = (p->kern && B > 0 && B <= c0->geo.Bmax && npairs <= kMaxUnits &&
                 nwg <= p->blocks_per_cu * c0->num_cus)
                    ? 1
                    : 0;
  return DMS_OK;
}

extern "C" int dms_step_layers_destroy(dms_step_layers* p) {
  if (!p) return DMS_OK;
  int s = DMS_OK;
  if (p->desc) {
    int dev = -1;
    s = check_hip(hipGetDevice(&dev), "hipGetDevice");
    if (!s && dev != p->device) s = check_hip(hipSetDevice(p->device), "hipSetDevice");
    if (!s) s = check_hip(hipFree(p->desc), "hipFree (layer descriptors)");
    if (dev >= 0 && dev != p->device) hipSetDevice(dev);
  }
  delete p;
  return s;
}

extern "C" int dms_decode_attn_noalloc(dms_cache* cache, const int32_t* seq_ids, const void* q, void* out, int B,
                                       void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  if (!q || !out) return fail(DMS_ERR_ARG, "q and out are required");
  const Geo& g = cache->geo;
  if (B <= 0) return fail(DMS_ERR_ARG, "B must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  const size_t need = decode_workspace_bytes(decode_grid_for(cache), B * g.Hkv, g.g, g.D);
  if (need > kNoAllocScratchBytes)
    return fail(DMS_ERR_CAPACITY, "this call needs " + std::to_string(need) +
                                      " bytes of decode scratch, above the static 8 MiB of dms_decode_attn_noalloc "
                                      "(use dms_decode_attn with a workspace)");
  int dev = -1;
  int s = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (s) return s;
  if (dev != cache->device) return fail(DMS_ERR_ARG, "the cache's device must be the current device");
  void* ws = nullptr;
  if ((s = noalloc_scratch(dev, &ws))) return s;
  return dms_decode_attn(cache, seq_ids, q, out, B, ws, kNoAllocScratchBytes, stream);
}
