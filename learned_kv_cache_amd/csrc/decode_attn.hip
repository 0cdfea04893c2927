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
        float* pr = d.partials + (static_cast<int64_t>(rec) * G + h) * (D + 2);
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
      for (int i = 0; i < n; ++i) M = fmaxf(M, a.d.partials[(static_cast<int64_t>(pb + i) * G + h) * (D + 2) + D]);
      float ov = 0.0f, lv = 0.0f;
      for (int i = 0; i < n; ++i) {
        const float* pr = a.d.partials + (static_cast<int64_t>(pb + i) * G + h) * (D + 2);
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
  int npairs;              // workgroups of the prepare role (B * Hkv), placed first in the grid
  int groups;              // arrival groups of the attention workgroups (min(kArriveGroups, their count))
  int agrid;               // attention workgroups
  int qneuron;             // the decision neuron (last element of each group's first query head) reads as zero
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

// The attention of dms_decode_attn (workgroup wg of `grid`).  STEP: the
// attention of the fused decode step, run before the current token is in the
// cache: each unit's rows are its live slots plus one more, the current
// token, read from the input rows; the slot the token overwrites in place is
// masked.  The same keys as after the append.  Once a workgroup has read the
// lengths, positions and ring entries it works from, it counts itself on its
// arrival group; the prepare role's commit waits for all of them.
template <int D, int G, int NP, bool FP8, int LPR, bool STEP>
__device__ __forceinline__ void decode_attn_fast_body(const DecodeArgs& a, const StepArgs* sa, int wg, int grid,
                                                      FastLds<G, D, STEP>& lds) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int RB = D * EB;
  constexpr int BPL = RB / LPR;
  constexpr int EPL = BPL / EB;
  constexpr int QW = EPL / 2;
  constexpr int RG = 64 / LPR;
  constexpr int RPP = 4 * RG;
  constexpr int NV = BPL / 16;
  static_assert(NP % 2 == 0, "passes are paired for the P.V dot products");
  static_assert(BPL % 16 == 0, "a lane loads whole 16-byte pieces");

  int* s_start = lds.start;
  int* s_tmp = lds.tmp;
  const DevCache& d = a.d;
  const Geo& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lane_row = lane / LPR, lane_col = lane % LPR;
  const int units = a.B * g.Hkv;

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
  const int W = s_start[units];
  const int c = max((W + grid - 1) / grid, RPP);
  // Few units: each unit gets workgroups of its own, ceil(slots / ca) of
  // them for a cap of ca = ceil(W / (grid - units)) slots per workgroup (at
  // most one per RPP rows and kMaxSplit in all), so no workgroup spans two
  // units (a second segment would repeat the setup and the merge);
  // sum(ceil(slots / ca)) <= W / ca + units <= grid.  Otherwise the
  // concatenated slots are cut into equal ranges.
  const bool aligned = units <= kAlignedUnits && 2 * units <= grid;
  int* s_wstart = lds.wstart;
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

  // heads without live slots have no workgroup: workgroup 0 writes zeros
  if (wg == 0) {
    uint16_t* ob = static_cast<uint16_t*>(a.out);
    for (int uu = 0; uu < units; ++uu) {
      if (s_start[uu + 1] != s_start[uu]) continue;
      const int row = uu / g.Hkv, kh = uu % g.Hkv;
      for (int idx = tid; idx < G * D; idx += 256) ob[(static_cast<size_t>(row) * g.Hq + kh * G) * D + idx] = 0;
    }
  }

  int a0, a1, u;
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
  bool first_seg = true;
  uint16_t* obase = static_cast<uint16_t*>(a.out);
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
  const int psh = g.Pshift, pmask = g.P - 1;

  while (a0 < a1) {
    const int ustart = s_start[u], uend = s_start[u + 1];
    const int seg_end = min(a1, uend);
    const int lo = a0 - ustart, hi = seg_end - ustart;
    const int row = u / g.Hkv, kh = u % g.Hkv;
    const int seq = a.seq_ids ? a.seq_ids[row] : row;
    const int32_t* pt = d.page_table + (static_cast<int64_t>(seq) * g.Hkv + kh) * g.maxp;
    int vrow = -1, skip = -1;
    const uint8_t* kin = nullptr;
    const uint8_t* vin = nullptr;
    if constexpr (STEP) {
      const int ext = lds.ext[u];
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
          const int page = skip >= 0 ? pt[skip >> psh] : d.cur_page[static_cast<int64_t>(seq) * g.Hkv + kh];
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
      const int pt_reg = (pb + lane <= plast) ? pt[pb + lane] : 0;
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
    __syncthreads();
    // the unit's workgroups w0..w1 (concatenated split: w0's record is its
    // second one when the unit starts inside w0's range)
    const int w0 = aligned ? s_wstart[u] : ustart / c;
    const int w1 = aligned ? s_wstart[u + 1] - 1 : (uend - 1) / c;
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
          ov += f * (lds.o[w][0][h][dd] + lds.o[w][1][h][dd] + lds.o[w][2][h][dd] + lds.o[w][3][h][dd]);
          lv += f * (lds.ml[w][0][h][1] + lds.ml[w][1][h][1] + lds.ml[w][2][h][1] + lds.ml[w][3][h][1]);
        }
      }
      if (!split) {
        obase[(static_cast<size_t>(row) * g.Hq + kh * G + h) * D + dd] = f32_to_bf16(lv > 0.0f ? ov / lv : 0.0f);
      } else {
        // device-coherent stores (no L2 write-back of the XCD needed)
        float* pr = d.partials + (static_cast<int64_t>(rec) * G + h) * (D + 2);
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
        merge_unit_records<D, G>(d.partials, w0, w1, odd, obase + (static_cast<size_t>(row) * g.Hq + kh * G) * D);
        if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    first_seg = false;
    a0 = seg_end;
    ++u;
    while (u < units && s_start[u + 1] <= a0) ++u;
  }
}


template <int D, int G, int NP, bool FP8, int LPR>
__global__ __launch_bounds__(256) void decode_attn_fast_kernel(DecodeArgs a) {
  __shared__ FastLds<G, D, false> lds;
  decode_attn_fast_body<D, G, NP, FP8, LPR, false>(a, nullptr, blockIdx.x, gridDim.x, lds);
}

// dms_decode_step: workgroups [0, npairs) prepare the current token of one
// (row, KV head) pair each (decision, placement, plan record); the others run
// the attention (STEP).  The last pair to finish waits until every attention
// workgroup has arrived (read the tables it works from), then commits.
template <int D, int G, int NP, bool FP8, int LPR>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a, AppendArgs ap, PrepIn pin, StepArgs sa) {
  constexpr int KV = FP8 ? DMS_FP8_E4M3 : DMS_BF16;
  __shared__ FastLds<G, D, true> lds;
  if (static_cast<int>(blockIdx.x) < sa.npairs) {
    PrepShared& sh = lds.prep;
    prep_pair<KV>(ap, pin, blockIdx.x, true, sh);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
      sh.last = __hip_atomic_fetch_add(ap.d.ctl + kCtlPrepArrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                sa.npairs - 1;
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
          if (__hip_atomic_load(gc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) break;
          if (it == kArriveSpinLimit) {
            ok = false;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      const bool all = __all(ok);
      if (lane == 0) sh.n = all ? 1 : 0;
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(sh.n)) {
      if (threadIdx.x == 0) set_status(ap.d.ctl, DMS_DEV_STEP_SYNC);
      return;
    }
    prep_commit<KV>(ap, pin, sa.npairs, sh);
    if (threadIdx.x < sa.groups)
      __hip_atomic_store(ap.d.arrive + threadIdx.x * kArriveStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  decode_attn_fast_body<D, G, NP, FP8, LPR, true>(a, &sa, blockIdx.x - sa.npairs, sa.agrid, lds);
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
static StepKernel step_kernel_dg(const Geo& g, int lanes_per_row) {
  if (g.kv_dtype == DMS_FP8_E4M3) return decode_step_kernel<D, G, 2, true, D / 16>;
  constexpr int RB = D * 2;
  constexpr int LPR1 = RB / 16 >= 16 ? 16 : RB / 16;
  if constexpr (RB / 16 >= 16) {
    if (lanes_per_row == 8) return decode_step_kernel<D, G, 2, false, 8>;
  }
  return decode_step_kernel<D, G, 2, false, LPR1>;
}

template <int D>
static StepKernel step_kernel_d(const Geo& g, int lanes_per_row) {
  switch (g.g) {
    case 1: return step_kernel_dg<D, 1>(g, lanes_per_row);
    case 2: return step_kernel_dg<D, 2>(g, lanes_per_row);
    case 4: return step_kernel_dg<D, 4>(g, lanes_per_row);
    case 8: return step_kernel_dg<D, 8>(g, lanes_per_row);
    default: return nullptr;
  }
}

static StepKernel step_kernel(const Geo& g, int lanes_per_row) {
  return g.D == 128 ? step_kernel_d<128>(g, lanes_per_row) : step_kernel_d<64>(g, lanes_per_row);
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

}  // namespace dms

using namespace dms;

extern "C" int dms_decode_attn(dms_cache* cache, const int32_t* seq_ids, const void* q, void* out, int B,
                               void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  if (!q || !out) return fail(DMS_ERR_ARG, "q and out are required");
  const Geo& g = cache->geo;
  if (B <= 0) return fail(DMS_ERR_ARG, "B must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  DecodeArgs a{cache->dev, g, seq_ids, q, out, B, cache->decode_lpr};
  const int grid = decode_grid_for(cache);
  hipStream_t st = as_stream(stream);
  int s;
  if (fast_decode_ok(cache, nullptr)) {
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
                               const void* v, void* out, int B, float* logits_out, uint8_t* evict_out, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  const dms_config& c = cache->cfg;
  const Geo& g = cache->geo;
  if (!q_inout || !out || !k || !v || !offsets || !evict_out)
    return fail(DMS_ERR_ARG, "q_inout, out, k, v, offsets and evict_out are required");
  if (B <= 0) return fail(DMS_ERR_ARG, "B must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  const bool linear = c.decide_mode == DMS_DECIDE_LINEAR;
  if (linear && (!hidden || !rms_gamma || !W)) return fail(DMS_ERR_ARG, "hidden, rms_gamma and W are required");
  uintptr_t al = reinterpret_cast<uintptr_t>(q_inout) | reinterpret_cast<uintptr_t>(k) |
                 reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if (linear)
    al |= reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(rms_gamma) |
          reinterpret_cast<uintptr_t>(W);
  const int npairs = B * g.Hkv;
  const int agrid = decode_grid_for(cache);
  bool fused = cache->step_fuse != 0 && fast_decode_ok(cache, nullptr) && al % 16 == 0 &&
               (!linear || c.hidden % 8 == 0) && npairs <= kMaxUnits;
  StepKernel kern = fused ? step_kernel(g, cache->decode_lpr) : nullptr;
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
    fused = npairs + agrid <= cache->step_blocks_per_cu * cache->num_cus;
  }
  hipStream_t st = as_stream(stream);
  if (!fused) {
    // other shapes, or a step too large for one resident launch: the two calls in turn
    int s = dms_decode_prepare(cache, seq_ids, hidden, rms_gamma, W, bias, offsets, q_inout, k, v, B, logits_out,
                               evict_out, stream);
    if (s) return s;
    return dms_decode_attn(cache, seq_ids, q_inout, out, B, stream);
  }
  DecodeArgs a{cache->dev, g, seq_ids, q_inout, out, B, cache->decode_lpr};
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
  StepArgs sa{static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), npairs, groups, agrid,
              linear ? 0 : 1};
  hipLaunchKernelGGL(kern, dim3(npairs + agrid), dim3(256), 0, st, a, ap, pin, sa);
  return check_hip(hipGetLastError(), "dms_decode_step launch");
}
