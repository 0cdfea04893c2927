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
// * Work balance: the live slots of all (row, KV head) units are concatenated
//   and cut into one contiguous range per workgroup, so every workgroup
//   streams the same number of bytes however ragged the heads are.  A range
//   that spans a unit boundary emits one partial per unit.
// * One workgroup serves all g query heads of a KV head, so K/V are read once.
// * Each lane loads 16 contiguous bytes of a K row and of a V row; LPR lanes
//   cover one row, a wave covers 64/LPR rows per pass, NP passes are in flight.
// * Online softmax per wave in base 2; waves merge through LDS; units split
//   over several workgroups are merged by a small combine kernel.
#include "dms_internal.h"

namespace dms {

struct DecodeArgs {
  DevCache d;
  Geo g;
  const int32_t* seq_ids;
  const void* q;
  void* out;
  int B;
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

}  // namespace dms

using namespace dms;

extern "C" int dms_decode_attn(dms_cache* cache, const int32_t* seq_ids, const void* q, void* out, int B,
                               void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  if (!q || !out) return fail(DMS_ERR_ARG, "q and out are required");
  const Geo& g = cache->geo;
  if (B <= 0) return fail(DMS_ERR_ARG, "B must be positive");
  if (B > g.Bmax) return fail(DMS_ERR_CAPACITY, "B above max_batch");
  DecodeArgs a{cache->dev, g, seq_ids, q, out, B};
  const int grid = decode_grid_for(cache);
  hipStream_t st = as_stream(stream);
  int s;
  switch (g.kv_dtype) {
    case DMS_F32: s = launch_decode<float, DMS_F32>(a, grid, st); break;
    case DMS_BF16: s = launch_decode<uint16_t, DMS_BF16>(a, grid, st); break;
    case DMS_FP8_E4M3: s = launch_decode<uint16_t, DMS_FP8_E4M3>(a, grid, st); break;
    default: return fail(DMS_ERR_UNSUPPORTED, "kv dtype");
  }
  if (s) return s;
  return check_hip(hipGetLastError(), "dms_decode_attn launch");
}
