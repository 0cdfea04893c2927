// dms_train_attn_bwd: gradients of the training-mode attention forward
// ("基于 DMS 的 KV Cache 压缩实战" walkthrough, 注意力 / 训练模式: causal
// attention whose scores at distance >= window carry the key's
// logsigmoid(-y) penalty; the gate logit y gets its gradient through it).
//
// With P = exp(s - lse) recomputed from the forward's log-sum-exp:
//   dP = dO V^T,  dS = P * (dP - delta),  delta_i = sum_d dO_i O_i,
//   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dO   (k, v summed over the
//   query heads of their group),
//   dy_j = -sigmoid(y_j) * sum of dS_ij over the penalised pairs (i - j >= w).
//
// Three kernels: delta (D / 8 lanes per query row and head; it also turns
// each gate logit into its penalty logsigmoid(-y) once); dk/dv/dy, one
// workgroup per 64 keys of a (sequence, KV head), each wave owning 16 keys
// whose K and V fragments stay in registers while the workgroup stages the
// Q and dO rows of each 64-query tile (for every query head of the group) in
// LDS; dq, one workgroup per 64 queries of a (sequence, query head), each
// wave owning 16 queries whose Q and dO fragments stay in registers while the
// workgroup stages the K and V rows of each causal 64-key tile.  All products
// run on bf16 16x16x32 matrix cores (fp32 accumulation) over 32-row blocks;
// P and dS are rounded to bf16 as operands, as in the forward.
//
// 16x16x32 operand layout (lane l, g = l / 16, i = 0..7): lane l supplies
// A[l % 16][8 g + i] and B[8 g + i][l % 16] and holds D[4 g + v][l % 16] in
// element v.  Two 16-row score blocks (rows 0..15 and 16..31 of a 32-row
// block) leave lane l the rows 4 g + v and 16 + 4 g + v of its column; with
// the contraction index k = 8 g + i read as row (i < 4 ? 4 g + i :
// 16 + 4 g + i - 4), those eight values are the lane's A operand of the next
// product (P^T dO and dS^T Q in dk/dv, dS K in dq), and the matching B
// operand, four rows at one column twice, comes from the transposing LDS
// read ds_read_b64_tr_b16 (within 16 lanes, lane j receives element j of
// each of the four 16-element rows the group addresses).
#include <algorithm>
#include <cmath>

#include "dms_internal.h"

namespace dms {
namespace {

typedef short tb_s4 __attribute__((ext_vector_type(4)));
typedef float tb_f4 __attribute__((ext_vector_type(4)));

struct BwdArgs {
  const uint16_t* q;      // [B][T][Hq][D] bf16
  const uint16_t* k;      // [B][T][Hkv][D]
  const uint16_t* v;
  const uint16_t* o;      // forward output [B][T][Hq][D]
  const uint16_t* dout;   // [B][T][Hq][D]
  const float* y;         // gate logits [B][Hkv][T]
  const float* lse;       // forward log-sum-exp [B][Hq][T]
  float* delta;           // [B][Hq][T] (written by the first kernel)
  float* pen;             // [B][Hkv][T]: logsigmoid(-y) * log2(e) (written by the first kernel)
  float* dq;              // [B][T][Hq][D] f32
  float* dk;              // [B][T][Hkv][D] f32
  float* dv;
  float* dy;              // [B][Hkv][T] f32
  int B, T, Hq, Hkv, w;
  float scale;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdKeyGroups = 1;          // 16-key groups per wave in the dk/dv kernel

__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

typedef __bf16 tb_bf8 __attribute__((ext_vector_type(8)));
typedef float tb_f8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) tb_s4 tb_lds_s4;

// 8 consecutive bf16 at p (16-byte aligned); zeros when !ok
__device__ __forceinline__ tb_bf8 load8(const uint16_t* p, bool ok) {
  if (!ok) return __builtin_bit_cast(tb_bf8, make_uint4(0u, 0u, 0u, 0u));
  return *reinterpret_cast<const tb_bf8*>(p);
}

// the eight products' operands of a 32-row block, rounded to bf16
__device__ __forceinline__ tb_bf8 pack8(const float* x) {
  const tb_f8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, tb_bf8);
}

// B operand of a 32-row contraction at LDS column c: rows r and r + 16 of
// the lane's group (see the layout note above); p points at row r's column
// c + 4 (l16 & 3) with r = 4 g + (l16 >> 2) relative to the block.
template <int LD>
__device__ __forceinline__ tb_bf8 lds_cols8(const uint16_t* p) {
  const tb_s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((tb_lds_s4*)(p));
  const tb_s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((tb_lds_s4*)(p + 16 * LD));
  return __builtin_bit_cast(tb_bf8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// logsigmoid(-y) = -softplus(y), stable for either sign
__device__ __forceinline__ float penalty(float yv) { return -(fmaxf(yv, 0.0f) + log1pf(__expf(-fabsf(yv)))); }

// delta of one (b, t, h) row per D / 8 lanes: 16-byte loads of dO and O,
// products summed in fp32, then over the row's lanes by xor shuffles.
template <int D>
__global__ __launch_bounds__(256) void train_bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;                // lanes per row
  const int64_t r = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / LPR;   // (b, t, h) row of O
  const int part = threadIdx.x % LPR;
  const int64_t rows = static_cast<int64_t>(a.B) * a.T * a.Hq;
  float s = 0.0f;
  if (r < rows) {
    const uint4 x = *reinterpret_cast<const uint4*>(a.dout + r * D + 8 * part);
    const uint4 y = *reinterpret_cast<const uint4*>(a.o + r * D + 8 * part);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s = fmaf(bf(static_cast<uint16_t>(xs[j] & 0xFFFF)), bf(static_cast<uint16_t>(ys[j] & 0xFFFF)), s);
      s = fmaf(bf(static_cast<uint16_t>(xs[j] >> 16)), bf(static_cast<uint16_t>(ys[j] >> 16)), s);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  // the keys' penalties, once per (b, kv, t), for the two gradient kernels
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid < static_cast<int64_t>(a.B) * a.Hkv * a.T) a.pen[gid] = penalty(a.y[gid]) * kLog2e;
  if (r < rows && part == 0) {
    const int h = static_cast<int>(r % a.Hq);
    const int64_t bt = r / a.Hq;
    const int t = static_cast<int>(bt % a.T), b = static_cast<int>(bt / a.T);
    a.delta[(static_cast<int64_t>(b) * a.Hq + h) * a.T + t] = s;
  }
}

// Rows [r0, r0 + 64) of one head of a [B][T][H][D] bf16 tensor, staged in
// two steps so that the next tile's global loads run under the current
// tile's products: fetch reads this thread's 16-byte chunks into registers
// (rows past T are zero), put writes them to LDS rows of stride D + 16
// elements.  With rows of 2 D + 32 bytes both the 16-byte row
// reads and the transposing column reads are free of bank conflicts.
template <int D>
struct TileRows {
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int LD = D + 16;
  static constexpr int NIT = 64 * CH / 256; // chunks per thread
  uint4 r[NIT];
  __device__ __forceinline__ void fetch(const uint16_t* src, int b, int r0, int T, int H, int h) {
    // row r0 + row of head h is base + row * stride; this thread's rows are
    // threadIdx.x / CH + (256 / CH) it, its column (threadIdx.x % CH) * 8
    const size_t stride = static_cast<size_t>(H) * D;
    const int row0 = threadIdx.x / CH;
    const uint16_t* p = src + (static_cast<size_t>(b) * T + r0 + row0) * stride + static_cast<size_t>(h) * D +
                        (threadIdx.x % CH) * 8;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int row = row0 + (256 / CH) * it;
      r[it] = r0 + row < T ? *reinterpret_cast<const uint4*>(p + static_cast<size_t>((256 / CH) * it) * stride)
                           : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void put(uint16_t* dst) const {
    uint16_t* p = dst + (threadIdx.x / CH) * LD + (threadIdx.x % CH) * 8;
#pragma unroll
    for (int it = 0; it < NIT; ++it) *reinterpret_cast<uint4*>(p + (256 / CH) * it * LD) = r[it];
  }
};

// Workgroup (pair, tile): keys [64 KG tile, 64 KG (tile + 1)) of (b, kv);
// wave w owns the 16 KG keys from k0 = 64 KG tile + 16 KG w, in KG groups of
// 16 that share every LDS operand read.  Per query tile of 64 rows and query
// head of the group, the workgroup stages the Q and dO rows (and their lse,
// delta) in LDS once; each wave then takes the two 32-query blocks.  Tiles
// with the most causal queries (low tile index) are dispatched first.
template <int D, int G, int KG>
__global__ __launch_bounds__(256, KG == 1 ? 2 : 1) void train_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int K32 = D / 32;               // k-steps of S and dP over head_dim
  constexpr int DT = D / 16;                // 16-column tiles of dK and dV
  constexpr int LD = D + 16;
  __shared__ __align__(16) uint16_t sQ[64 * LD];
  __shared__ __align__(16) uint16_t sO[64 * LD];
  __shared__ __align__(16) float sL[64];
  __shared__ __align__(16) float sDl[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int pair = blockIdx.x, b = pair / a.Hkv, kv = pair % a.Hkv;
  const int kt0 = blockIdx.y * 64 * KG;
  const int k0 = kt0 + wave * 16 * KG;
  // K and V fragments of the wave's keys (B operands of S = Q K^T, dP = dO V^T);
  // lane column l16 of group kg is key k0 + 16 kg + l16
  tb_bf8 kf[KG][K32], vf[KG][K32];
  float pen2[KG], yk[KG];
#pragma unroll
  for (int kg = 0; kg < KG; ++kg) {
    const int key = k0 + 16 * kg + l16;
    const bool ok = key < a.T;
    const size_t krow = ((static_cast<size_t>(b) * a.T + (ok ? key : 0)) * a.Hkv + kv) * D;
#pragma unroll
    for (int ks = 0; ks < K32; ++ks) {
      kf[kg][ks] = load8(a.k + krow + 32 * ks + 8 * g, ok);
      vf[kg][ks] = load8(a.v + krow + 32 * ks + 8 * g, ok);
    }
    yk[kg] = ok ? a.y[(static_cast<int64_t>(b) * a.Hkv + kv) * a.T + key] : 0.0f;
    pen2[kg] = ok ? a.pen[(static_cast<int64_t>(b) * a.Hkv + kv) * a.T + key] : 0.0f;
  }
  tb_f4 dk[KG][DT], dv[KG][DT];
#pragma unroll
  for (int kg = 0; kg < KG; ++kg)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dk[kg][dt] = tb_f4{0.f, 0.f, 0.f, 0.f};
      dv[kg][dt] = tb_f4{0.f, 0.f, 0.f, 0.f};
    }
  float dyacc[KG];
#pragma unroll
  for (int kg = 0; kg < KG; ++kg) dyacc[kg] = 0.0f;
  const float sl2 = a.scale * kLog2e;
  // tiles in the order (query tile, head of the group); the next one's rows
  // are fetched into registers while the current one is computed
  TileRows<D> nq, no;
  float nrow = 0.0f;                        // lse (threads 0..63) or delta (64..127) of the next tile
  auto fetch = [&](int qb, int h) {
    nq.fetch(a.q, b, qb, a.T, a.Hq, h);
    no.fetch(a.dout, b, qb, a.T, a.Hq, h);
    if (threadIdx.x < 128) {
      const int t = qb + (threadIdx.x & 63);
      const int64_t li = (static_cast<int64_t>(b) * a.Hq + h) * a.T + t;
      nrow = t >= a.T ? 0.0f : threadIdx.x < 64 ? a.lse[li] * kLog2e : a.delta[li];
    }
  };
  int nqb = kt0, nhh = 0;
  if (nqb < a.T) fetch(nqb, kv * G);
  while (nqb < a.T) {
    const int qb = nqb;
    __syncthreads();                        // previous tile fully read
    nq.put(sQ);
    no.put(sO);
    if (threadIdx.x < 64) sL[threadIdx.x] = nrow;
    else if (threadIdx.x < 128) sDl[threadIdx.x - 64] = nrow;
    __syncthreads();
    if (++nhh == G) {
      nhh = 0;
      nqb += 64;
    }
    if (nqb < a.T) fetch(nqb, kv * G + nhh);
    // both blocks' score products first, so that the second block's run on
    // the matrix cores while the first block's P and dS are formed
    bool act[2];
    tb_f4 sb[2][KG][2], dpb[2][KG][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int i0 = qb + 32 * blk;
      // skipped: past T, or every query of the block before the wave's keys
      act[blk] = i0 < a.T && k0 < a.T && i0 + 31 >= k0;
      if (!act[blk]) continue;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint16_t* qr = sQ + (32 * blk + 16 * c + l16) * LD + 8 * g;
        const uint16_t* orow = sO + (32 * blk + 16 * c + l16) * LD + 8 * g;
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
          sb[blk][kg][c] = tb_f4{0.f, 0.f, 0.f, 0.f};
          dpb[blk][kg][c] = tb_f4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < K32; ++ks) {
          const tb_bf8 qa = *reinterpret_cast<const tb_bf8*>(qr + 32 * ks);
          const tb_bf8 oa = *reinterpret_cast<const tb_bf8*>(orow + 32 * ks);
#pragma unroll
          for (int kg = 0; kg < KG; ++kg) {
            sb[blk][kg][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[kg][ks], sb[blk][kg][c], 0, 0, 0);
            dpb[blk][kg][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vf[kg][ks], dpb[blk][kg][c], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      if (!act[blk]) continue;
      const int i0 = qb + 32 * blk;
      const auto& s = sb[blk];
      const auto& dp = dpb[blk];
      // element (c, e) of group kg: query i0 + 16 c + 4 g + e, key k0 + 16 kg + l16.
      // A block with every query after every key of the wave, inside T, and
      // all of its pairs either inside the window or past it takes no
      // per-element test (the wave agrees on the branch).
      const int klast = k0 + 16 * KG - 1;
      const bool inside = i0 + 31 < a.T && klast < a.T && i0 >= klast;
      const bool pen_all = i0 - klast >= a.w, pen_none = i0 + 31 - k0 < a.w;
      tb_bf8 pA[KG], dA[KG];
      if (inside && (pen_all || pen_none)) {
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
          const float pb = pen_all ? pen2[kg] : 0.0f;
          float p[8], ds[8], dsum = 0.0f;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float4 L4 = *reinterpret_cast<const float4*>(sL + 32 * blk + 16 * c + 4 * g);
            const float4 D4 = *reinterpret_cast<const float4*>(sDl + 32 * blk + 16 * c + 4 * g);
            const float Lr[4] = {L4.x, L4.y, L4.z, L4.w}, Dr[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pv = __builtin_amdgcn_exp2f(fmaf(s[kg][c][e], sl2, pb - Lr[e]));
              const float dsv = pv * (dp[kg][c][e] - Dr[e]);
              dsum += dsv;
              p[4 * c + e] = pv;
              ds[4 * c + e] = dsv;
            }
          }
          if (pen_all) dyacc[kg] += dsum;
          pA[kg] = pack8(p);
          dA[kg] = pack8(ds);
        }
      } else {
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
          const int key = k0 + 16 * kg + l16;
          float p[8], ds[8];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rr = 32 * blk + 16 * c + 4 * g + e;
              const int qi = qb + rr;
              float pv = 0.0f, dsv = 0.0f;
              if (qi < a.T && key < a.T && qi >= key) {
                const bool penalised = qi - key >= a.w;
                pv = __builtin_amdgcn_exp2f(s[kg][c][e] * sl2 + (penalised ? pen2[kg] : 0.0f) - sL[rr]);
                dsv = pv * (dp[kg][c][e] - sDl[rr]);
                if (penalised) dyacc[kg] += dsv;
              }
              p[4 * c + e] = pv;
              ds[4 * c + e] = dsv;
            }
          }
          pA[kg] = pack8(p);
          dA[kg] = pack8(ds);
        }
      }
      // dV += P^T dO, dK += dS^T Q: B operands dO / Q at rows (query)
      // 4 g + i and 16 + 4 g + i of the block, column 16 dt + l16
      const int cofs = (32 * blk + 4 * g + (l16 >> 2)) * LD + 4 * (l16 & 3);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const tb_bf8 ob = lds_cols8<LD>(sO + cofs + 16 * dt);
        const tb_bf8 qb8 = lds_cols8<LD>(sQ + cofs + 16 * dt);
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
          dv[kg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pA[kg], ob, dv[kg][dt], 0, 0, 0);
          dk[kg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dA[kg], qb8, dk[kg][dt], 0, 0, 0);
        }
      }
    }
  }
  if (k0 >= a.T) return;
#pragma unroll
  for (int kg = 0; kg < KG; ++kg) {
    // dK, dV: element v of tile dt is key k0 + 16 kg + 4 g + v, dim 16 dt + l16
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = k0 + 16 * kg + 4 * g + e;
        if (kk < a.T) {
          const size_t r = ((static_cast<size_t>(b) * a.T + kk) * a.Hkv + kv) * D + 16 * dt + l16;
          a.dk[r] = dk[kg][dt][e] * a.scale;
          a.dv[r] = dv[kg][dt][e];
        }
      }
    }
    // dy: this lane's key summed over the four query groups (lanes l16 + 16 m)
    float d = dyacc[kg];
    d += __shfl_xor(d, 16);
    d += __shfl_xor(d, 32);
    const int key = k0 + 16 * kg + l16;
    if (g == 0 && key < a.T) {
      const float sig = 1.0f / (1.0f + __expf(-yk[kg]));
      a.dy[(static_cast<int64_t>(b) * a.Hkv + kv) * a.T + key] = -sig * d;
    }
  }
}

// Workgroup (row, tile): queries [64 tile, 64 tile + 64) of (b, h); wave w
// owns queries q0 = 64 tile + 16 w .. + 16.  Per key tile of 64 rows the
// workgroup stages the K and V rows (and the keys' penalties) in LDS; each
// wave takes the 32-key blocks that are causal for it.  Tiles with the most
// keys (high tile index) are dispatched first.
template <int D, int G>
__global__ __launch_bounds__(256, 3) void train_bwd_dq_kernel(BwdArgs a) {
  constexpr int K32 = D / 32;
  constexpr int DT = D / 16;
  constexpr int LD = D + 16;
  __shared__ __align__(16) uint16_t sK[64 * LD];
  __shared__ __align__(16) uint16_t sV[64 * LD];
  __shared__ __align__(16) float sP[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int row = blockIdx.x, b = row / a.Hq, h = row % a.Hq, kv = h / G;
  const int qt0 = (static_cast<int>(gridDim.y) - 1 - static_cast<int>(blockIdx.y)) * 64;
  const int q0 = qt0 + wave * 16;
  const int qi = q0 + l16;                  // this lane's query (column of S^T)
  const bool q_ok = qi < a.T;
  // Q and dO fragments of the wave's queries (B operands of S^T = K Q^T, dP^T = V dO^T)
  const size_t qrow = ((static_cast<size_t>(b) * a.T + (q_ok ? qi : 0)) * a.Hq + h) * D;
  tb_bf8 qf[K32], of[K32];
#pragma unroll
  for (int ks = 0; ks < K32; ++ks) {
    qf[ks] = load8(a.q + qrow + 32 * ks + 8 * g, q_ok);
    of[ks] = load8(a.dout + qrow + 32 * ks + 8 * g, q_ok);
  }
  const int64_t li = (static_cast<int64_t>(b) * a.Hq + h) * a.T + (q_ok ? qi : 0);
  const float lse2 = q_ok ? a.lse[li] * kLog2e : 0.0f;
  const float dlt = q_ok ? a.delta[li] : 0.0f;
  tb_f4 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = tb_f4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.scale * kLog2e;
  const int kend = min(a.T, qt0 + 64);
  // the next key tile's rows are fetched into registers while the current
  // one is computed
  TileRows<D> nk, nv;
  float npen = 0.0f;                        // threads 0..63: the next tile's key penalties
  auto fetch = [&](int kb) {
    nk.fetch(a.k, b, kb, a.T, a.Hkv, kv);
    nv.fetch(a.v, b, kb, a.T, a.Hkv, kv);
    const int t = kb + threadIdx.x;
    if (threadIdx.x < 64)
      npen = t < a.T ? a.pen[(static_cast<int64_t>(b) * a.Hkv + kv) * a.T + t] : 0.0f;
  };
  if (kend > 0) fetch(0);
  for (int kb = 0; kb < kend; kb += 64) {
    __syncthreads();                        // previous tile fully read
    nk.put(sK);
    nv.put(sV);
    if (threadIdx.x < 64) sP[threadIdx.x] = npen;
    __syncthreads();
    if (kb + 64 < kend) fetch(kb + 64);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int j0 = kb + 32 * blk;
      if (j0 >= a.T || j0 > q0 + 15 || q0 >= a.T) break;   // keys past every query of the wave
      tb_f4 s[2], dp[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint16_t* kr = sK + (32 * blk + 16 * c + l16) * LD + 8 * g;
        const uint16_t* vr = sV + (32 * blk + 16 * c + l16) * LD + 8 * g;
        s[c] = tb_f4{0.f, 0.f, 0.f, 0.f};
        dp[c] = tb_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < K32; ++ks) {
          s[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const tb_bf8*>(kr + 32 * ks), qf[ks], s[c],
                                                         0, 0, 0);
          dp[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const tb_bf8*>(vr + 32 * ks), of[ks],
                                                          dp[c], 0, 0, 0);
        }
      }
      // element (c, e): key j0 + 16 c + 4 g + e, query qi.  A block with
      // every key before every query of the wave, inside T, and all of its
      // pairs either inside the window or past it takes no per-element test.
      const bool inside = j0 + 31 < a.T && q0 + 15 < a.T && j0 + 31 <= q0;
      const bool pen_all = q0 - (j0 + 31) >= a.w, pen_none = q0 + 15 - j0 < a.w;
      float ds[8];
      if (inside && (pen_all || pen_none)) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float4 P4 = pen_all ? *reinterpret_cast<const float4*>(sP + 32 * blk + 16 * c + 4 * g)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
          const float Pr[4] = {P4.x, P4.y, P4.z, P4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[c][e], sl2, Pr[e] - lse2));
            ds[4 * c + e] = pv * (dp[c][e] - dlt);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rr = 32 * blk + 16 * c + 4 * g + e;
            const int kj = kb + rr;
            float dsv = 0.0f;
            if (q_ok && kj < a.T && kj <= qi) {
              const float pv = __builtin_amdgcn_exp2f(s[c][e] * sl2 - lse2 + (qi - kj >= a.w ? sP[rr] : 0.0f));
              dsv = pv * (dp[c][e] - dlt);
            }
            ds[4 * c + e] = dsv;
          }
        }
      }
      const tb_bf8 dA = pack8(ds);
      // dQ += dS K: B operand K at rows (key) 4 g + i and 16 + 4 g + i of the
      // block, column 16 dt + l16
      const int cofs = (32 * blk + 4 * g + (l16 >> 2)) * LD + 4 * (l16 & 3);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        dq[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dA, lds_cols8<LD>(sK + cofs + 16 * dt), dq[dt], 0, 0, 0);
    }
  }
  if (q0 >= a.T) return;
  // element v of tile dt: query q0 + 4 g + v, dim 16 dt + l16
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int qq = q0 + 4 * g + e;
      if (qq < a.T) a.dq[((static_cast<size_t>(b) * a.T + qq) * a.Hq + h) * D + 16 * dt + l16] = dq[dt][e] * a.scale;
    }
  }
}

template <int D, int G>
void launch_bwd(const BwdArgs& a, hipStream_t st) {
  constexpr int KG = kBwdKeyGroups;
  const int tiles = (a.T + 63) / 64;
  const int ktiles = (a.T + 64 * KG - 1) / (64 * KG);
  hipLaunchKernelGGL((train_bwd_dkdv_kernel<D, G, KG>), dim3(a.B * a.Hkv, ktiles), dim3(256), 0, st, a);
  hipLaunchKernelGGL((train_bwd_dq_kernel<D, G>), dim3(a.B * a.Hq, tiles), dim3(256), 0, st, a);
}

template <int D>
int launch_bwd_d(const BwdArgs& a, int g, hipStream_t st) {
  switch (g) {
    case 1: launch_bwd<D, 1>(a, st); return DMS_OK;
    case 2: launch_bwd<D, 2>(a, st); return DMS_OK;
    case 4: launch_bwd<D, 4>(a, st); return DMS_OK;
    default: return fail(DMS_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2 or 4");
  }
}

}  // namespace
}  // namespace dms

using namespace dms;

extern "C" int dms_train_attn_bwd_workspace_bytes(int B, int T, int num_q_heads, size_t* bytes) {
  if (!bytes || B < 0 || T < 0 || num_q_heads <= 0) return fail(DMS_ERR_ARG, "bad sizes or NULL bytes");
  *bytes = 2 * static_cast<size_t>(B) * T * num_q_heads * sizeof(float);   // delta, then the key penalties
  return DMS_OK;
}

extern "C" int dms_train_attn_bwd(int B, int T, int num_q_heads, int num_kv_heads, int head_dim, int window,
                                  float softmax_scale, const void* q, const void* k, const void* v, const void* out,
                                  const void* dout, const float* gate_logits, const float* lse, void* dq, void* dk,
                                  void* dv, float* dgate, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || T < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || window < 0) return fail(DMS_ERR_ARG, "bad sizes");
  if (num_q_heads % num_kv_heads) return fail(DMS_ERR_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (head_dim != 64 && head_dim != 128) return fail(DMS_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (B == 0 || T == 0) return DMS_OK;
  if (!q || !k || !v || !out || !dout || !gate_logits || !lse || !dq || !dk || !dv || !dgate)
    return fail(DMS_ERR_ARG, "every tensor argument is required");
  const size_t need = 2 * static_cast<size_t>(B) * T * num_q_heads * sizeof(float);
  if (!workspace || workspace_bytes < need)
    return fail(DMS_ERR_CAPACITY, "workspace smaller than dms_train_attn_bwd_workspace_bytes");
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(dout);
  if ((al | reinterpret_cast<uintptr_t>(out)) % 16)
    return fail(DMS_ERR_UNSUPPORTED, "q, k, v, out and dout must be 16-byte aligned");
  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.y = gate_logits;
  a.lse = lse;
  a.delta = static_cast<float*>(workspace);
  a.pen = a.delta + static_cast<size_t>(B) * T * num_q_heads;   // Hkv <= Hq keys per (b, t)
  a.dq = static_cast<float*>(dq);
  a.dk = static_cast<float*>(dk);
  a.dv = static_cast<float*>(dv);
  a.dy = dgate;
  a.B = B;
  a.T = T;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.w = window;
  a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  hipStream_t st = as_stream(stream);
  const int64_t rows = static_cast<int64_t>(B) * T * num_q_heads;
  const int64_t rows_per_block = 256 / (head_dim / 8);
  const dim3 dgrid(static_cast<unsigned>((rows + rows_per_block - 1) / rows_per_block));
  if (head_dim == 128) hipLaunchKernelGGL(train_bwd_delta_kernel<128>, dgrid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(train_bwd_delta_kernel<64>, dgrid, dim3(256), 0, st, a);
  const int g = num_q_heads / num_kv_heads;
  const int s = head_dim == 128 ? launch_bwd_d<128>(a, g, st) : launch_bwd_d<64>(a, g, st);
  if (s) return s;
  return check_hip(hipGetLastError(), "dms_train_attn_bwd launch");
}
