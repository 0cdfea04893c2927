// dms_decide: the per-KV-head keep/evict decision.
//
// Linear adapter ("基于 DMS 的 KV Cache 压缩实战" walkthrough, 决策来源二):
//   logit[b][k][t] = alpha * (W_k . RMSNorm(h[b][t])) - offset_k.
// Repurposed query neuron (same page, 决策来源一):
//   logit[b][k][t] = alpha * q[b][t][k*g][D-1] - offset_k, then that element is
//   set to zero.
// Granularity (决策粒度): "layer" gives every head head 0's logit.
// Threshold (Gumbel section, inference): evict = logit > 0; with
// disable_eviction nothing is evicted.
//
// The projection reads h once (2 bytes per element for bf16) and does
// Hkv + 1 fused multiply-adds per element, so it is bound by HBM (prefill) or
// by latency (decode), not by arithmetic; it runs in fp32 on the vector ALUs.
// Rounding the normalised activations to bf16 for a matrix-core product would
// move logits by ~0.1, far more than the 1e-2 margin decisions are compared at.
#include <algorithm>
#include <cstdlib>

#include "dms_internal.h"

namespace dms {

struct DecideArgs {
  const void* hidden;
  const float* gamma;
  const float* W;
  const float* bias;
  const float* offsets;
  int ntok;            // B * T
  int T;
  int H;
  float alpha;
  float eps;
  int per_layer;
  int disable;
  float* logits;       // [B][Hkv][T] or null
  uint8_t* evict;      // [B][Hkv][T]
};

template <int N> __device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __shfl_xor(v[i], o);
  }
}

// TT tokens per 256-thread workgroup.  Thread t owns the elements
// [4t + 1024i, 4t + 1024i + 4) of the hidden vector for i = 0..H/1024-1 and
// keeps its W and gamma values in registers for all TT tokens; every lane
// accumulates sum(h^2) and, per head, sum(W_k * gamma * h); waves reduce with
// shuffles, the four waves through LDS; then z_k = r * dot_k with
// r = 1 / sqrt(mean(h^2) + eps).
template <typename ACT, int HKV, int TT, int NCH>
__global__ __launch_bounds__(256) void decide_linear_kernel(DecideArgs a) {
  __shared__ float s_red[4][TT][HKV + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok0 = blockIdx.x * TT;
  float acc[TT][HKV + 1];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int k = 0; k <= HKV; ++k) acc[t][k] = 0.0f;
  for (int m0 = 4 * tid; m0 < a.H; m0 += 1024 * NCH) {
    float4 w[NCH][HKV];
    float4 gm[NCH];
    bool okc[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int m = m0 + 1024 * c;
      okc[c] = m < a.H;
      gm[c] = okc[c] ? *reinterpret_cast<const float4*>(a.gamma + m) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < HKV; ++k)
        w[c][k] = okc[c] ? *reinterpret_cast<const float4*>(a.W + static_cast<size_t>(k) * a.H + m)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int tok = tok0 + t;
      if (tok >= a.ntok) break;
      const ACT* h = static_cast<const ACT*>(a.hidden) + static_cast<size_t>(tok) * a.H;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (!okc[c]) continue;
        const int m = m0 + 1024 * c;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = load_act<ACT>(h, m + e);
        const float gx[4] = {gm[c].x * x[0], gm[c].y * x[1], gm[c].z * x[2], gm[c].w * x[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][HKV] = fmaf(x[e], x[e], acc[t][HKV]);
#pragma unroll
        for (int k = 0; k < HKV; ++k) {
          acc[t][k] = fmaf(w[c][k].x, gx[0], acc[t][k]);
          acc[t][k] = fmaf(w[c][k].y, gx[1], acc[t][k]);
          acc[t][k] = fmaf(w[c][k].z, gx[2], acc[t][k]);
          acc[t][k] = fmaf(w[c][k].w, gx[3], acc[t][k]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) wave_sum_n<HKV + 1>(acc[t]);
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int k = 0; k <= HKV; ++k) s_red[wave][t][k] = acc[t][k];
  }
  __syncthreads();
  if (tid >= TT) return;
  const int tok = tok0 + tid;
  if (tok >= a.ntok) return;
  float tot[HKV + 1];
#pragma unroll
  for (int k = 0; k <= HKV; ++k) tot[k] = s_red[0][tid][k] + s_red[1][tid][k] + s_red[2][tid][k] + s_red[3][tid][k];
  const float r = 1.0f / sqrtf(tot[HKV] / static_cast<float>(a.H) + a.eps);
  const int b = tok / a.T, t = tok % a.T;
  float lg0 = 0.0f;
#pragma unroll
  for (int k = 0; k < HKV; ++k) {
    float z = r * tot[k];
    if (a.bias) z += a.bias[k];
    float lg = a.alpha * z - a.offsets[k];
    if (k == 0) lg0 = lg;
    if (a.per_layer) lg = lg0;
    const size_t o = (static_cast<size_t>(b) * HKV + k) * a.T + t;
    if (a.logits) a.logits[o] = lg;
    a.evict[o] = (!a.disable && lg > 0.0f) ? 1 : 0;
  }
}

// One token per 256-thread workgroup, bf16 hidden states with H a multiple
// of 16: thread t owns elements [16t + 4096i, 16t + 4096i + 16); its loads
// (two 16-byte pieces of h, gamma and the W rows) are all in flight at once;
// the Hkv + 1 sums reduce with DPP, then across the four waves through LDS.
template <int HKV>
__global__ __launch_bounds__(256) void decide_linear_tok_kernel(DecideArgs a) {
  __shared__ float s_red[4][HKV + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = blockIdx.x;
  const uint16_t* h = static_cast<const uint16_t*>(a.hidden) + static_cast<size_t>(tok) * a.H;
  float acc[HKV + 1];
#pragma unroll
  for (int k = 0; k <= HKV; ++k) acc[k] = 0.0f;
  for (int m = 16 * tid; m < a.H; m += 4096) {
    const uint4 h0 = *reinterpret_cast<const uint4*>(h + m);
    const uint4 h1 = *reinterpret_cast<const uint4*>(h + m + 8);
    float4 gm[4];
    float4 w[HKV][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      gm[c] = *reinterpret_cast<const float4*>(a.gamma + m + 4 * c);
#pragma unroll
      for (int k = 0; k < HKV; ++k) w[k][c] = *reinterpret_cast<const float4*>(a.W + static_cast<size_t>(k) * a.H + m + 4 * c);
    }
    const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
    float x[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(hw[i] << 16);
      x[2 * i + 1] = __uint_as_float(hw[i] & 0xFFFF0000u);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float gx[4] = {gm[c].x * x[4 * c], gm[c].y * x[4 * c + 1], gm[c].z * x[4 * c + 2], gm[c].w * x[4 * c + 3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[HKV] = fmaf(x[4 * c + e], x[4 * c + e], acc[HKV]);
#pragma unroll
      for (int k = 0; k < HKV; ++k) {
        acc[k] = fmaf(w[k][c].x, gx[0], acc[k]);
        acc[k] = fmaf(w[k][c].y, gx[1], acc[k]);
        acc[k] = fmaf(w[k][c].z, gx[2], acc[k]);
        acc[k] = fmaf(w[k][c].w, gx[3], acc[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k <= HKV; ++k) acc[k] = wave_sum_dpp(acc[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k <= HKV; ++k) s_red[wave][k] = acc[k];
  }
  __syncthreads();
  if (tid >= HKV) return;
  const float ss = s_red[0][HKV] + s_red[1][HKV] + s_red[2][HKV] + s_red[3][HKV];
  const float r = 1.0f / sqrtf(ss / static_cast<float>(a.H) + a.eps);
  auto logit = [&](int k) {
    float z = r * (s_red[0][k] + s_red[1][k] + s_red[2][k] + s_red[3][k]);
    if (a.bias) z += a.bias[k];
    return a.alpha * z - a.offsets[k];
  };
  const int k = tid;
  const float lg = a.per_layer ? logit(0) : logit(k);
  const int b = tok / a.T, t = tok % a.T;
  const size_t o = (static_cast<size_t>(b) * HKV + k) * a.T + t;
  if (a.logits) a.logits[o] = lg;
  a.evict[o] = (!a.disable && lg > 0.0f) ? 1 : 0;
}


struct QneuronArgs {
  void* q;             // [B][T][Hq][D]
  const float* offsets;
  int ntok, T, Hkv, g, D;
  float alpha;
  int per_layer, disable;
  float* logits;
  uint8_t* evict;
};

// One thread per token: read every group's neuron first, then zero them.
template <typename ACT>
__global__ void decide_qneuron_kernel(QneuronArgs a) {
  const int tok = blockIdx.x * blockDim.x + threadIdx.x;
  if (tok >= a.ntok) return;
  ACT* q = static_cast<ACT*>(a.q) + static_cast<size_t>(tok) * a.Hkv * a.g * a.D;
  const int b = tok / a.T, t = tok % a.T;
  const float lg0 = a.alpha * load_act<ACT>(q, static_cast<size_t>(a.D) - 1) - a.offsets[0];
  for (int k = 0; k < a.Hkv; ++k) {
    const size_t qi = static_cast<size_t>(k) * a.g * a.D + a.D - 1;
    const float lg = a.per_layer ? lg0 : a.alpha * load_act<ACT>(q, qi) - a.offsets[k];
    const size_t o = (static_cast<size_t>(b) * a.Hkv + k) * a.T + t;
    if (a.logits) a.logits[o] = lg;
    a.evict[o] = (!a.disable && lg > 0.0f) ? 1 : 0;
  }
  for (int k = 0; k < a.Hkv; ++k) store_act<ACT>(q, static_cast<size_t>(k) * a.g * a.D + a.D - 1, 0.0f);
}


// Prefill chunks, bf16 hidden states, H a multiple of 8: TT tokens per
// 256-thread workgroup.  Thread t owns elements [8t + 2048i, 8t + 2048i + 8)
// of each token row; per slab it keeps gamma * W_k of its 8 elements in
// registers and issues the TT 16-byte loads of h together, so h streams from
// HBM once, in full 4 KB rows per wave-instruction.  The TT x (Hkv + 1) sums
// reduce with DPP inside each wave, then across the four waves through LDS.
template <int HKV, int TT>
__global__ __launch_bounds__(256) void decide_linear_chunk_kernel(DecideArgs a) {
  __shared__ float s_red[4][TT][HKV + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok0 = blockIdx.x * TT;
  const int ntt = min(TT, a.ntok - tok0);
  const uint16_t* hb = static_cast<const uint16_t*>(a.hidden) + static_cast<size_t>(tok0) * a.H;
  float acc[TT][HKV + 1];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int k = 0; k <= HKV; ++k) acc[t][k] = 0.0f;
  for (int m = 8 * tid; m < a.H; m += 2048) {
    uint4 hv[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t)
      hv[t] = t < ntt ? *reinterpret_cast<const uint4*>(hb + static_cast<size_t>(t) * a.H + m) : make_uint4(0, 0, 0, 0);
    const float4 g0 = *reinterpret_cast<const float4*>(a.gamma + m);
    const float4 g1 = *reinterpret_cast<const float4*>(a.gamma + m + 4);
    const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    float gw[HKV][8];
#pragma unroll
    for (int k = 0; k < HKV; ++k) {
      const float4 w0 = *reinterpret_cast<const float4*>(a.W + static_cast<size_t>(k) * a.H + m);
      const float4 w1 = *reinterpret_cast<const float4*>(a.W + static_cast<size_t>(k) * a.H + m + 4);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) gw[k][e] = wv[e] * gm[e];
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const uint32_t u[4] = {hv[t].x, hv[t].y, hv[t].z, hv[t].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = __uint_as_float((e & 1) ? (u[e >> 1] & 0xFFFF0000u) : (u[e >> 1] << 16));
        acc[t][HKV] = fmaf(x, x, acc[t][HKV]);
#pragma unroll
        for (int k = 0; k < HKV; ++k) acc[t][k] = fmaf(gw[k][e], x, acc[t][k]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int k = 0; k <= HKV; ++k) acc[t][k] = wave_sum_dpp(acc[t][k]);
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int k = 0; k <= HKV; ++k) s_red[wave][t][k] = acc[t][k];
  }
  __syncthreads();
  if (tid >= ntt) return;
  const int tok = tok0 + tid;
  float tot[HKV + 1];
#pragma unroll
  for (int k = 0; k <= HKV; ++k) tot[k] = (s_red[0][tid][k] + s_red[1][tid][k]) + (s_red[2][tid][k] + s_red[3][tid][k]);
  const float r = 1.0f / sqrtf(tot[HKV] / static_cast<float>(a.H) + a.eps);
  const int b = tok / a.T, t = tok % a.T;
  float lg0 = 0.0f;
#pragma unroll
  for (int k = 0; k < HKV; ++k) {
    float z = r * tot[k];
    if (a.bias) z += a.bias[k];
    float lg = a.alpha * z - a.offsets[k];
    if (k == 0) lg0 = lg;
    if (a.per_layer) lg = lg0;
    const size_t o = (static_cast<size_t>(b) * HKV + k) * a.T + t;
    if (a.logits) a.logits[o] = lg;
    a.evict[o] = (!a.disable && lg > 0.0f) ? 1 : 0;
  }
}

// Prefill chunks on the matrix cores (bf16 hidden states, H a multiple of
// 2048, at most 8 KV heads).  decide_w_kernel first writes gamma * W of each
// head as two bf16 parts, the nearest bf16 and the rest, whose sum carries
// about 16 significant bits of the fp32 product (so z differs from the fp32
// sum by about 1e-6 of its terms' magnitude), laid out as the matrix cores
// read it.  decide_linear_mfma_kernel then takes 16 tokens per workgroup,
// each of its four waves over a quarter of H: v_mfma_f32_16x16x32_bf16 with
// the tokens as rows (A: lane (g, n) holds elements 32s + 8g.. of token n's
// row, as stored) and 16 columns (head c's two parts in columns c and c + 8),
// the hidden states streaming from HBM once with 8 to 16 steps (8-16 KB per
// wave) in flight; the sums of squares run on the vector ALU beside them.
typedef __bf16 dc_bf16x8 __attribute__((ext_vector_type(8)));
typedef float dc_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t dc_pack_bf16(float lo, float hi) {
  typedef __bf16 dc_bf16x2 __attribute__((ext_vector_type(2)));
  typedef float dc_f32x2 __attribute__((ext_vector_type(2)));
  dc_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, dc_bf16x2));
}

// gw[kb][n] = 8 bf16 of column n (head n % 8, part n / 8) for elements 8kb..8kb+7
template <int HKV>
__global__ __launch_bounds__(256) void decide_w_kernel(DecideArgs a, uint4* gw) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int kb = i >> 4, n = i & 15, c = n & 7;
  if (kb >= a.H / 8) return;
  float part[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = 8 * kb + e;
    const float p = c < HKV ? a.gamma[k] * a.W[static_cast<size_t>(c) * a.H + k] : 0.0f;
    const float hi = static_cast<float>(static_cast<__bf16>(p));
    part[e] = n >= 8 ? p - hi : p;
  }
  gw[i] = make_uint4(dc_pack_bf16(part[0], part[1]), dc_pack_bf16(part[2], part[3]), dc_pack_bf16(part[4], part[5]),
                     dc_pack_bf16(part[6], part[7]));
}

constexpr int kDcWaves = 4;

template <int HKV>
__global__ __launch_bounds__(64 * kDcWaves) void decide_linear_mfma_kernel(DecideArgs a, const uint4* __restrict__ gw) {
  constexpr int U = 8;                              // steps per round; two rounds in flight
  constexpr int NW = kDcWaves;
  __shared__ float s_acc[NW][16][16];
  __shared__ float s_ss[NW][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, n16 = lane & 15;
  const int tok0 = blockIdx.x * 16;
  const bool live = tok0 + n16 < a.ntok;
  const uint16_t* hrow = static_cast<const uint16_t*>(a.hidden) +
                         static_cast<size_t>(live ? tok0 + n16 : tok0) * a.H;
  const int kq = a.H / NW;                          // this wave's share
  const int k0 = wave * kq;
  const int nsteps = kq / 32;                       // a multiple of U
  const int nr = nsteps / U;
  dc_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float ss = 0.0f;
  uint4 ha[U], ba[U], hb[U], bb[U];
  // round r's loads (past the last round: the last round again, from cache)
  auto load = [&](uint4 (&h)[U], uint4 (&b)[U], int r) {
    const int s0 = min(r, nr - 1) * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 32 * (s0 + u) + 8 * g4;
      h[u] = *reinterpret_cast<const uint4*>(hrow + k);
      b[u] = gw[(k >> 3) * 16 + n16];
    }
  };
  auto compute = [&](const uint4 (&h)[U], const uint4 (&b)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint4 x4 = live ? h[u] : make_uint4(0, 0, 0, 0);
      const uint32_t hw[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = __uint_as_float((e & 1) ? (hw[e >> 1] & 0xFFFF0000u) : (hw[e >> 1] << 16));
        ss = fmaf(x, x, ss);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dc_bf16x8, x4),
                                                    __builtin_bit_cast(dc_bf16x8, b[u]), acc, 0, 0, 0);
    }
  };
  load(ha, ba, 0);
  for (int r = 0; r < nr; r += 2) {
    __builtin_amdgcn_sched_barrier(0);
    load(hb, bb, r + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(ha, ba);
    __builtin_amdgcn_sched_barrier(0);
    load(ha, ba, r + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (r + 1 < nr) compute(hb, bb);
  }
  // sums of squares: lane (g, n) has token n's over its elements; fold the row groups
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  // acc[i] = this wave's share of token 4g + i, column n
#pragma unroll
  for (int i = 0; i < 4; ++i) s_acc[wave][4 * g4 + i][n16] = acc[i];
  if (g4 == 0) s_ss[wave][n16] = ss;
  __syncthreads();
  if (tid >= 16 || tok0 + tid >= a.ntok) return;
  const int tok = tok0 + tid;
  float s2 = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) s2 += s_ss[w][tid];
  const float r = 1.0f / sqrtf(s2 / static_cast<float>(a.H) + a.eps);
  const int b = tok / a.T, t = tok % a.T;
  float lg0 = 0.0f;
#pragma unroll
  for (int k = 0; k < HKV; ++k) {
    float dot = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) dot += s_acc[w][tid][k] + s_acc[w][tid][k + 8];
    float z = r * dot;
    if (a.bias) z += a.bias[k];
    float lg = a.alpha * z - a.offsets[k];
    if (k == 0) lg0 = lg;
    if (a.per_layer) lg = lg0;
    const size_t o = (static_cast<size_t>(b) * HKV + k) * a.T + t;
    if (a.logits) a.logits[o] = lg;
    a.evict[o] = (!a.disable && lg > 0.0f) ? 1 : 0;
  }
}

// DMS_DECIDE_MFMA=0 keeps prefill chunks on the vector-ALU kernel.
static bool dc_mfma_enabled() {
  const char* e = std::getenv("DMS_DECIDE_MFMA");
  return !e || std::atoi(e) != 0;
}

template <typename ACT, int HKV>
static void launch_linear_h(const DecideArgs& a, uint4* gw, hipStream_t st) {
  // few tokens (decode): one token per workgroup, all loads of a thread in
  // flight at once; many tokens (prefill chunks): 8 tokens share gamma * W
  // registers (bf16), or 4 tokens share W (fp32 activations)
  if (a.ntok <= 512) {
    if (sizeof(ACT) == 2 && HKV <= 8 && a.H % 16 == 0)
      hipLaunchKernelGGL((decide_linear_tok_kernel<HKV <= 8 ? HKV : 8>), dim3(a.ntok), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((decide_linear_kernel<ACT, HKV, 1, (HKV <= 8 ? 4 : 2)>), dim3(a.ntok), dim3(256), 0, st, a);
  } else if (sizeof(ACT) == 2 && HKV <= 8 && a.H % 2048 == 0 && reinterpret_cast<uintptr_t>(a.hidden) % 16 == 0 &&
             gw && dc_mfma_enabled()) {
    constexpr int HK = HKV <= 8 ? HKV : 8;
    hipLaunchKernelGGL((decide_w_kernel<HK>), dim3((a.H / 8 * 16 + 255) / 256), dim3(256), 0, st, a, gw);
    hipLaunchKernelGGL((decide_linear_mfma_kernel<HK>), dim3((a.ntok + 15) / 16), dim3(64 * kDcWaves), 0, st, a,
                       static_cast<const uint4*>(gw));
  } else if (sizeof(ACT) == 2 && HKV <= 8 && a.H % 8 == 0 && reinterpret_cast<uintptr_t>(a.hidden) % 16 == 0) {
    constexpr int TT = 8;
    hipLaunchKernelGGL((decide_linear_chunk_kernel<HKV <= 8 ? HKV : 8, TT>), dim3((a.ntok + TT - 1) / TT), dim3(256),
                       0, st, a);
  } else {
    constexpr int NCH = HKV <= 8 ? 2 : 1;
    hipLaunchKernelGGL((decide_linear_kernel<ACT, HKV, 4, NCH>), dim3((a.ntok + 3) / 4), dim3(256), 0, st, a);
  }
}

template <typename ACT>
static void launch_linear(const DecideArgs& a, int hkv, uint4* gw, hipStream_t st) {
  switch (hkv) {
    case 1: launch_linear_h<ACT, 1>(a, gw, st); break;
    case 2: launch_linear_h<ACT, 2>(a, gw, st); break;
    case 4: launch_linear_h<ACT, 4>(a, gw, st); break;
    case 8: launch_linear_h<ACT, 8>(a, gw, st); break;
    case 16: launch_linear_h<ACT, 16>(a, gw, st); break;
    default: break;
  }
}

}  // namespace dms

using namespace dms;

extern "C" int dms_decide(dms_cache* cache, const void* hidden, const float* rms_gamma, const float* W,
                          const float* bias, const float* offsets, void* q_inout, int B, int T,
                          float* logits_out, uint8_t* evict_out, void* stream) {
  if (!cache) return fail(DMS_ERR_ARG, "cache is NULL");
  const dms_config& c = cache->cfg;
  if (B <= 0 || T <= 0) return fail(DMS_ERR_ARG, "B and T must be positive");
  if (!offsets || !evict_out) return fail(DMS_ERR_ARG, "offsets and evict_out are required");
  const bool act_f32 = c.kv_dtype == DMS_F32;
  hipStream_t st = as_stream(stream);
  if (c.decide_mode == DMS_DECIDE_LINEAR) {
    if (!hidden || !rms_gamma || !W) return fail(DMS_ERR_ARG, "hidden, rms_gamma and W are required");
    const int hkv = c.num_kv_heads;
    if (hkv != 1 && hkv != 2 && hkv != 4 && hkv != 8 && hkv != 16)
      return fail(DMS_ERR_UNSUPPORTED, "linear decision needs num_kv_heads in {1,2,4,8,16}");
    if ((reinterpret_cast<uintptr_t>(rms_gamma) | reinterpret_cast<uintptr_t>(W)) % 16 != 0)
      return fail(DMS_ERR_ARG, "rms_gamma and W must be 16-byte aligned");
    DecideArgs a{hidden, rms_gamma, W, bias, offsets, B * T, T, c.hidden, c.alpha_scale, c.rms_eps,
                 c.alpha_per == DMS_ALPHA_PER_LAYER, c.disable_eviction != 0, logits_out, evict_out};
    if (act_f32) launch_linear<float>(a, hkv, nullptr, st);
    else launch_linear<uint16_t>(a, hkv, cache->dev.decide_w, st);
  } else {
    if (!q_inout) return fail(DMS_ERR_ARG, "q_inout is required for the query-neuron decision");
    QneuronArgs a{q_inout, offsets, B * T, T, c.num_kv_heads, c.num_q_heads / c.num_kv_heads, c.head_dim,
                  c.alpha_scale, c.alpha_per == DMS_ALPHA_PER_LAYER, c.disable_eviction != 0, logits_out,
                  evict_out};
    const dim3 grid((B * T + 255) / 256), block(256);
    if (act_f32) hipLaunchKernelGGL(decide_qneuron_kernel<float>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(decide_qneuron_kernel<uint16_t>, grid, block, 0, st, a);
  }
  return check_hip(hipGetLastError(), "dms_decide launch");
}

// ---------------------------------------------------------------------------
// Training-time gating (walkthrough, Gumbel 噪声与可微门控): the decision logit
// plus the caller's noise, over the temperature, through a sigmoid; the
// straight-through decision's forward value is 1 where the probability
// exceeds 1/2, i.e. where y > 0 (taken on y, so that no rounding of the
// sigmoid near 1/2 decides it).

namespace dms {

__global__ __launch_bounds__(256) void train_gate_kernel(const float* __restrict__ logits,
                                                         const float* __restrict__ noise, float inv_tau, int64_t n,
                                                         float* __restrict__ y_out, float* __restrict__ probs_out,
                                                         float* __restrict__ hard_out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float y = (logits[i] + (noise ? noise[i] : 0.0f)) * inv_tau;
    if (y_out) y_out[i] = y;
    if (probs_out) probs_out[i] = 1.0f / (1.0f + __expf(-y));
    if (hard_out) hard_out[i] = y > 0.0f ? 1.0f : 0.0f;
  }
}

// dlogits = (dy + (dhard + dprobs) * p * (1 - p)) / tau, p = sigmoid(y); a
// missing gradient is zero.
__global__ __launch_bounds__(256) void train_gate_bwd_kernel(const float* __restrict__ logits,
                                                             const float* __restrict__ noise, float inv_tau, int64_t n,
                                                             const float* __restrict__ dy,
                                                             const float* __restrict__ dhard,
                                                             const float* __restrict__ dprobs,
                                                             float* __restrict__ dlogits) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float y = (logits[i] + (noise ? noise[i] : 0.0f)) * inv_tau;
    const float p = 1.0f / (1.0f + __expf(-y));
    const float via_p = (dhard ? dhard[i] : 0.0f) + (dprobs ? dprobs[i] : 0.0f);
    dlogits[i] = ((dy ? dy[i] : 0.0f) + via_p * (p * (1.0f - p))) * inv_tau;
  }
}

}  // namespace dms

extern "C" int dms_train_gate_bwd(const float* logits, const float* noise, float tau, int64_t n, const float* dy,
                                  const float* dhard, const float* dprobs, float* dlogits_out, void* stream) {
  if (!logits || !dlogits_out) return fail(DMS_ERR_ARG, "logits and dlogits_out are required");
  if (n < 0) return fail(DMS_ERR_ARG, "n must be non-negative");
  if (!(tau > 0.0f)) return fail(DMS_ERR_ARG, "tau must be positive");
  if (n == 0) return DMS_OK;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(train_gate_bwd_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, as_stream(stream),
                     logits, noise, 1.0f / tau, n, dy, dhard, dprobs, dlogits_out);
  return check_hip(hipGetLastError(), "dms_train_gate_bwd launch");
}

extern "C" int dms_train_gate(const float* logits, const float* noise, float tau, int64_t n, float* y_out,
                              float* probs_out, float* hard_out, void* stream) {
  if (!logits) return fail(DMS_ERR_ARG, "logits is required");
  if (n < 0) return fail(DMS_ERR_ARG, "n must be non-negative");
  if (!(tau > 0.0f)) return fail(DMS_ERR_ARG, "tau must be positive");
  if (n == 0) return DMS_OK;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(train_gate_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, as_stream(stream), logits,
                     noise, 1.0f / tau, n, y_out, probs_out, hard_out);
  return check_hip(hipGetLastError(), "dms_train_gate launch");
}
