// dms_kvzap_score: the KVzap scorers and their threshold.
//
// KVzap-linear page ("动态内存稀疏化（DMS）策略：KVzap-linear-Llama-3.1-8B-Instruct的核心创新点",
// KVzap-linear的技术架构): one float32 linear layer from the layer's hidden
// state (4096) to one score per KV head (8):  s = W . h + b.
// KVzap-mlp page ("革命性LLM加速技术：NVIDIA KVzap-mlp-Qwen3-8B如何实现高效KV缓存修剪？",
// 模型架构): two layers with a GELU between them:  s = W2 . gelu(W1 . h + b1) + b2
// (inner width 512 for Qwen3-8B).  Both pages: a token is pruned when its
// score is below the threshold (-4 by default) once it has left the window of
// the last 128 tokens; the decision goes to the delayed-eviction cache as
// evict = [s < threshold] (window 128 in the cache configuration).
//
// Linear: HBM-bound on h (2 bytes per element of bf16 against Hkv FMAs);
// same structure as the DMS adapter's projection without the RMSNorm.
// MLP, more than 16 tokens: W1 . h is a dense [N x H] by [H x Hm] contraction
// and runs on the matrix cores in fp32 (v_mfma_f32_16x16x4_f32: bf16 hidden
// states widen exactly, weights stay fp32, so scores keep fp32 accuracy and
// decisions agree with a float64 reference away from the threshold); each
// workgroup takes 64 tokens by 64 inner units, applies b1 and the GELU in
// registers and writes its share of W2 . gelu(...) to the caller's workspace.
// MLP, up to 16 tokens (decode): bound by reading W1 once; workgroups of 4
// inner units reduce over H with all tokens' activations in registers, then
// write their share the same way.  A last pass adds the shares in a fixed
// order (deterministic scores) with b2 and applies the threshold.
#include <algorithm>
#include <cmath>

#include "dms_internal.h"

namespace dms {
namespace {

struct KzArgs {
  const void* hidden;   // [N][H] activations (f32 or bf16), N = B * T
  const float* W1;      // linear: [Hkv][H]; MLP: [Hm][H]
  const float* b1;      // linear: [Hkv]; MLP: [Hm]; or null
  const float* W2;      // MLP: [Hkv][Hm]
  const float* b2;      // MLP: [Hkv] or null
  int N, T, H, Hkv, Hm;
  float thr;
  float* scores;        // [B][Hkv][T] or null
  uint8_t* evict;       // [B][Hkv][T]
  float* part;          // MLP: [parts][N][Hkv] shares of the inner-unit workgroups
  int parts;
};

typedef float kz_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ size_t out_index(const KzArgs& a, int n, int k) {
  const int b = n / a.T, t = n % a.T;
  return (static_cast<size_t>(b) * a.Hkv + k) * a.T + t;
}

template <typename ACT> __device__ __forceinline__ void load4(const ACT* p, float (&x)[4]);
template <> __device__ __forceinline__ void load4<float>(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x;
  x[1] = v.y;
  x[2] = v.z;
  x[3] = v.w;
}
template <> __device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  x[0] = __uint_as_float(v.x << 16);
  x[1] = __uint_as_float(v.x & 0xFFFF0000u);
  x[2] = __uint_as_float(v.y << 16);
  x[3] = __uint_as_float(v.y & 0xFFFF0000u);
}

__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Wave reduce-scatter of 64 values: afterwards lane l holds the sum over the
// wave of v[l] in v[0].  Each step exchanges half of the remaining values
// with the partner lane (lane ^ C/2) and keeps the half its lane bit selects:
// 32 + 16 + ... + 1 = 63 shuffles instead of 6 per value.
template <int C>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[64], int lane) {
  if constexpr (C > 1) {
    constexpr int H = C / 2;
    const bool up = (lane & H) != 0;            // this lane keeps the upper half
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float mine = up ? v[i + H] : v[i];
      const float other = up ? v[i] : v[i + H];
      v[i] = mine + __shfl_xor(other, H);
    }
    reduce_scatter_step<H>(v, lane);
  }
}

__device__ __forceinline__ void wave_reduce_scatter64(float (&v)[64], int lane) { reduce_scatter_step<64>(v, lane); }

// The same for V <= 64 values (a power of two): afterwards every lane l
// holds the wave sum of v[l % V] in v[0].
template <int V, int C>
__device__ __forceinline__ void reduce_scatter_v(float (&v)[V], int lane) {
  if constexpr (C > 1) {
    constexpr int H = C / 2;
    const bool up = (lane & H) != 0;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float mine = up ? v[i + H] : v[i];
      const float other = up ? v[i] : v[i + H];
      v[i] = mine + __shfl_xor(other, H);
    }
    reduce_scatter_v<V, H>(v, lane);
  }
}
template <int V>
__device__ __forceinline__ void wave_sum_scatter(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "a power of two up to 64");
  reduce_scatter_v<V, V>(v, lane);
#pragma unroll
  for (int o = V; o < 64; o <<= 1) v[0] += __shfl_xor(v[0], o);
}

template <typename ACT> __device__ __forceinline__ void load8(const ACT* p, float (&x)[8]) {
  float a[4], b[4];
  load4<ACT>(p, a);
  load4<ACT>(p + 4, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

constexpr int kSmallThreads = 512;   // decode-size workgroups: 8 elements of H per thread and pass
constexpr int kSmallTokens = 16;     // tokens per decode-size workgroup

// Decode-size dot products: workgroup (x, y) takes R weight rows
// [R x, R x + R) and tokens [16 y, 16 y + 16); thread t owns elements
// [8t + 4096i, 8t + 4096i + 8) of H, all its loads of a pass issued
// together (one round of loads per 4096 elements).  Returns, in lanes of
// wave 0 ... (through LDS), the R x 16 sums.
template <typename ACT, int R>
__device__ __forceinline__ void small_dots(const KzArgs& a, const float* W, int nrows, int r0, int n0,
                                           float (&s_red)[8][R * kSmallTokens]) {
  constexpr int NT = kSmallTokens;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float acc[R * NT];
#pragma unroll
  for (int i = 0; i < R * NT; ++i) acc[i] = 0.0f;
  for (int m = 8 * tid; m < a.H; m += 8 * kSmallThreads) {
    float w[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r0 + r < nrows) {
        load8<float>(W + static_cast<size_t>(r0 + r) * a.H + m, w[r]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[r][e] = 0.0f;
      }
    }
    float x[NT][8];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n0 + n < a.N) {
        load8<ACT>(static_cast<const ACT*>(a.hidden) + static_cast<size_t>(n0 + n) * a.H + m, x[n]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[n][e] = 0.0f;
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r * NT + n] = fmaf(w[r][e], x[n][e], acc[r * NT + n]);
  }
  wave_sum_scatter<R * NT>(acc, lane);
  if (lane < R * NT) s_red[wave][lane] = acc[0];
  __syncthreads();
}

// Linear scorer, up to 64 tokens: workgroup (k, y) takes head k and tokens [16 y, 16 y + 16).
template <typename ACT>
__global__ __launch_bounds__(kSmallThreads) void kz_linear_small_kernel(KzArgs a) {
  __shared__ float s_red[8][kSmallTokens];
  const int k = blockIdx.x, n0 = blockIdx.y * kSmallTokens;
  small_dots<ACT, 1>(a, a.W1, a.Hkv, k, n0, s_red);
  const int tid = threadIdx.x;
  if (tid < kSmallTokens && n0 + tid < a.N) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) s += s_red[w][tid];
    if (a.b1) s += a.b1[k];
    const size_t o = out_index(a, n0 + tid, k);
    if (a.scores) a.scores[o] = s;
    a.evict[o] = s < a.thr ? 1 : 0;
  }
}

// Four activations as loaded (bf16 pairs or f32), widened to f32 later.
template <typename ACT> struct Raw4;
template <> struct Raw4<float> {
  typedef float4 T;
  __device__ static T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ static void widen(const T& v, float (&x)[4]) {
    x[0] = v.x;
    x[1] = v.y;
    x[2] = v.z;
    x[3] = v.w;
  }
};
template <> struct Raw4<uint16_t> {
  typedef uint2 T;
  __device__ static T zero() { return make_uint2(0u, 0u); }
  __device__ static void widen(const T& v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x << 16);
    x[1] = __uint_as_float(v.x & 0xFFFF0000u);
    x[2] = __uint_as_float(v.y << 16);
    x[3] = __uint_as_float(v.y & 0xFFFF0000u);
  }
};

// The linear scorers' last step: each wave's TT x HKV partial dot products
// summed over its lanes, the four waves' sums through LDS, then bias,
// score and threshold for token tok0 + t and head k (one thread each).
template <int HKV, int TT>
__device__ __forceinline__ void kz_linear_finish(float (&acc)[TT * HKV], float (&s_red)[4][TT][HKV],
                                                 const KzArgs& a, int tok0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (TT * HKV == 64) {
    wave_reduce_scatter64(acc, lane);
    (&s_red[wave][0][0])[lane] = acc[0];
  } else {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
      for (int i = 0; i < TT * HKV; ++i) acc[i] += __shfl_xor(acc[i], o);
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < TT * HKV; ++i) (&s_red[wave][0][0])[i] = acc[i];
    }
  }
  __syncthreads();
  if (tid >= TT * a.Hkv) return;
  const int t = tid / a.Hkv, k = tid % a.Hkv;
  const int tok = tok0 + t;
  if (tok >= a.N) return;
  float s = s_red[0][t][k] + s_red[1][t][k] + s_red[2][t][k] + s_red[3][t][k];
  if (a.b1) s += a.b1[k];
  const size_t o = out_index(a, tok, k);
  if (a.scores) a.scores[o] = s;
  a.evict[o] = s < a.thr ? 1 : 0;
}

// Linear scorer: TT tokens per 256-thread workgroup; thread t owns elements
// [4t + 1024i, 4t + 1024i + 4) and keeps its W values in registers for the
// TT tokens; waves reduce with shuffles, the four waves through LDS.
// HKV bounds the heads (a.Hkv <= HKV).
template <typename ACT, int HKV, int TT>
__global__ __launch_bounds__(256) void kz_linear_kernel(KzArgs a) {
  __shared__ float s_red[4][TT][HKV];
  const int tid = threadIdx.x;
  const int tok0 = blockIdx.x * TT;
  float acc[TT * HKV];
#pragma unroll
  for (int i = 0; i < TT * HKV; ++i) acc[i] = 0.0f;
  for (int m = 4 * tid; m < a.H; m += 1024) {
    float4 w[HKV];
#pragma unroll
    for (int k = 0; k < HKV; ++k)
      w[k] = k < a.Hkv ? *reinterpret_cast<const float4*>(a.W1 + static_cast<size_t>(k) * a.H + m)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (tok0 + t < a.N) load4<ACT>(static_cast<const ACT*>(a.hidden) + static_cast<size_t>(tok0 + t) * a.H + m, x);
#pragma unroll
      for (int k = 0; k < HKV; ++k) {
        float& c = acc[t * HKV + k];
        c = fmaf(w[k].x, x[0], c);
        c = fmaf(w[k].y, x[1], c);
        c = fmaf(w[k].z, x[2], c);
        c = fmaf(w[k].w, x[3], c);
      }
    }
  }
  kz_linear_finish<HKV, TT>(acc, s_red, a, tok0);
}

// Linear scorer for H <= 1024 NS: as kz_linear_kernel, but every slab's
// hidden-state loads are issued before the first product, so a thread's rows
// arrive after one memory latency instead of one per slab (the grid holds
// only a few waves per SIMD to hide them).
template <typename ACT, int HKV, int TT, int NS>
__global__ __launch_bounds__(256) void kz_linear_pre_kernel(KzArgs a) {
  __shared__ float s_red[4][TT][HKV];
  const int tid = threadIdx.x;
  const int tok0 = blockIdx.x * TT;
  typedef typename Raw4<ACT>::T R;
  R raw[NS][TT];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int m = 4 * tid + 1024 * sl;
#pragma unroll
    for (int t = 0; t < TT; ++t)
      raw[sl][t] = (m < a.H && tok0 + t < a.N)
                       ? *reinterpret_cast<const R*>(static_cast<const ACT*>(a.hidden) +
                                                     static_cast<size_t>(tok0 + t) * a.H + m)
                       : Raw4<ACT>::zero();
  }
  float acc[TT * HKV];
#pragma unroll
  for (int i = 0; i < TT * HKV; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int m = 4 * tid + 1024 * sl;
    if (m < a.H) {
      float4 w[HKV];
#pragma unroll
      for (int k = 0; k < HKV; ++k)
        w[k] = k < a.Hkv ? *reinterpret_cast<const float4*>(a.W1 + static_cast<size_t>(k) * a.H + m)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        float x[4];
        Raw4<ACT>::widen(raw[sl][t], x);
#pragma unroll
        for (int k = 0; k < HKV; ++k) {
          float& c = acc[t * HKV + k];
          c = fmaf(w[k].x, x[0], c);
          c = fmaf(w[k].y, x[1], c);
          c = fmaf(w[k].z, x[2], c);
          c = fmaf(w[k].w, x[3], c);
        }
      }
    }
  }
  kz_linear_finish<HKV, TT>(acc, s_red, a, tok0);
}

// MLP: s = b2 + the inner-unit workgroups' shares (a fixed order of
// additions), then the threshold.  Up to 16 shares: one thread per score
// with its loads unrolled; more: one wave per score.
constexpr int kFinalThreadParts = 16;

__device__ __forceinline__ void kz_store(const KzArgs& a, int64_t i, float s) {
  const int n = static_cast<int>(i / a.Hkv), k = static_cast<int>(i % a.Hkv);
  if (a.b2) s += a.b2[k];
  const size_t o = out_index(a, n, k);
  if (a.scores) a.scores[o] = s;
  a.evict[o] = s < a.thr ? 1 : 0;
}

__global__ __launch_bounds__(256) void kz_finalize_thread_kernel(KzArgs a) {
  const int64_t total = static_cast<int64_t>(a.N) * a.Hkv;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  float v[kFinalThreadParts];
#pragma unroll
  for (int p = 0; p < kFinalThreadParts; ++p) v[p] = p < a.parts ? a.part[p * total + i] : 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int p = 0; p < kFinalThreadParts; ++p) s += v[p];
  kz_store(a, i, s);
}

__global__ __launch_bounds__(256) void kz_finalize_wave_kernel(KzArgs a) {
  const int64_t total = static_cast<int64_t>(a.N) * a.Hkv;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= total) return;
  float s = 0.0f;
  for (int p = lane; p < a.parts; p += 64) s += a.part[p * total + i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) kz_store(a, i, s);
}

constexpr int kGemvTokens = 16;   // at most this many tokens on the MLP's decode-size path
constexpr int kGemvUnits = 4;     // inner units per workgroup

// MLP, N <= 16 tokens: workgroup x owns inner units [4x, 4x + 4) for all
// tokens (one round of loads: W1 is read once over the grid), then writes
// its share of the second layer.
template <typename ACT>
__global__ __launch_bounds__(kSmallThreads) void kz_mlp_gemv_kernel(KzArgs a) {
  constexpr int NT = kSmallTokens, HP = kGemvUnits;
  __shared__ float s_red[8][HP * NT];
  __shared__ float s_act[NT][HP];
  const int tid = threadIdx.x;
  const int u0 = blockIdx.x * HP;
  small_dots<ACT, HP>(a, a.W1, a.Hm, u0, 0, s_red);
  if (tid < NT * HP) {
    const int j = tid / NT, n = tid % NT;          // value index r * NT + n
    float act = 0.0f;
    if (n < a.N && u0 + j < a.Hm) {
      float z = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) z += s_red[w][tid];
      if (a.b1) z += a.b1[u0 + j];
      act = gelu_erf(z);
    }
    s_act[n][j] = act;
  }
  __syncthreads();
  if (tid < NT * a.Hkv) {
    const int n = tid / a.Hkv, k = tid % a.Hkv;
    if (n < a.N) {
      float p = 0.0f;
#pragma unroll
      for (int j = 0; j < HP; ++j)
        if (u0 + j < a.Hm) p = fmaf(a.W2[static_cast<size_t>(k) * a.Hm + u0 + j], s_act[n][j], p);
      a.part[(static_cast<int64_t>(blockIdx.x) * a.N + n) * a.Hkv + k] = p;
    }
  }
}

constexpr int kMfTok = 64;        // tokens per workgroup
constexpr int kMfUnits = 64;      // inner units per workgroup
constexpr int kMfK = 32;          // H elements per LDS stage
constexpr int kMfLd = kMfK + 1;   // padded LDS row

// MLP, more than 16 tokens: workgroup (x, y) takes tokens [64x, 64x + 64) and
// inner units [64y, 64y + 64).  Wave w computes the 16 x 64 block of
// z = h . W1^T for tokens 16w.. as four 16 x 16 fp32 MFMA tiles; per stage of
// 32 elements of H the hidden rows (widened to fp32) and the W1 rows go
// through LDS.  In a 16x16x4 f32 MFMA, lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and receives D[4 (l / 16) + v][l % 16] in element v.
template <typename ACT>
__global__ __launch_bounds__(256) void kz_mlp_mfma_kernel(KzArgs a) {
  __shared__ float hs[kMfTok][kMfLd];
  __shared__ float ws[kMfUnits][kMfLd];
  __shared__ float w2s[16][kMfUnits];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok0 = blockIdx.x * kMfTok, u0 = blockIdx.y * kMfUnits;
  kz_f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = kz_f32x4{0.f, 0.f, 0.f, 0.f};
  // stage fill: thread t loads row t / 4 (a token and an inner unit), 8 elements at (t % 4) * 8
  const int fr = tid >> 2, fc = (tid & 3) * 8;
  const int ftok = tok0 + fr;
  const ACT* hrow = static_cast<const ACT*>(a.hidden) + static_cast<size_t>(ftok < a.N ? ftok : 0) * a.H;
  const float* wrow = a.W1 + static_cast<size_t>(u0 + fr) * a.H;
  for (int k0 = 0; k0 < a.H; k0 += kMfK) {
    float xh[8], xw[8];
    if (ftok < a.N) {
      float t4[4];
      load4<ACT>(hrow + k0 + fc, t4);
#pragma unroll
      for (int e = 0; e < 4; ++e) xh[e] = t4[e];
      load4<ACT>(hrow + k0 + fc + 4, t4);
#pragma unroll
      for (int e = 0; e < 4; ++e) xh[4 + e] = t4[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xh[e] = 0.0f;
    }
    {
      float t4[4];
      load4<float>(wrow + k0 + fc, t4);
#pragma unroll
      for (int e = 0; e < 4; ++e) xw[e] = t4[e];
      load4<float>(wrow + k0 + fc + 4, t4);
#pragma unroll
      for (int e = 0; e < 4; ++e) xw[4 + e] = t4[e];
    }
    __syncthreads();   // the previous stage's reads are done
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hs[fr][fc + e] = xh[e];
      ws[fr][fc + e] = xw[e];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kMfK; kk += 4) {
      const float av = hs[16 * wave + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float bv = ws[16 * c + (lane & 15)][kk + (lane >> 4)];
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[c], 0, 0, 0);
      }
    }
  }
  for (int i = tid; i < a.Hkv * kMfUnits; i += 256)
    w2s[i / kMfUnits][i % kMfUnits] = a.W2[static_cast<size_t>(i / kMfUnits) * a.Hm + u0 + i % kMfUnits];
  __syncthreads();
  // acc[c][v]: token tok0 + 16 wave + 4 (lane / 16) + v, inner unit u0 + 16 c + lane % 16
  float act[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float bias = a.b1 ? a.b1[u0 + 16 * c + (lane & 15)] : 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) act[c][v] = gelu_erf(acc[c][v] + bias);
  }
  for (int k = 0; k < a.Hkv; ++k) {
    float p[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) p[v] = fmaf(w2s[k][16 * c + (lane & 15)], act[c][v], p[v]);
    }
    // sum over the 16 lanes of the same tokens (lane % 16 = inner unit)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) p[v] += __shfl_xor(p[v], o);
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = tok0 + 16 * wave + 4 * (lane >> 4) + v;
        if (tok < a.N) a.part[(static_cast<int64_t>(blockIdx.y) * a.N + tok) * a.Hkv + k] = p[v];
      }
    }
  }
}

template <typename ACT>
int launch_kvzap(const KzArgs& a, hipStream_t st) {
  if (a.Hm == 0) {
    if (a.N <= 4 * kSmallTokens) {
      hipLaunchKernelGGL((kz_linear_small_kernel<ACT>), dim3(a.Hkv, (a.N + kSmallTokens - 1) / kSmallTokens),
                         dim3(kSmallThreads), 0, st, a);
    } else {
      if (a.H <= 4096) {
        if (a.Hkv <= 8) hipLaunchKernelGGL((kz_linear_pre_kernel<ACT, 8, 8, 4>), dim3((a.N + 7) / 8), dim3(256), 0, st, a);
        else hipLaunchKernelGGL((kz_linear_pre_kernel<ACT, 16, 4, 4>), dim3((a.N + 3) / 4), dim3(256), 0, st, a);
      } else if (a.Hkv <= 8) {
        hipLaunchKernelGGL((kz_linear_kernel<ACT, 8, 8>), dim3((a.N + 7) / 8), dim3(256), 0, st, a);
      } else {
        hipLaunchKernelGGL((kz_linear_kernel<ACT, 16, 4>), dim3((a.N + 3) / 4), dim3(256), 0, st, a);
      }
    }
    return check_hip(hipGetLastError(), "kz_linear_kernel launch");
  }
  const int64_t total = static_cast<int64_t>(a.N) * a.Hkv;
  if (a.N <= kGemvTokens) {
    hipLaunchKernelGGL((kz_mlp_gemv_kernel<ACT>), dim3(a.parts), dim3(kSmallThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((kz_mlp_mfma_kernel<ACT>), dim3((a.N + kMfTok - 1) / kMfTok, a.parts), dim3(256), 0, st, a);
  }
  if (a.parts <= kFinalThreadParts)
    hipLaunchKernelGGL(kz_finalize_thread_kernel, dim3(static_cast<int>((total + 255) / 256)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(kz_finalize_wave_kernel, dim3(static_cast<int>((total + 3) / 4)), dim3(256), 0, st, a);
  return check_hip(hipGetLastError(), "kvzap MLP launch");
}

}  // namespace
}  // namespace dms

using namespace dms;

namespace {
int kvzap_parts(int64_t n, int Hm) {
  if (Hm == 0) return 0;
  return n <= kGemvTokens ? (Hm + kGemvUnits - 1) / kGemvUnits : Hm / kMfUnits;
}
}  // namespace

extern "C" int dms_kvzap_workspace_bytes(int B, int T, int Hkv, int Hm, size_t* bytes) {
  if (!bytes || B < 0 || T < 0 || Hkv <= 0 || Hm < 0) return fail(DMS_ERR_ARG, "bad sizes or NULL bytes");
  const int64_t n = static_cast<int64_t>(B) * T;
  *bytes = static_cast<size_t>(kvzap_parts(n, Hm)) * static_cast<size_t>(n) * Hkv * sizeof(float);
  return DMS_OK;
}

extern "C" int dms_kvzap_score(int B, int T, int H, int Hkv, int Hm, int act_dtype, const void* hidden,
                               const float* W1, const float* b1, const float* W2, const float* b2, float threshold,
                               float* scores_out, uint8_t* evict_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (B < 0 || T < 0 || H <= 0 || Hkv <= 0 || Hm < 0) return fail(DMS_ERR_ARG, "bad sizes");
  const int64_t n = static_cast<int64_t>(B) * T;
  if (n > (1LL << 31) - 1) return fail(DMS_ERR_ARG, "B * T too large");
  if (n == 0) return DMS_OK;   // nothing to score (empty tensors may carry null pointers)
  if (!hidden || !W1 || !evict_out) return fail(DMS_ERR_ARG, "hidden, W1 and evict_out are required");
  if (act_dtype != DMS_F32 && act_dtype != DMS_BF16) return fail(DMS_ERR_UNSUPPORTED, "activations must be f32 or bf16");
  if (Hkv > 16) return fail(DMS_ERR_UNSUPPORTED, "at most 16 KV heads");
  if (H % kMfK != 0) return fail(DMS_ERR_UNSUPPORTED, "H must be a multiple of 32");
  if (Hm % kMfUnits != 0) return fail(DMS_ERR_UNSUPPORTED, "the MLP inner width must be a multiple of 64");
  if (reinterpret_cast<uintptr_t>(hidden) % 16 || reinterpret_cast<uintptr_t>(W1) % 16)
    return fail(DMS_ERR_UNSUPPORTED, "hidden and W1 must be 16-byte aligned");
  if (!std::isfinite(threshold)) return fail(DMS_ERR_ARG, "threshold must be finite");
  const int parts = kvzap_parts(n, Hm);
  if (Hm > 0) {
    if (!W2) return fail(DMS_ERR_ARG, "the MLP scorer needs W2");
    const size_t need = static_cast<size_t>(parts) * static_cast<size_t>(n) * Hkv * sizeof(float);
    if (!workspace || workspace_bytes < need)
      return fail(DMS_ERR_CAPACITY, "workspace smaller than dms_kvzap_workspace_bytes");
  }
  KzArgs a{hidden, W1, b1, W2, b2, static_cast<int>(n), T, H, Hkv, Hm, threshold, scores_out, evict_out,
           static_cast<float*>(workspace), parts};
  hipStream_t st = as_stream(stream);
  return act_dtype == DMS_F32 ? launch_kvzap<float>(a, st) : launch_kvzap<uint16_t>(a, st);
}
