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
// Three kernels: delta (one wave per query row and head); dk/dv/dy, one
// workgroup per 64 keys of a (sequence, KV head), each wave owning 16 keys
// whose K and V fragments stay in registers while it walks the causal query
// blocks of its group's heads; dq, one workgroup per 64 queries of a
// (sequence, query head), each wave owning 16 queries whose Q and dO
// fragments stay in registers while it walks their causal key blocks.  The
// four products of a 16 x 16 block run on bf16 16x16x16 matrix cores (fp32
// accumulation); P and dS are rounded to bf16 as products' operands, as in
// the forward.  Layout of a 16x16x16 product D = A B: lane l supplies
// A[l % 16][4 (l / 16) + 0..3] and B[4 (l / 16) + 0..3][l % 16] and holds
// D[4 (l / 16) + v][l % 16] in element v, so the scores of S = Q K^T
// (rows queries, columns keys) are, lane by lane, the A operand of
// dV = P^T dO and dK = dS^T Q, and those of S^T = K Q^T the A operand of
// dQ = dS K.
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
  float* dq;              // [B][T][Hq][D] f32
  float* dk;              // [B][T][Hkv][D] f32
  float* dv;
  float* dy;              // [B][Hkv][T] f32
  int B, T, Hq, Hkv, w;
  float scale;
};

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

__device__ __forceinline__ short to_bf16(float f) {
  return static_cast<short>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

// 4 consecutive bf16 at p (8-byte aligned) as an MFMA operand; zeros when !ok
__device__ __forceinline__ tb_s4 frag4(const uint16_t* p, bool ok) {
  if (!ok) return tb_s4{0, 0, 0, 0};
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return tb_s4{static_cast<short>(u.x & 0xFFFF), static_cast<short>(u.x >> 16), static_cast<short>(u.y & 0xFFFF),
               static_cast<short>(u.y >> 16)};
}

// logsigmoid(-y) = -softplus(y), stable for either sign
__device__ __forceinline__ float penalty(float yv) { return -(fmaxf(yv, 0.0f) + log1pf(__expf(-fabsf(yv)))); }

__global__ __launch_bounds__(256) void train_bwd_delta_kernel(BwdArgs a, int D) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);   // (b, t, h) row of O
  const int64_t rows = static_cast<int64_t>(a.B) * a.T * a.Hq;
  if (r >= rows) return;
  float s = 0.0f;
  for (int d = lane; d < D; d += 64) s = fmaf(bf(a.dout[r * D + d]), bf(a.o[r * D + d]), s);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) {
    const int h = static_cast<int>(r % a.Hq);
    const int64_t bt = r / a.Hq;
    const int t = static_cast<int>(bt % a.T), b = static_cast<int>(bt / a.T);
    a.delta[(static_cast<int64_t>(b) * a.Hq + h) * a.T + t] = s;
  }
}

// Workgroup (tile, pair): keys [64 tile, 64 tile + 64) of (b, kv); wave w
// owns keys k0 = 64 tile + 16 w .. + 16.
template <int D, int G>
__global__ __launch_bounds__(256) void train_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, l4 = lane >> 4;
  const int pair = blockIdx.y, b = pair / a.Hkv, kv = pair % a.Hkv;
  const int k0 = blockIdx.x * 64 + wave * 16;
  if (k0 >= a.T) return;
  const int key = k0 + l16;                 // this lane's key (column of S)
  const bool key_ok = key < a.T;
  // K and V fragments of the wave's keys (B operands of S = Q K^T, dP = dO V^T)
  tb_s4 kf[KS], vf[KS];
  const size_t krow = ((static_cast<size_t>(b) * a.T + (key_ok ? key : 0)) * a.Hkv + kv) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = frag4(a.k + krow + 16 * ks + 4 * l4, key_ok);
    vf[ks] = frag4(a.v + krow + 16 * ks + 4 * l4, key_ok);
  }
  const float yk = key_ok ? a.y[(static_cast<int64_t>(b) * a.Hkv + kv) * a.T + key] : 0.0f;
  const float pen = penalty(yk);
  tb_f4 dk[KS], dv[KS];
#pragma unroll
  for (int dt = 0; dt < KS; ++dt) {
    dk[dt] = tb_f4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = tb_f4{0.f, 0.f, 0.f, 0.f};
  }
  float dyacc = 0.0f;
  const float sl2 = a.scale * kLog2e;
  for (int i0 = (k0 / 16) * 16; i0 < a.T; i0 += 16) {
#pragma unroll 1
    for (int hh = 0; hh < G; ++hh) {
      const int h = kv * G + hh;
      // A operands: Q and dO rows of query i0 + l16
      const int qa = i0 + l16;
      const bool qa_ok = qa < a.T;
      const size_t qrow = ((static_cast<size_t>(b) * a.T + (qa_ok ? qa : 0)) * a.Hq + h) * D;
      tb_f4 s = tb_f4{0.f, 0.f, 0.f, 0.f}, dp = tb_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(frag4(a.q + qrow + 16 * ks + 4 * l4, qa_ok), kf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(frag4(a.dout + qrow + 16 * ks + 4 * l4, qa_ok), vf[ks], dp, 0,
                                                      0, 0);
      }
      // element e: query i0 + 4 l4 + e, key `key`
      short pa[4], da[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int qi = i0 + 4 * l4 + e;
        float p = 0.0f, ds = 0.0f;
        if (qi < a.T && key_ok && qi >= key) {
          const int64_t li = (static_cast<int64_t>(b) * a.Hq + h) * a.T + qi;
          const bool penalised = qi - key >= a.w;
          const float x = s[e] * sl2 + (penalised ? pen * kLog2e : 0.0f) - a.lse[li] * kLog2e;
          p = __builtin_amdgcn_exp2f(x);
          ds = p * (dp[e] - a.delta[li]);
          if (penalised) dyacc += ds;
        }
        pa[e] = to_bf16(p);
        da[e] = to_bf16(ds);
      }
      const tb_s4 pA = tb_s4{pa[0], pa[1], pa[2], pa[3]}, dA = tb_s4{da[0], da[1], da[2], da[3]};
      // dV += P^T dO, dK += dS^T Q: B operands dO / Q [query 4 l4 + e][d 16 dt + l16]
#pragma unroll
      for (int dt = 0; dt < KS; ++dt) {
        short ob[4], qb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qi = i0 + 4 * l4 + e;
          const bool ok = qi < a.T;
          const size_t r = ((static_cast<size_t>(b) * a.T + (ok ? qi : 0)) * a.Hq + h) * D + 16 * dt + l16;
          ob[e] = ok ? static_cast<short>(a.dout[r]) : 0;
          qb[e] = ok ? static_cast<short>(a.q[r]) : 0;
        }
        dv[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pA, tb_s4{ob[0], ob[1], ob[2], ob[3]}, dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dA, tb_s4{qb[0], qb[1], qb[2], qb[3]}, dk[dt], 0, 0, 0);
      }
    }
  }
  // dK, dV: element v of tile dt is key k0 + 4 l4 + v, dim 16 dt + l16
#pragma unroll
  for (int dt = 0; dt < KS; ++dt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = k0 + 4 * l4 + e;
      if (kk < a.T) {
        const size_t r = ((static_cast<size_t>(b) * a.T + kk) * a.Hkv + kv) * D + 16 * dt + l16;
        a.dk[r] = dk[dt][e] * a.scale;
        a.dv[r] = dv[dt][e];
      }
    }
  }
  // dy: this lane's key summed over the four query groups (lanes l16 + 16 m)
  dyacc += __shfl_xor(dyacc, 16);
  dyacc += __shfl_xor(dyacc, 32);
  if (l4 == 0 && key_ok) {
    const float sig = 1.0f / (1.0f + __expf(-yk));
    a.dy[(static_cast<int64_t>(b) * a.Hkv + kv) * a.T + key] = -sig * dyacc;
  }
}

// Workgroup (tile, row): queries [64 tile, 64 tile + 64) of (b, h); wave w
// owns queries q0 = 64 tile + 16 w .. + 16.
template <int D, int G>
__global__ __launch_bounds__(256) void train_bwd_dq_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, l4 = lane >> 4;
  const int row = blockIdx.y, b = row / a.Hq, h = row % a.Hq, kv = h / G;
  const int q0 = blockIdx.x * 64 + wave * 16;
  if (q0 >= a.T) return;
  const int qi = q0 + l16;                  // this lane's query (column of S^T)
  const bool q_ok = qi < a.T;
  const size_t qrow = ((static_cast<size_t>(b) * a.T + (q_ok ? qi : 0)) * a.Hq + h) * D;
  tb_s4 qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = frag4(a.q + qrow + 16 * ks + 4 * l4, q_ok);
    of[ks] = frag4(a.dout + qrow + 16 * ks + 4 * l4, q_ok);
  }
  const int64_t li = (static_cast<int64_t>(b) * a.Hq + h) * a.T + (q_ok ? qi : 0);
  const float lse2 = q_ok ? a.lse[li] * kLog2e : 0.0f;
  const float dlt = q_ok ? a.delta[li] : 0.0f;
  tb_f4 dq[KS];
#pragma unroll
  for (int dt = 0; dt < KS; ++dt) dq[dt] = tb_f4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.scale * kLog2e;
  const int kend = min(a.T, q0 + 16);
  for (int j0 = 0; j0 < kend; j0 += 16) {
    // A operands: K and V rows of key j0 + l16
    const int ka = j0 + l16;
    const bool ka_ok = ka < a.T;
    const size_t krow = ((static_cast<size_t>(b) * a.T + (ka_ok ? ka : 0)) * a.Hkv + kv) * D;
    tb_f4 s = tb_f4{0.f, 0.f, 0.f, 0.f}, dp = tb_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(frag4(a.k + krow + 16 * ks + 4 * l4, ka_ok), qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(frag4(a.v + krow + 16 * ks + 4 * l4, ka_ok), of[ks], dp, 0, 0, 0);
    }
    // element e: key j0 + 4 l4 + e, query qi
    short da[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kj = j0 + 4 * l4 + e;
      float ds = 0.0f;
      if (q_ok && kj < a.T && kj <= qi) {
        const bool penalised = qi - kj >= a.w;
        float x = s[e] * sl2 - lse2;
        if (penalised) x += penalty(a.y[(static_cast<int64_t>(b) * a.Hkv + kv) * a.T + kj]) * kLog2e;
        const float p = __builtin_amdgcn_exp2f(x);
        ds = p * (dp[e] - dlt);
      }
      da[e] = to_bf16(ds);
    }
    const tb_s4 dA = tb_s4{da[0], da[1], da[2], da[3]};
    // dQ += dS K: B operand K [key 4 l4 + e][d 16 dt + l16]
#pragma unroll
    for (int dt = 0; dt < KS; ++dt) {
      short kb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kj = j0 + 4 * l4 + e;
        const bool ok = kj < a.T;
        kb[e] = ok ? static_cast<short>(a.k[((static_cast<size_t>(b) * a.T + kj) * a.Hkv + kv) * D + 16 * dt + l16]) : 0;
      }
      dq[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dA, tb_s4{kb[0], kb[1], kb[2], kb[3]}, dq[dt], 0, 0, 0);
    }
  }
  // element v of tile dt: query q0 + 4 l4 + v, dim 16 dt + l16
#pragma unroll
  for (int dt = 0; dt < KS; ++dt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int qq = q0 + 4 * l4 + e;
      if (qq < a.T) a.dq[((static_cast<size_t>(b) * a.T + qq) * a.Hq + h) * D + 16 * dt + l16] = dq[dt][e] * a.scale;
    }
  }
}

template <int D, int G>
void launch_bwd(const BwdArgs& a, hipStream_t st) {
  const int tiles = (a.T + 63) / 64;
  hipLaunchKernelGGL((train_bwd_dkdv_kernel<D, G>), dim3(tiles, a.B * a.Hkv), dim3(256), 0, st, a);
  hipLaunchKernelGGL((train_bwd_dq_kernel<D, G>), dim3(tiles, a.B * a.Hq), dim3(256), 0, st, a);
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
  *bytes = static_cast<size_t>(B) * T * num_q_heads * sizeof(float);
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
  const size_t need = static_cast<size_t>(B) * T * num_q_heads * sizeof(float);
  if (!workspace || workspace_bytes < need)
    return fail(DMS_ERR_CAPACITY, "workspace smaller than dms_train_attn_bwd_workspace_bytes");
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(dout);
  if (al % 8) return fail(DMS_ERR_UNSUPPORTED, "q, k, v and dout must be 8-byte aligned");
  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.y = gate_logits;
  a.lse = lse;
  a.delta = static_cast<float*>(workspace);
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
  hipLaunchKernelGGL(train_bwd_delta_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, st, a,
                     head_dim);
  const int g = num_q_heads / num_kv_heads;
  const int s = head_dim == 128 ? launch_bwd_d<128>(a, g, st) : launch_bwd_d<64>(a, g, st);
  if (s) return s;
  return check_hip(hipGetLastError(), "dms_train_attn_bwd launch");
}
