// Internal declarations of the DMS HIP library: the device layout of one
// cache, launch helpers and small device utilities shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "dms.h"
#include "host_logic.h"

namespace dms {

constexpr int kCtlFreeCount = 0;
constexpr int kCtlStatus = 1;
constexpr int kCtlPrepArrive = 2;    // arrival counter of the fused decode decision + append
constexpr int kArriveSpinLimit = 1 << 18;   // polls (each a device-scope load and a short sleep)

// Device pointers carved out of the caller's buffer (see compute_layout).
struct DevCache {
  uint8_t* k_pages;      // [pool][P][D] kv dtype
  uint8_t* v_pages;      // [pool][P][D]
  float* scales;         // [pool][2] fp8 K/V scales
  uint32_t* page_amax;   // [pool][2] fp8 amax of the opening call (float bits)
  int32_t* slot_meta;    // [pool][P] position | evict << 31
  int32_t* page_table;   // [Bmax][Hkv][maxp]
  int32_t* lengths;      // [Bmax][Hkv]
  int32_t* ring;         // [Bmax][Hkv][w] slot | evict << 31 of position p at p % w
  int32_t* ring_row;     // [Bmax][Hkv][w] flat page row (page * P + slot % P) of that slot
  int32_t* cur_page;     // [Bmax][Hkv] page holding slot L-1 (-1: none)
  int32_t* pos;          // [Bmax]
  int32_t* free_stack;   // [pool]
  int32_t* ctl;          // [kCtlWords]
  int32_t* chunk_slot;   // [Bmax*Hkv][max_chunk] slot of each chunk token
  int32_t* chunk_info;   // [Bmax*Hkv][8]
  int32_t* unit_info;    // [kMaxUnits][4] decode: partial base, partial count, merge counter
  int32_t* arrive;       // [kArriveGroups][kArriveStride] decode step arrival counters (word 0 of each)
  int32_t* plan;         // decode plan of the fused step: [kPlanHeader] header, [Bmax] rows, [kPlanMaxWgs][kPlanRec]
  uint4* decide_w;       // [hidden / 8][16] linear adapter's gamma * W, split bf16 (prefill chunk decisions)
};

// Decode plan header words (plan[0] = 1 marks the plan valid; every other
// call that changes lengths, positions, ring entries or page tables clears it).
constexpr int kPlanValid = 0, kPlanB = 1, kPlanGrid = 2, kPlanSeqNull = 3, kPlanVariant = 4, kPlanNrec = 5;
__device__ __forceinline__ void plan_invalidate(const DevCache& d) { d.plan[kPlanValid] = 0; }

// Geometry shared by every kernel of one cache.
struct Geo {
  int Bmax, Hq, Hkv, D, g, H, w, P, maxp, pool, max_tokens, max_chunk;
  int kv_dtype;
  int Pshift;            // log2(P) when P is a power of two, else -1
  float scale_log2;      // softmax scale * log2(e)
};

}  // namespace dms

struct dms_cache {
  dms_config cfg;
  dms::Geo geo;
  dms::DevCache dev;
  dms::Layout layout;
  int device;
  int num_cus;
  int decode_grid;       // the decode attention's workgroups at most (2 per CU, or DMS_DECODE_WGS)
  bool decode_grid_fixed;  // DMS_DECODE_WGS was set: every call uses decode_grid
  int decode_np;         // passes in flight per round of the decode kernel (DMS_DECODE_NP; 0: default)
  int decode_lpr;        // lanes per row of the decode kernel (DMS_DECODE_LPR; 0: default)
  int decode_mfma;       // matrix-core decode for bf16 pages of >= 16 rows (DMS_DECODE_MFMA; default 1)
  bool force_generic;    // DMS_GENERIC_KERNELS=1: vector-ALU decode and prefill attention kernels only
  int step_fuse;         // dms_decode_step in one launch: -1 when all its workgroups fit at once (default),
                         // 0 never, 1 always (DMS_DECODE_STEP_FUSE)
  int step_blocks_per_cu;  // resident workgroups per CU of the one-launch step kernel (-1: not queried yet)
};

namespace dms {

// Error reporting (thread-local message).
int fail(int status, const std::string& msg);
int check_hip(hipError_t e, const char* what);
int decode_grid_for(const dms_cache* c);
int decode_grid_call(const dms_cache* c, int units);
// Decode attention workgroups on a device with `cus` compute units (2 per CU,
// or DMS_DECODE_WGS), capped at kMaxDecodeGrid.
int decode_grid_default(int cus);
// Partial records of one decode call: two per attention workgroup (its first
// and last unit segment may be split units) plus one per (row, KV head) unit
// (the generic kernel's records per unit), each G * (D + 2) floats.
size_t decode_workspace_bytes(int grid, int units, int g, int D);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------
// device utilities

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_act(const T* p, size_t i);
template <> __device__ __forceinline__ float load_act<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}
template <typename T> __device__ __forceinline__ void store_act(T* p, size_t i, float v);
template <> __device__ __forceinline__ void store_act<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_act<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// e4m3fn ("OCP" fp8: bias 7, largest finite 448, no infinities).
// Encode: |x| already clamped to <= 448; nearest value, ties to even code;
// a result of magnitude zero is stored as +0.
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of 2^-9
    float qf = rintf(a * 512.0f);            // exact scaling, nearest-even integer 0..8
    code = static_cast<uint32_t>(qf);        // 8 becomes the smallest normal (exp 1, man 0)
  } else {
    uint32_t au = __float_as_uint(a);
    int e = static_cast<int>((au >> 23) & 0xFF) - 127;
    uint32_t m = au & 0x7FFFFFu;
    uint32_t keep = m >> 20;
    uint32_t rem = m & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep++;
    if (keep == 8u) { keep = 0; e++; }
    code = (static_cast<uint32_t>(e + 7) << 3) | keep;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return static_cast<uint8_t>(code == 0 ? 0u : (code | sign));
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t sign = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu;
  uint32_t m = c & 0x7u;
  float mag = (e == 0) ? static_cast<float>(m) * 0.001953125f
                       : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | sign);
}

// Power-of-two page scale: the smallest 2^e with amax <= 448 * 2^e, times 4.
__device__ __forceinline__ float page_scale_from_amax(float amax) {
  if (!(amax > 0.0f)) return ldexpf(1.0f, -98);
  int k;
  float m = frexpf(amax, &k);               // amax = m * 2^k, m in [0.5, 1)
  int e = k - 9 + (m > 0.875f ? 1 : 0);
  return ldexpf(1.0f, e + 2);
}

__device__ __forceinline__ void set_status(int32_t* ctl, int bits) {
  atomicOr(reinterpret_cast<int*>(ctl + kCtlStatus), bits);
}

// ---- cross-lane reductions on DPP (full-rate VALU; no LDS crossbar) ----
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float x, float old) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, x),
                                                               CTRL, ROW_MASK, 0xF, false));
}

// Sum over the LPR (2, 4, 8 or 16) lanes of a row; every lane of the row gets it.
template <int LPR>
__device__ __forceinline__ float row_sum_dpp(float x) {
  if (LPR >= 2) x += dpp_f<0xB1, 0xF>(x, 0.0f);      // quad_perm [1,0,3,2]
  if (LPR >= 4) x += dpp_f<0x4E, 0xF>(x, 0.0f);      // quad_perm [2,3,0,1]
  if (LPR >= 8) x += dpp_f<0x141, 0xF>(x, 0.0f);     // row_half_mirror
  if (LPR >= 16) x += dpp_f<0x140, 0xF>(x, 0.0f);    // row_mirror
  return x;
}
template <int LPR>
__device__ __forceinline__ float row_max_dpp(float x) {
  if (LPR >= 2) x = fmaxf(x, dpp_f<0xB1, 0xF>(x, -INFINITY));
  if (LPR >= 4) x = fmaxf(x, dpp_f<0x4E, 0xF>(x, -INFINITY));
  if (LPR >= 8) x = fmaxf(x, dpp_f<0x141, 0xF>(x, -INFINITY));
  if (LPR >= 16) x = fmaxf(x, dpp_f<0x140, 0xF>(x, -INFINITY));
  return x;
}

// After a row-level reduction (every lane of each 16-lane row holds its row's
// value), fold the four rows: row_bcast15 feeds rows 1 and 3 from the rows
// before them, row_bcast31 feeds rows 2 and 3 from lane 31; lane 63 then
// holds the result of all four rows.
__device__ __forceinline__ float rows_sum_to_last(float x) {
  x += dpp_f<0x142, 0xA>(x, 0.0f);
  x += dpp_f<0x143, 0xC>(x, 0.0f);
  return x;
}
__device__ __forceinline__ float rows_max_to_last(float x) {
  x = fmaxf(x, dpp_f<0x142, 0xA>(x, -INFINITY));
  x = fmaxf(x, dpp_f<0x143, 0xC>(x, -INFINITY));
  return x;
}
// Fold row groups of LPR lanes inside each 16-lane row (row_ror moves lane
// i + k to lane i), so every lane of a row ends with the row's value; for
// per-column data this sums the same column of the row's groups.
template <int LPR>
__device__ __forceinline__ float fold_groups_sum(float x) {
  if (LPR <= 8) x += dpp_f<0x128, 0xF>(x, 0.0f);     // row_ror:8
  if (LPR <= 4) x += dpp_f<0x124, 0xF>(x, 0.0f);     // row_ror:4
  return x;
}
template <int LPR>
__device__ __forceinline__ float fold_groups_max(float x) {
  if (LPR <= 8) x = fmaxf(x, dpp_f<0x128, 0xF>(x, -INFINITY));
  if (LPR <= 4) x = fmaxf(x, dpp_f<0x124, 0xF>(x, -INFINITY));
  return x;
}

__device__ __forceinline__ float lane63(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
// Whole-wave sum / max, returned to every lane.
__device__ __forceinline__ float wave_sum_dpp(float x) { return lane63(rows_sum_to_last(row_sum_dpp<16>(x))); }
__device__ __forceinline__ float wave_max_dpp(float x) { return lane63(rows_max_to_last(row_max_dpp<16>(x))); }

// Wave-wide (64 lanes) prefix count of a predicate: returns the number of set
// lanes below this one; *total receives the wave's count.
__device__ __forceinline__ int wave_rank(bool pred, int* total) {
  uint64_t m = __ballot(pred);
  int lane = threadIdx.x & 63;
  uint64_t below = (lane == 0) ? 0ull : (m & ((~0ull) >> (64 - lane)));
  *total = __popcll(m);
  return __popcll(below);
}

}  // namespace dms
