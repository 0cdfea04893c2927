// Machine-rate probes for MI355X (gfx950): a streaming HBM read and a dense
// bf16 matrix-core loop.  They measure the peaks that the DMS kernels are
// compared against (decode against HBM bandwidth, prefill against the bf16
// matrix rate), on the box itself rather than from the vendor's figures.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "dms_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Grid-stride read of n16 16-byte pieces: each thread keeps U loads in flight
// (U consecutive pieces spaced one grid apart), folds them with XOR, and
// writes nothing unless the fold equals a value no real input produces, so
// the loads stay live.  The piece count is a multiple of U * the thread count
// (the host rounds the buffer down).
template <int U>
__global__ __launch_bounds__(256) void read_kernel(const u32x4_t* __restrict__ src, size_t n16, uint32_t* sink) {
  const size_t nthreads = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * nthreads < n16; i += U * nthreads) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * nthreads);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// Each wave runs `iters` rounds of 8 independent 16x16x32 bf16 products
// (register operands, no memory traffic), each accumulating in place into its
// own registers, then stores a fold of its accumulators only if it equals an
// impossible value.  The products are written out (a compiler left to itself
// may rotate accumulators between registers with extra moves, which measures
// the moves instead of the matrix cores); eight chains keep each product's
// input well clear of the previous product on the same accumulator.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.001f * static_cast<float>((lane + e) & 7));
    b[e] = static_cast<__bf16>(0.002f * static_cast<float>((lane * 3 + e) & 7));
  }
  f32x4_t c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
        : "v"(a), "v"(b));
  }
  // let the last products finish before vector instructions read their results
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const f32x4_t t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const float s = t[0] + t[1] + t[2] + t[3];
  if (__float_as_uint(s) == 0x7FBADBADu) sink[blockIdx.x] = 1u;
}

}  // namespace

extern "C" {

int dms_probe_read(const void* buf, size_t bytes, int grid, int unroll, uint32_t* sink, void* stream) {
  if (!buf || !sink || grid <= 0) return -1;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return -1;
  const size_t nthreads = static_cast<size_t>(grid) * 256;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  size_t n16 = bytes / 16;
  switch (unroll) {
    case 4:
      n16 -= n16 % (4 * nthreads);
      hipLaunchKernelGGL(read_kernel<4>, dim3(grid), dim3(256), 0, st, static_cast<const u32x4_t*>(buf), n16, sink);
      break;
    case 8:
      n16 -= n16 % (8 * nthreads);
      hipLaunchKernelGGL(read_kernel<8>, dim3(grid), dim3(256), 0, st, static_cast<const u32x4_t*>(buf), n16, sink);
      break;
    case 16:
      n16 -= n16 % (16 * nthreads);
      hipLaunchKernelGGL(read_kernel<16>, dim3(grid), dim3(256), 0, st, static_cast<const u32x4_t*>(buf), n16, sink);
      break;
    default:
      return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

size_t dms_probe_read_bytes(size_t bytes, int grid, int unroll) {
  const size_t per = static_cast<size_t>(grid) * 256 * static_cast<size_t>(unroll);
  const size_t n16 = bytes / 16;
  return (per ? n16 - n16 % per : 0) * 16;
}

int dms_probe_mfma_bf16(int grid, int iters, uint32_t* sink, void* stream) {
  if (!sink || grid <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

double dms_probe_mfma_bf16_flops(int grid, int iters) {
  // 4 waves per workgroup, 8 products of 16 x 16 x 32 per round, 2 flops per multiply-add
  return static_cast<double>(grid) * 4.0 * 8.0 * static_cast<double>(iters) * (16.0 * 16.0 * 32.0 * 2.0);
}

}  // extern "C"
