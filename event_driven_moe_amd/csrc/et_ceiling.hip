// et_ceiling.hip -- microbenchmarks of the device's two roofs, for the
// roofline fractions the measurements report (no workload uses them).
//
//   MFMA-only: every wave issues chains of v_mfma_f32_16x16x32_bf16 on
//   register operands (no memory traffic), eight independent accumulators
//   per wave so each MFMA issues at the unit's throughput, one workgroup of
//   four waves per compute unit -- the sustained bf16 matrix rate, at the
//   clock the device holds under that load.
//   Streaming read: 16-byte loads of a buffer in a grid-stride loop, four in
//   flight per lane, folded into a register so none is dead -- the sustained
//   HBM read rate once the buffer exceeds the caches.
#include <hip/hip_runtime.h>

#include "../../include/et.h"
#include "et_device.hpp"

namespace et {

// The MFMAs are written as one asm block of eight with each accumulator tied
// to its own registers: with the builtin, the compiler moved the loop-carried
// accumulators between registers every iteration (v_accvgpr moves and nops
// between the MFMAs), which measured the moves, not the matrix unit.
//
// Operands: small constants (the same bits in every lane), or -- with `ops`
// -- a fragment pair each lane loads from memory once (operand values decide
// how much the matrix unit switches, and the device's clock under the load
// follows its power).  `stamps`: per workgroup the shader clock counter and
// the 100 MHz real-time counter at the start and at the end, so the clock
// the loop ran at is their ratio.
__global__ __launch_bounds__(kThreads, 1) void ceiling_mfma_kernel(const i32x4* ops, float* out,
                                                                   long long* stamps, int iters) {
  const int lane = threadIdx.x & 63;
  i32x4 a, b;
  if (ops) {
    const size_t i = 2 * ((size_t)blockIdx.x * kThreads + threadIdx.x);
    a = ops[i];
    b = ops[i + 1];
  } else {
    // small finite bf16 operands (exponent field well below all ones)
    const int v = 0x3c003c00 + (lane << 2);
    a = i32x4{v, v + 1, v + 2, v + 3};
    b = i32x4{v + 4, v + 5, v + 6, v + 7};
  }
  if (stamps && threadIdx.x == 0) {
    stamps[4 * blockIdx.x] = __builtin_amdgcn_s_memtime();
    stamps[4 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
  }
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int it = 0; it < iters; ++it) {
    // four rounds of the eight chains per block; the leading nop covers the
    // write of the operands by ordinary instructions before the first round
    asm volatile(
        "s_nop 4\n\t"
        ".rept 4\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7\n\t"
        ".endr"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
        : "v"(a), "v"(b));
  }
  // the results of the last MFMAs are read by ordinary instructions next:
  // wait out the matrix pipeline's write latency explicitly
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const f32x4 t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  __syncthreads();
  if (stamps && threadIdx.x == 0) {
    stamps[4 * blockIdx.x + 2] = __builtin_amdgcn_s_memtime();
    stamps[4 * blockIdx.x + 3] = __builtin_amdgcn_s_memrealtime();
  }
  if (lane == 0) out[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = (t[0] + t[1]) + (t[2] + t[3]);
}

__global__ __launch_bounds__(kThreads) void ceiling_stream_kernel(const i32x4* src, size_t n16,
                                                                  int* out) {
  i32x4 acc = {0, 0, 0, 0};
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const i32x4 a0 = src[i], a1 = src[i + stride], a2 = src[i + 2 * stride], a3 = src[i + 3 * stride];
    acc ^= a0 ^ a1 ^ a2 ^ a3;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const int r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = r;
}

}  // namespace et

using namespace et;

extern "C" {

int et_ceiling_mfma(const void* operands, float* out, long long* stamps, int iters,
                    hipStream_t stream) {
  if (!out || iters <= 0) return ET_EINVAL;
  if ((reinterpret_cast<uintptr_t>(operands) & 15) != 0) return ET_EINVAL;
  const int g = et_num_workers();
  if (g < 0) return -g;
  hipLaunchKernelGGL(ceiling_mfma_kernel, dim3(g), dim3(kThreads), 0, stream,
                     static_cast<const i32x4*>(operands), out, stamps, iters);
  return hipGetLastError() == hipSuccess ? ET_OK : ET_EHIP;
}

int et_ceiling_stream(const void* src, size_t bytes, int* out, int wgs_per_cu, hipStream_t stream) {
  if (!src || !out || bytes < 16 || wgs_per_cu < 1 || wgs_per_cu > 16) return ET_EINVAL;
  if ((reinterpret_cast<uintptr_t>(src) & 15) != 0) return ET_EINVAL;
  const int g = et_num_workers();
  if (g < 0) return -g;
  hipLaunchKernelGGL(ceiling_stream_kernel, dim3(g * wgs_per_cu), dim3(kThreads), 0, stream,
                     static_cast<const i32x4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? ET_OK : ET_EHIP;
}

}  // extern "C"
