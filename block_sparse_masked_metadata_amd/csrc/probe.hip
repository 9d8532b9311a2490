// Machine probe for the measurement harness (libbsm_probe.so, not part of
// the attention path): the dense bf16 MFMA rate this GPU sustains and the
// shader clock it runs at while doing so.  The attention kernels' TFLOP/s
// are reported against both the published peak and this measured one.
//
// Each wave issues `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16
// (8 accumulator chains, operands in registers, no memory traffic).  Lane 0 of
// every wave records the shader cycle counter and the constant 100 MHz
// real-time counter before and after; their ratio is the shader clock.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(int32_t iters, uint64_t* stamps, float* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][lane & 15];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    stamps[wave * 4 + 0] = t0;
    stamps[wave * 4 + 1] = t1;
    stamps[wave * 4 + 2] = r0;
    stamps[wave * 4 + 3] = r1;
  }
  if (s == 1234.5f) sink[wave] = s;  // keeps the chains live
}

}  // namespace

extern "C" {

// blocks workgroups of 256 threads (4 waves); stamps: device uint64[blocks * 4
// * 4] (per wave: cycle start, cycle end, real-time start, real-time end);
// sink: device float[blocks * 4], written only in a case that never occurs.
// Stream-ordered on `stream`; 0 on success, -1 on bad arguments, -4 when
// the launch fails.  FLOPs per launch: blocks * 4 * iters * 8 * 32768.
int bsm_probe_mfma(int32_t blocks, int32_t iters, uint64_t* stamps, float* sink, void* stream) {
  if (blocks < 1 || iters < 1 || !stamps || !sink) return -1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, iters, stamps,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
