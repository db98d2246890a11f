// Sustained bf16 MFMA rate of the running GPU, for the benchmark's roofline.
//
// One workgroup of 512 threads per CU (two waves per SIMD); every wave issues
// v_mfma_f32_32x32x16_bf16 back to back on four accumulators, with A and B
// operands rotating through eight register sets loaded from the caller's
// buffer.  On a power-limited part the rate depends on the operand data
// (random bf16 sustains less than the published peak, zeros about the peak),
// so the caller passes the data to test.
#include "crisp_device.hpp"
#include "crisp_internal.h"

namespace crisp {

namespace {

typedef int i32x4p __attribute__((ext_vector_type(4)));
typedef float f32x16p __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void mfma_probe_kernel(const i32x4p* __restrict__ src, float* __restrict__ sink,
                                                         int iters) {
  i32x4p a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[(threadIdx.x * 16 + i) & 4095];
    b[i] = src[(threadIdx.x * 16 + 8 + i) & 4095];
  }
  f32x16p c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c0) : "v"(a[j]), "v"(b[(j + 1) & 7]));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c1) : "v"(a[(j + 2) & 7]), "v"(b[(j + 3) & 7]));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c2) : "v"(a[(j + 4) & 7]), "v"(b[(j + 5) & 7]));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c3) : "v"(a[(j + 6) & 7]), "v"(b[(j + 7) & 7]));
    }
  }
  // wait states before VALU code reads the accumulators written by the asm MFMAs
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  if (threadIdx.x == 0) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    sink[blockIdx.x % PROBE_SINK_FLOATS] = s;
  }
}

}  // namespace

hipError_t launch_mfma_probe(const void* operands, float* sink, int iters, double* flop, hipStream_t st) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  mfma_probe_kernel<<<cus, 512, 0, st>>>(static_cast<const i32x4p*>(operands), sink, iters);
  *flop = (double)cus * 8.0 * (double)iters * 32.0 * 32768.0;
  return hipGetLastError();
}

}  // namespace crisp
