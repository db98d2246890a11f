// Device helpers shared by the CRISP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace crisp {

constexpr int BLK = 128;      // block size B == proxy size b == anchor width
constexpr int NTHR = 256;     // threads per workgroup of the tile kernels (4 waves)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// wave index, known to the compiler to be uniform across the wave
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l supplies A[row l%32][k 8*(l/32) .. +7] and B[k 8*(l/32) .. +7][col l%32];
// accumulator register r of lane l holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32-key sub-tile that lane l loads as its A (key) operand in the
// S^T = K Q^T product.  Swapping quads 1 and 2 inside each 16-row half makes
// accumulator register r of lane l hold key 16*(r/8) + 8*(l/32) + r%8, which is
// exactly the k-index order the following P^T operand of O^T = V^T P^T needs,
// so the S^T accumulators convert to bf16 B operands in place.
__device__ __forceinline__ int key_row_of_lane(int l32) {
  return (l32 & ~12) | (((l32 >> 2) & 1) << 3) | (((l32 >> 3) & 1) << 2);
}
// Key (inside a 32-key sub-tile) held by accumulator register r of lane l.
__device__ __forceinline__ int key_of_reg(int r, int lane) {
  return 16 * (r >> 3) + 8 * (lane >> 5) + (r & 7);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Two floats -> packed bf16 pair (low half = lo), one v_cvt_pk_bf16_f32
// (round to nearest even under the default rounding mode).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Fixed-order butterfly sum over the 64 lanes of a wave (every lane gets the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += xor_shfl(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, xor_shfl(v, m));
  return v;
}

}  // namespace crisp
