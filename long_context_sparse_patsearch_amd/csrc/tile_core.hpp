// The 128x128 QK^T tile core on bf16 MFMA, shared by the proxy passes and the
// attention kernels.
//
// A workgroup of four waves owns one 128-row query block; wave w owns query
// rows 32w..32w+31 and keeps them in registers as the B operand of
// S^T = K Q^T (so each lane's accumulators belong to one query column and the
// softmax row statistics need only the lane and its partner lane l^32).
// K tiles are staged through LDS with a padded row stride.
#pragma once

#include "crisp_device.hpp"

namespace crisp {

template <int D>
struct Tile {
  static constexpr int KSTR = D + 8;                  // LDS row stride of a K tile (bf16 elements)
  static constexpr int NSTEP = D / 16;                // MFMA k-steps over the head dimension
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int KCH = BLK * CPR / NTHR;        // 16-byte K loads per thread per tile
  static constexpr int KLDS = BLK * KSTR;             // bf16 elements of one K tile in LDS
};

// The wave's 32 query rows (row 0 at `qrows`) as B operands of S^T = K Q^T.
template <int D>
__device__ __forceinline__ void load_q_operands(const uint16_t* __restrict__ qrows,
                                                bf16x8 (&qf)[Tile<D>::NSTEP]) {
  const int lane = lane_id();
  const uint16_t* p = qrows + (size_t)(lane & 31) * D + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < Tile<D>::NSTEP; ++s) qf[s] = as_bf16x8(ld16(p + 16 * s));
}

// Global -> registers part of staging a [128][D] K tile.
template <int D>
__device__ __forceinline__ void load_k_regs(const uint16_t* __restrict__ ktile, uint4 (&r)[Tile<D>::KCH]) {
#pragma unroll
  for (int i = 0; i < Tile<D>::KCH; ++i) {
    const int c = i * NTHR + threadIdx.x;
    r[i] = ld16(ktile + (size_t)(c / Tile<D>::CPR) * D + (c % Tile<D>::CPR) * 8);
  }
}

// Registers -> LDS part of staging a K tile.
template <int D>
__device__ __forceinline__ void store_k_lds(uint16_t* __restrict__ klds, const uint4 (&r)[Tile<D>::KCH]) {
#pragma unroll
  for (int i = 0; i < Tile<D>::KCH; ++i) {
    const int c = i * NTHR + threadIdx.x;
    st16(klds + (c / Tile<D>::CPR) * Tile<D>::KSTR + (c % Tile<D>::CPR) * 8, r[i]);
  }
}

// S^T for one 128-key tile against the wave's 32 queries.  s[ks] holds keys
// 32ks + key_of_reg(r, lane) for query column lane%32, unscaled dot products.
template <int D>
__device__ __forceinline__ void qk_tile(const uint16_t* __restrict__ klds,
                                        const bf16x8 (&qf)[Tile<D>::NSTEP], f32x16 (&s)[4]) {
  const int lane = lane_id();
  const uint16_t* base = klds + key_row_of_lane(lane & 31) * Tile<D>::KSTR + 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    f32x16 acc = {};
    const uint16_t* p = base + 32 * ks * Tile<D>::KSTR;
#pragma unroll
    for (int st = 0; st < Tile<D>::NSTEP; ++st) acc = mfma_32x32x16(as_bf16x8(ld16(p + 16 * st)), qf[st], acc);
    s[ks] = acc;
  }
}

}  // namespace crisp
