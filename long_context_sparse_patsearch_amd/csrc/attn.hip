// Exact block-sparse (and dense) causal attention on gfx950 bf16 MFMA.
//
// Computes A(Q,K,V,S) = Softmax(QK^T/sqrt(d) + M_S) V of the digest page
// "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
// Structural-Mass-Motivated Routing" (prerequisite section on prefill and
// sparse attention; method-steps step 4), with M_S given as a block CSR, and
// the dense causal result the digest's FlashAttention baseline computes.
//
// One workgroup (four waves) per (head, query block).  Wave w keeps query rows
// 32w..32w+31 in registers.  For every selected key block the K tile (row
// major) and the V tile (transposed: keys contiguous per head-dim row) are
// staged in LDS, S^T = K Q^T runs on 32x32x16 bf16 MFMA, the online softmax
// runs in fp32 registers (each lane owns one query column, so row statistics
// need only the lane and lane^32), P is rounded to bf16 in place and
// O^T += V^T P^T runs on the same MFMA.  Global loads of the next tile are
// issued before the current tile's MFMA work.
#include <math.h>

#include "crisp_internal.h"
#include "tile_core.hpp"

namespace crisp {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int NXCD = 8;   // accelerator complex dies of an MI355X

template <int D>
struct VTile {
  static constexpr int VSTR = BLK + 8;                 // LDS row stride of V^T (bf16 elements)
  static constexpr int VLDS = D * VSTR;
  static constexpr int NB8 = (BLK / 8) * (D / 8);      // 8x8 sub-blocks per tile
  static constexpr int PER_THR = (NB8 + NTHR - 1) / NTHR;
};

// Global -> registers: thread t loads 8 consecutive key rows x 8 head-dim
// values (one 8x8 sub-block).  Sub-block id = t: head-dim group t/16, key group t%16.
template <int D>
__device__ __forceinline__ void load_v_regs(const uint16_t* __restrict__ vtile, uint4 (&r)[8]) {
  const int blk = threadIdx.x;
  if (blk < VTile<D>::NB8) {
    const int d0 = 8 * (blk >> 4), k0 = 8 * (blk & 15);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = ld16(vtile + (size_t)(k0 + i) * D + d0);
  }
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// Registers -> LDS, transposing the 8x8 sub-block so that V^T[d][k0..k0+7] is one 16-byte row.
template <int D>
__device__ __forceinline__ void store_vt_lds(uint16_t* __restrict__ vlds, const uint4 (&r)[8]) {
  const int blk = threadIdx.x;
  if (blk < VTile<D>::NB8) {
    const int d0 = 8 * (blk >> 4), k0 = 8 * (blk & 15);
    uint32_t w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w[i][0] = r[i].x; w[i][1] = r[i].y; w[i][2] = r[i].z; w[i][3] = r[i].w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint4 o;
      const int word = j >> 1;
      if (j & 1) {
        o.x = hi_pair(w[0][word], w[1][word]); o.y = hi_pair(w[2][word], w[3][word]);
        o.z = hi_pair(w[4][word], w[5][word]); o.w = hi_pair(w[6][word], w[7][word]);
      } else {
        o.x = lo_pair(w[0][word], w[1][word]); o.y = lo_pair(w[2][word], w[3][word]);
        o.z = lo_pair(w[4][word], w[5][word]); o.w = lo_pair(w[6][word], w[7][word]);
      }
      st16(vlds + (d0 + j) * VTile<D>::VSTR + k0, o);
    }
  }
}

// Work queues.  Items are (head, query block) rows.  Queue x (one per XCD;
// workgroup i serves queue i % 8, and workgroups are dispatched to XCDs
// round-robin) holds the chunks c = x, x+8, x+16, ... of QC consecutive query
// blocks counted from the last one (longest causal rows first); inside a
// chunk the items run head by head, so the CUs of an XCD work on adjacent
// query blocks of one head at once and share its K/V tiles in their L2.
// Workgroups take items from the queue's counter until it runs dry, so the
// work balances whatever the heads' routes and row lengths.
struct Queue {
  int nb, qc;              // query blocks per head; chunk length
  int64_t bh_total;        // batch * h_q
  int64_t per_queue;       // items per queue
};

__host__ __device__ inline int queue_chunk(int nb) {
  int qc = nb / 32;
  return qc < 1 ? 1 : (qc > 32 ? 32 : qc);
}

__host__ inline Queue make_queue(int nb, int64_t bh_total) {
  Queue qd;
  qd.nb = nb;
  qd.qc = queue_chunk(nb);
  qd.bh_total = bh_total;
  const int64_t chunks = (nb + qd.qc - 1) / qd.qc;
  qd.per_queue = (chunks + NXCD - 1) / NXCD * bh_total * qd.qc;
  return qd;
}

// Item u of queue x -> (query block, head row); false for the padding past the last block.
__device__ __forceinline__ bool queue_item(const Queue& qd, int x, int64_t u, int& qb, int64_t& bh) {
  const int64_t span = qd.bh_total * qd.qc;
  const int64_t j = u / span, rem = u % span;
  bh = rem / qd.qc;
  const int64_t qtop = (j * NXCD + x) * qd.qc + rem % qd.qc;
  if (qtop >= qd.nb) return false;
  qb = qd.nb - 1 - (int)qtop;
  return true;
}

template <int D, bool DENSE, bool OUT_BF16>
__device__ __forceinline__ void attn_row(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_cap,
    void* __restrict__ out, int n, int h_q, int group, int qb, int64_t bh, float c2,
    uint16_t* __restrict__ klds, uint16_t* __restrict__ vlds) {
  const int nb = n / BLK;
  const int b = (int)(bh / h_q), h = (int)(bh % h_q);
  const int h_kv = h_q / group, g = h / group;
  const uint16_t* qh = q + (size_t)bh * n * D;
  const uint16_t* kg = k + ((size_t)b * h_kv + g) * n * D;
  const uint16_t* vg = v + ((size_t)b * h_kv + g) * n * D;
  const int w = wave_id(), lane = lane_id();
  const int qloc = 32 * w + (lane & 31);

  int64_t t0, t1;
  if (DENSE) {
    t0 = 0;
    t1 = qb + 1;
  } else {
    const int64_t r = bh * nb + qb;
    t0 = row_ptr[r];
    t1 = row_ptr[r + 1];
    t0 = t0 < 0 ? 0 : (t0 > col_cap ? col_cap : t0);
    t1 = t1 < t0 ? t0 : (t1 > col_cap ? col_cap : t1);
  }
  auto kb_at = [&](int64_t t) -> int {
    return DENSE ? (int)t : __builtin_amdgcn_readfirstlane(col_idx[t]);
  };
  auto next_valid = [&](int64_t t) -> int64_t {
    if (DENSE) return t;
    while (t < t1) {
      const int kb = kb_at(t);
      if (kb >= 0 && kb <= qb) break;
      ++t;
    }
    return t;
  };

  bf16x8 qf[Tile<D>::NSTEP];
  load_q_operands<D>(qh + (size_t)(qb * BLK + 32 * w) * D, qf);

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  int64_t t = next_valid(t0);
  uint4 kr[Tile<D>::KCH];
  uint4 vr[8];
  if (t < t1) {
    const int kb = kb_at(t);
    load_k_regs<D>(kg + (size_t)kb * BLK * D, kr);
    load_v_regs<D>(vg + (size_t)kb * BLK * D, vr);
  }
  while (t < t1) {
    const int kb = kb_at(t);
    store_k_lds<D>(klds, kr);
    store_vt_lds<D>(vlds, vr);
    __syncthreads();
    const int64_t tn = next_valid(t + 1);
    if (tn < t1) {
      const int kbn = kb_at(tn);
      load_k_regs<D>(kg + (size_t)kbn * BLK * D, kr);
      load_v_regs<D>(vg + (size_t)kbn * BLK * D, vr);
    }

    f32x16 s[4];
    qk_tile<D>(klds, qf, s);
    const bool diag = (kb == qb);
    float tmax = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[ks][r] * c2;
        if (diag && 32 * ks + key_of_reg(r, lane) > qloc) x = -INFINITY;
        s[ks][r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, xor_shfl(tmax, 32));
    const float mn = fmaxf(m, tmax);
    const float corr = fast_exp2(m - mn);
    m = mn;
    float ls = 0.f;
    bf16x8 pb[8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(s[ks][r] - mn);
        ls += p[r];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint4 u;
        u.x = pack_bf16x2(p[8 * c + 0], p[8 * c + 1]);
        u.y = pack_bf16x2(p[8 * c + 2], p[8 * c + 3]);
        u.z = pack_bf16x2(p[8 * c + 4], p[8 * c + 5]);
        u.w = pack_bf16x2(p[8 * c + 6], p[8 * c + 7]);
        pb[2 * ks + c] = as_bf16x8(u);
      }
    }
    l = l * corr + ls;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[ds][r] *= corr;

    const uint16_t* vb = vlds + (lane & 31) * VTile<D>::VSTR + 8 * (lane >> 5);
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        o[ds] = mfma_32x32x16(as_bf16x8(ld16(vb + 32 * ds * VTile<D>::VSTR + 16 * c)), pb[c], o[ds]);
    __syncthreads();
    t = tn;
  }

  l += xor_shfl(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t orow = (size_t)bh * n + (size_t)qb * BLK + qloc;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int d = 32 * ds + 8 * grp + 4 * (lane >> 5);
      const float a0 = o[ds][4 * grp] * inv, a1 = o[ds][4 * grp + 1] * inv;
      const float a2 = o[ds][4 * grp + 2] * inv, a3 = o[ds][4 * grp + 3] * inv;
      if (OUT_BF16) {
        uint2 u;
        u.x = pack_bf16x2(a0, a1);
        u.y = pack_bf16x2(a2, a3);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + orow * D + d) = u;
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + orow * D + d) = make_float4(a0, a1, a2, a3);
      }
    }
}

template <int D, bool DENSE, bool OUT_BF16>
__global__ __launch_bounds__(NTHR) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_cap,
    void* __restrict__ out, int n, int h_q, int group, Queue qd, int* __restrict__ counters, float c2) {
  __shared__ __align__(16) uint16_t klds[Tile<D>::KLDS];
  __shared__ __align__(16) uint16_t vlds[VTile<D>::VLDS];
  __shared__ int64_t item;
  const int x = (int)(blockIdx.x % NXCD);
  for (;;) {
    if (threadIdx.x == 0) item = atomicAdd(&counters[x], 1);
    __syncthreads();
    const int64_t u = item;
    __syncthreads();
    if (u >= qd.per_queue) break;
    int qb;
    int64_t bh;
    if (!queue_item(qd, x, u, qb, bh)) continue;
    attn_row<D, DENSE, OUT_BF16>(q, k, v, row_ptr, col_idx, col_cap, out, n, h_q, group, qb, bh, c2, klds, vlds);
  }
}

__global__ void zero_counters_kernel(int* __restrict__ c) {
  if (threadIdx.x < NXCD) c[threadIdx.x] = 0;
}

int workgroup_slots() {
  static int slots = 0;
  if (!slots) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    slots = cus;   // one attention workgroup fits per CU (register file and LDS)
  }
  return slots;
}

template <int D, bool DENSE>
hipError_t attn_launch(const Dims& dm, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int64_t* row_ptr, const int32_t* col_idx, int64_t cap, void* out,
                       int out_bf16, int* counters, hipStream_t st) {
  const float c2 = LOG2E / sqrtf((float)D);
  const Queue qd = make_queue(dm.nb, dm.bh);
  int slots = workgroup_slots();
  slots = (slots + NXCD - 1) / NXCD * NXCD;
  const int64_t items = qd.per_queue * NXCD;
  const unsigned grid = (unsigned)(items < slots ? (items + NXCD - 1) / NXCD * NXCD : slots);
  zero_counters_kernel<<<1, 64, 0, st>>>(counters);
  if (out_bf16)
    attn_kernel<D, DENSE, true><<<grid, NTHR, 0, st>>>(q, k, v, row_ptr, col_idx, cap, out, dm.n, dm.h_q,
                                                       dm.group, qd, counters, c2);
  else
    attn_kernel<D, DENSE, false><<<grid, NTHR, 0, st>>>(q, k, v, row_ptr, col_idx, cap, out, dm.n, dm.h_q,
                                                        dm.group, qd, counters, c2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const Dims& dm, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int64_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                              void* out, int out_bf16, void* ws, hipStream_t st) {
  int* counters = static_cast<int*>(ws);
  if (dm.d == 128)
    return attn_launch<128, false>(dm, q, k, v, row_ptr, col_idx, col_capacity, out, out_bf16, counters, st);
  return attn_launch<64, false>(dm, q, k, v, row_ptr, col_idx, col_capacity, out, out_bf16, counters, st);
}

hipError_t launch_dense_attn(const Dims& dm, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             void* out, int out_bf16, void* ws, hipStream_t st) {
  int* counters = static_cast<int*>(ws);
  if (dm.d == 128) return attn_launch<128, true>(dm, q, k, v, nullptr, nullptr, 0, out, out_bf16, counters, st);
  return attn_launch<64, true>(dm, q, k, v, nullptr, nullptr, 0, out, out_bf16, counters, st);
}

size_t attn_ws_bytes() { return 256; }

}  // namespace crisp
