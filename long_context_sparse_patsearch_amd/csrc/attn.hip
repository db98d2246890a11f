// Exact block-sparse (and dense) causal attention on gfx950 bf16 MFMA.
//
// Computes A(Q,K,V,S) = Softmax(QK^T/sqrt(d) + M_S) V of the digest page
// "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
// Structural-Mass-Motivated Routing" (prerequisite section on prefill and
// sparse attention; method-steps step 4), with M_S given as a block CSR, and
// the dense causal result the digest's FlashAttention baseline computes.
//
// Work item = one (head, 128-row query block); a workgroup of four waves runs
// it, wave w holding query rows 32w..32w+31 as B operands of S^T = K Q^T.
// Key blocks are walked in 64-key stages, double-buffered in LDS and filled by
// direct global->LDS loads (no register staging): the K stage row-major, the
// V stage from a V^T copy made once per call (keys contiguous per head-dim
// row), both with an XOR swizzle of the 16-byte chunks so that every operand
// read is bank-conflict free.  S^T and O^T += V^T P^T run on 32x32x16 bf16
// MFMA; the online softmax stays in fp32 registers (each lane owns one query
// column), with the 1/sqrt(d)*log2(e) scale folded into one FMA feeding exp2
// and the output rescaled only in stages where some row maximum of the wave grows.
// Two workgroups share a CU so that one wave's softmax runs under another
// wave's MFMAs.  Items come from per-XCD work queues (see Queue).
#include <math.h>

#include "crisp_device.hpp"
#include "crisp_internal.h"

namespace crisp {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int NXCD = 8;                  // accelerator complex dies of an MI355X
constexpr int KS = 64;                   // keys per pipeline stage
constexpr int WG_PER_CU = 2;
constexpr float RESCALE_LOG2 = 0.f;      // rescale whenever a row maximum grows (keeps the max weight exactly 1)
constexpr float M_INIT = -1e30f;         // running-max sentinel (finite: keeps fma/exp2 NaN-free)

template <int D>
struct Stage {
  static constexpr int KROW = D * 2;                 // bytes per K row
  static constexpr int KCPR = KROW / 16;             // 16-byte chunks per K row (8 or 16)
  static constexpr int KBYTES = KS * KROW;
  static constexpr int VROW = KS * 2;                // bytes per V^T row (64 keys)
  static constexpr int VCPR = VROW / 16;             // 8
  static constexpr int VBYTES = D * VROW;
  static constexpr int BYTES = KBYTES + VBYTES;
  static constexpr int KLOADS = KBYTES / 16 / NTHR;  // direct loads per thread per stage
  static constexpr int VLOADS = VBYTES / 16 / NTHR;
  static constexpr int NSTEP = D / 16;
};

// Physical 16-byte chunk of logical chunk c in LDS row `row`.
template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (CPR == 16) return c ^ (row & 15);
  else return c ^ ((row >> 1) & 7);
}

// One direct global->LDS load of 16 bytes per lane: lane i writes LDS bytes
// [lds_off + 16 i, lds_off + 16 i + 16).  Issued as asm so that the compiler does
// not treat the other LDS buffer as aliased and wait for these loads before
// every LDS read; the kernel waits for them itself (vm_wait) before the barrier
// that publishes a stage.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_off) : "memory", "m0");
}
// The same with a scalar base address: lane i loads 16 bytes at gbase + voff_i
// into LDS bytes [lds_base + IMM + 16 i, ...).
template <uint32_t IMM>
__device__ __forceinline__ void dma16s(uint32_t voff, const void* gbase, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds_base),
               "i"(IMM)
               : "memory", "m0", "scc");
}
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
  int per_queue;           // items per queue
};

inline int queue_chunk(int nb) {
  int qc = nb / 32;
  return qc < 1 ? 1 : (qc > 32 ? 32 : qc);
}

inline Queue make_queue(int nb, int64_t bh_total) {
  Queue qd;
  qd.nb = nb;
  qd.qc = queue_chunk(nb);
  qd.bh_total = bh_total;
  const int64_t chunks = (nb + qd.qc - 1) / qd.qc;
  qd.per_queue = (int)((chunks + NXCD - 1) / NXCD * bh_total * qd.qc);
  return qd;
}

// Item u of queue x -> (query block, head row); false for the padding past the last block.
__device__ __forceinline__ bool queue_item(const Queue& qd, int x, int u, int& qb, int64_t& bh) {
  const int64_t span = qd.bh_total * qd.qc;
  const int64_t j = u / span, rem = u % span;
  bh = rem / qd.qc;
  const int64_t qtop = (j * NXCD + x) * qd.qc + rem % qd.qc;
  if (qtop >= qd.nb) return false;
  qb = qd.nb - 1 - (int)qtop;
  return true;
}

template <int D, bool DENSE, bool OUT_BF16>
__global__ __launch_bounds__(NTHR, WG_PER_CU) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_cap,
    void* __restrict__ out, int n, int h_q, int group, Queue qd, int* __restrict__ counters, float c2) {
  using S = Stage<D>;
  __shared__ __align__(16) char lds[2 * S::BYTES];
  __shared__ int item;
  const int x = (int)(blockIdx.x % NXCD);
  const int w = wave_id(), lane = lane_id();
  const int hi = lane >> 5;
  const int qloc = 32 * w + (lane & 31);
  const int nb = n / BLK;
  const int h_kv = h_q / group;

  // per-lane LDS read offsets, the same for every stage
  const int krow = key_row_of_lane(lane & 31);                 // + 32 ks
  const int kfix = (S::KCPR == 16) ? (krow & 15) : ((krow >> 1) & 7);
  const int vrow = lane & 31;                                  // + 32 ds
  const int vfix = (vrow >> 1) & 7;
  static_assert(S::KLOADS == 2 || S::KLOADS == 4, "direct loads per stage");
  static_assert(S::VLOADS == 2 || S::VLOADS == 4, "direct loads per stage");
  // Direct-load byte offsets, the same for every stage.  Load i of wave w fills
  // LDS chunks p = (4i + w)*64 + lane of a stage buffer with the (row, logical
  // chunk) the swizzle maps there; the swizzle term does not depend on i (rows
  // advance by a multiple of its period), so load i's offset is load 0's plus
  // a fixed step (16 K rows, 32 V^T rows).
  uint32_t kdma[S::KLOADS], vdma[S::VLOADS];
  {
    const int p = w * 64 + lane;
    const int kr0 = p / S::KCPR, vr0 = p / S::VCPR;
    const uint32_t k0 = (uint32_t)(kr0 * D + swz<S::KCPR>(kr0, p % S::KCPR) * 8) * 2u;
    const uint32_t v0 = (uint32_t)(vr0 * n + swz<S::VCPR>(vr0, p % S::VCPR) * 8) * 2u;
#pragma unroll
    for (int i = 0; i < S::KLOADS; ++i) kdma[i] = k0 + i * (4 * 64 / S::KCPR * S::KROW);
#pragma unroll
    for (int i = 0; i < S::VLOADS; ++i) vdma[i] = v0 + (uint32_t)(i * (4 * 64 / S::VCPR)) * (uint32_t)n * 2u;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)(char*)lds);
  const uint32_t lds0w = lds0 + (uint32_t)__builtin_amdgcn_readfirstlane(w) * 1024u;   // this wave's first KiB

  for (;;) {
    if (threadIdx.x == 0) item = atomicAdd(&counters[x], 1);
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(item);
    __syncthreads();
    if (u >= qd.per_queue) break;
    int qb;
    int64_t bh;
    if (!queue_item(qd, x, u, qb, bh)) continue;

    const int b = (int)(bh / h_q), h = (int)(bh % h_q), g = h / group;
    const uint16_t* kg = k + ((size_t)b * h_kv + g) * n * D;
    const uint16_t* vtg = vt + ((size_t)b * h_kv + g) * (size_t)D * n;

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
    auto kb_at = [&](int64_t t) -> int { return DENSE ? (int)t : col_idx[t]; };
    auto next_valid = [&](int64_t t) -> int64_t {
      if (DENSE) return t;
      while (t < t1) {
        const int kb = kb_at(t);
        if (kb >= 0 && kb <= qb) break;
        ++t;
      }
      return t;
    };

    // issue the direct loads of stage (block kb, half hf) into buffer bf
    const char* kgb = reinterpret_cast<const char*>(kg);
    const char* vgb = reinterpret_cast<const char*>(vtg);
    auto issue = [&](int kb, int hf, int bf) {
      const int key0 = kb * BLK + hf * KS;
      const char* gk = kgb + (size_t)key0 * D * 2;
      const char* gv = vgb + (size_t)key0 * 2;
      const uint32_t lk = lds0w + bf * S::BYTES, lv = lk + S::KBYTES;
      dma16s<0>(kdma[0], gk, lk);
      dma16s<4096>(kdma[1], gk, lk);
      if constexpr (S::KLOADS > 2) {
        dma16s<8192>(kdma[2], gk, lk);
        dma16s<12288>(kdma[3], gk, lk);
      }
      dma16s<0>(vdma[0], gv, lv);
      dma16s<4096>(vdma[1], gv, lv);
      if constexpr (S::VLOADS > 2) {
        dma16s<8192>(vdma[2], gv, lv);
        dma16s<12288>(vdma[3], gv, lv);
      }
    };

    bf16x8 qf[S::NSTEP];
    {
      const uint16_t* qp = q + ((size_t)bh * n + (size_t)qb * BLK + qloc) * D + 8 * hi;
#pragma unroll
      for (int s = 0; s < S::NSTEP; ++s) qf[s] = as_bf16x8(ld16(qp + 16 * s));
      // consume the query loads here (an empty asm reading the registers), so
      // that the compiler completes them before the stage loop and places no
      // vector-memory waits inside it
      if constexpr (S::NSTEP == 8)
        asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]), "v"(qf[7]));
      else
        asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]));
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
    float m = M_INIT, l = 0.f;

    // stage sequence: (block kb, half 0), (kb, 1), (next block, 0), ...; the next
    // entry of the row is fetched one stage before it is needed and validated
    // only then (entries outside [0, qb] are skipped)
    int64_t t = next_valid(t0);
    int kb = t < t1 ? kb_at(t) : 0;
    int64_t tn = t + 1;
    int kbn = tn < t1 ? kb_at(tn) : -1;
    int hf = 0, bf = 0;
    if (t < t1) issue(kb, 0, 0);
    while (t < t1) {
      vm_wait();
      __syncthreads();
      // stage after this one: the second half of kb, or the first half of the next entry
      if (hf == 0) {
        issue(kb, 1, bf ^ 1);
      } else {
        if (!DENSE && tn < t1 && (kbn < 0 || kbn > qb)) {
          tn = next_valid(tn + 1);
          kbn = tn < t1 ? kb_at(tn) : -1;
        }
        if (tn < t1) issue(kbn, 0, bf ^ 1);
      }

      const char* kbuf = lds + bf * S::BYTES;
      const char* vbuf = kbuf + S::KBYTES;
      const bool diag = (kb == qb);
      const int kloc0 = hf * KS;                 // first key of the stage inside the block
      // a wave whose queries all precede the stage has nothing to do in it
      if (!(diag && 32 * w + 31 < kloc0)) {
        // the two 32-key accumulators alternate, so consecutive MFMAs are independent
        f32x16 s[2] = {f32x16{}, f32x16{}};
        const char* kr = kbuf + krow * S::KROW;
#pragma unroll
        for (int st = 0; st < S::NSTEP; ++st)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            s[ks] = mfma_32x32x16(as_bf16x8(ld16(kr + 32 * ks * S::KROW + ((2 * st + hi) ^ kfix) * 16)), qf[st], s[ks]);
        if (diag && 32 * w < kloc0 + KS - 1) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kloc0 + 32 * ks + key_of_reg(r, lane) > qloc) s[ks][r] = -INFINITY;
        }
        float tmax = s[0][0];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[ks][r]);
        tmax = fmaxf(tmax, xor_shfl(tmax, 32));
        const float tmu = tmax * c2;
        const bool need = tmu > m + RESCALE_LOG2;
        if (__ballot(need)) {
          const float mn = need ? tmu : m;
          const float corr = fast_exp2(m - mn);
          l *= corr;
#pragma unroll
          for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[ds][r] *= corr;
          m = mn;
        }
        const float nm = -m;
        bf16x8 pb[4];
        const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            uint32_t wv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float a0 = fast_exp2(fmaf(s[ks][8 * c + 2 * e], c2, nm));
              const float a1 = fast_exp2(fmaf(s[ks][8 * c + 2 * e + 1], c2, nm));
              wv[e] = pack_bf16x2(a0, a1);
              // the row sum uses the rounded weights, the same ones the PV product uses
              l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv[e]), one2, l, false);
            }
            pb[2 * ks + c] = as_bf16x8(make_uint4(wv[0], wv[1], wv[2], wv[3]));
          }
        }
        const char* vr = vbuf + vrow * S::VROW;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int ds = 0; ds < D / 32; ++ds)
            o[ds] = mfma_32x32x16(as_bf16x8(ld16(vr + 32 * ds * S::VROW + ((2 * cc + hi) ^ vfix) * 16)), pb[cc], o[ds]);
      }
      if (hf == 0) {
        hf = 1;
      } else {
        hf = 0;
        t = tn;
        kb = kbn;
        tn = t + 1;
        kbn = tn < t1 ? kb_at(tn) : -1;
      }
      bf ^= 1;
    }

    l += xor_shfl(l, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t orow = (size_t)bh * n + (size_t)qb * BLK + qloc;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d = 32 * ds + 8 * grp + 4 * hi;
        const float a0 = o[ds][4 * grp] * inv, a1 = o[ds][4 * grp + 1] * inv;
        const float a2 = o[ds][4 * grp + 2] * inv, a3 = o[ds][4 * grp + 3] * inv;
        if (OUT_BF16) {
          uint2 uu;
          uu.x = pack_bf16x2(a0, a1);
          uu.y = pack_bf16x2(a2, a3);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + orow * D + d) = uu;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + orow * D + d) = make_float4(a0, a1, a2, a3);
        }
      }
  }
}

// V [bg][n][D] -> V^T [bg][D][n], 64-key tiles through LDS.
template <int D>
__global__ __launch_bounds__(NTHR) void transpose_v_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt,
                                                           int n) {
  __shared__ uint16_t tile[KS][D + 2];
  const int64_t bg = blockIdx.y;
  const int key0 = blockIdx.x * KS;
  const uint16_t* src = v + ((size_t)bg * n + key0) * D;
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < KS * CPR; c += NTHR) {
    const int row = c / CPR, cc = c % CPR;
    const uint4 u = ld16(src + (size_t)row * D + cc * 8);
    const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[row][cc * 8 + 2 * j] = (uint16_t)(wds[j] & 0xFFFFu);
      tile[row][cc * 8 + 2 * j + 1] = (uint16_t)(wds[j] >> 16);
    }
  }
  __syncthreads();
  uint16_t* dst = vt + (size_t)bg * D * n + key0;
  for (int c = threadIdx.x; c < D * (KS / 8); c += NTHR) {
    const int d = c / (KS / 8), kc = c % (KS / 8);
    uint4 u;
    u.x = tile[kc * 8 + 0][d] | ((uint32_t)tile[kc * 8 + 1][d] << 16);
    u.y = tile[kc * 8 + 2][d] | ((uint32_t)tile[kc * 8 + 3][d] << 16);
    u.z = tile[kc * 8 + 4][d] | ((uint32_t)tile[kc * 8 + 5][d] << 16);
    u.w = tile[kc * 8 + 6][d] | ((uint32_t)tile[kc * 8 + 7][d] << 16);
    st16(dst + (size_t)d * n + kc * 8, u);
  }
}

__global__ void zero_counters_kernel(int* __restrict__ c) {
  if (threadIdx.x < NXCD) c[threadIdx.x] = 0;
}

int cu_count() {
  static int cus = 0;
  if (!cus) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cus = c;
  }
  return cus;
}

constexpr size_t COUNTER_BYTES = 256;

size_t vt_bytes(const Dims& dm) { return (size_t)dm.batch * dm.h_kv * dm.n * dm.d * 2; }

template <int D, bool DENSE>
hipError_t attn_launch(const Dims& dm, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int64_t* row_ptr, const int32_t* col_idx, int64_t cap, void* out,
                       int out_bf16, void* ws, hipStream_t st) {
  int* counters = static_cast<int*>(ws);
  uint16_t* vt = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + COUNTER_BYTES);
  const float c2 = LOG2E / sqrtf((float)D);
  const Queue qd = make_queue(dm.nb, dm.bh);
  const int64_t slots = (int64_t)(cu_count() * WG_PER_CU + NXCD - 1) / NXCD * NXCD;
  const int64_t items = qd.per_queue * NXCD;
  const unsigned grid = (unsigned)(items < slots ? items : slots);
  zero_counters_kernel<<<1, 64, 0, st>>>(counters);
  transpose_v_kernel<D><<<dim3(dm.n / KS, (unsigned)(dm.batch * dm.h_kv)), NTHR, 0, st>>>(v, vt, dm.n);
  if (out_bf16)
    attn_kernel<D, DENSE, true><<<grid, NTHR, 0, st>>>(q, k, vt, row_ptr, col_idx, cap, out, dm.n, dm.h_q,
                                                       dm.group, qd, counters, c2);
  else
    attn_kernel<D, DENSE, false><<<grid, NTHR, 0, st>>>(q, k, vt, row_ptr, col_idx, cap, out, dm.n, dm.h_q,
                                                        dm.group, qd, counters, c2);
  return hipGetLastError();
}

}  // namespace

size_t attn_ws_bytes(const Dims& dm) { return COUNTER_BYTES + vt_bytes(dm); }

hipError_t launch_sparse_attn(const Dims& dm, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int64_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                              void* out, int out_bf16, void* ws, hipStream_t st) {
  if (dm.d == 128)
    return attn_launch<128, false>(dm, q, k, v, row_ptr, col_idx, col_capacity, out, out_bf16, ws, st);
  return attn_launch<64, false>(dm, q, k, v, row_ptr, col_idx, col_capacity, out, out_bf16, ws, st);
}

hipError_t launch_dense_attn(const Dims& dm, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             void* out, int out_bf16, void* ws, hipStream_t st) {
  if (dm.d == 128) return attn_launch<128, true>(dm, q, k, v, nullptr, nullptr, 0, out, out_bf16, ws, st);
  return attn_launch<64, true>(dm, q, k, v, nullptr, nullptr, 0, out, out_bf16, ws, st);
}

}  // namespace crisp
