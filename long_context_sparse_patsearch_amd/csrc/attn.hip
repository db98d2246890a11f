// Exact block-sparse (and dense) causal attention on gfx950 bf16 MFMA.
//
// Computes A(Q,K,V,S) = Softmax(QK^T/sqrt(d) + M_S) V of the digest page
// "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
// Structural-Mass-Motivated Routing" (prerequisite section on prefill and
// sparse attention; method-steps step 4), with M_S given as a block CSR, and
// the dense causal result the digest's FlashAttention baseline computes.
//
// Work item = one (head, 128-row query block).  Key blocks are walked in
// 64-key stages, double-buffered in LDS and filled by direct global->LDS loads
// (no register staging): the K stage row-major, the V stage from a V^T copy
// made once per call (keys contiguous per head-dim row), both with an XOR
// swizzle of the 16-byte chunks so that every operand read is bank-conflict
// free.  S^T = K Q^T and O^T += V^T P^T run on 32x32x16 bf16 MFMA; the online
// softmax stays in fp32 registers (each lane owns one query column), with the
// 1/sqrt(d)*log2(e) scale folded into one FMA feeding exp2 and the output
// rescaled only in stages where some row maximum outgrows its reference by
// more than 2^8.  Items come from
// per-XCD work queues (see Queue).
//
// Two kernels share this frame.  d = 128 (attn_q64_kernel): two waves per
// workgroup, 64 query rows per wave, one wave per SIMD, so that each operand
// read from LDS feeds two MFMAs.  d = 64 (attn_kernel): four waves of 32 rows,
// two workgroups per CU, so that one wave's softmax runs under another wave's
// MFMAs.
#include <math.h>

#include <type_traits>

#include "crisp_device.hpp"
#include "crisp_internal.h"

namespace crisp {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int NXCD = 8;                  // accelerator complex dies of an MI355X
constexpr int KS = 64;                   // keys per pipeline stage
constexpr int WG_PER_CU = 2;
// A row's reference maximum m is raised (and its output rescaled) only when a
// stage's maximum exceeds it by more than 2^8, so weights 2^(s c2 - m) stay
// <= 256.  The result is the same softmax: the row sum is taken over the same
// bf16-rounded weights the PV product uses, so the choice of m cancels.
constexpr float RESCALE_LOG2 = 8.f;
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

// One direct global->LDS load of 16 bytes per lane: lane i loads 16 bytes at
// gbase + voff_i into LDS bytes [lds_base + IMM + 16 i, ...).  Issued as asm so
// that the compiler does not treat the other LDS buffers as aliased and wait
// for these loads before every LDS read; the kernel waits for them itself
// (vm_wait) before the barrier that publishes a stage.
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
// work inside an XCD balances whatever the heads' routes and row lengths; a
// workgroup whose queue is dry then takes items from the next queues in turn
// (x+1, x+2, ... mod 8) until all eight are dry.  Queue 0 holds the longest
// chunk of every round, so without this the other XCDs would idle at the end
// of the launch while it drains (on a dense causal map queue 0 holds 11% more
// tiles than the mean queue at N_b = 1024 and 5.5% more at N_b = 4096).
struct Queue {
  int nb, qc;              // query blocks per head; chunk length
  int64_t bh_total;        // batch * h_q
  int per_queue;           // items per queue
};

// Chunk length: N_b / 32 query blocks, at most 32 up to N_b = 1024 and at most
// 64 above (measured on the 32k, 128k, 256k and 512k layers with the queues
// drained across XCDs: 1-1.4% faster than 16 / 32, and within 0.3% of N_b / 32
// uncapped and of N_b / 16; a length that does not split an XCD's 64
// workgroups evenly over heads, such as 24, was slower at 128k, 256k and 512k).
inline int queue_chunk(int nb) {
  const int cap = nb <= 1024 ? 32 : 64;
  const int qc = nb / 32;
  return qc < 1 ? 1 : (qc > cap ? cap : qc);
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

// sched_group_barrier instruction classes
constexpr int SG_VALU = 0x2, SG_MFMA = 0x8, SG_DSR = 0x100;
constexpr int LDS_AHEAD = 6;             // operand reads kept in flight ahead of the MFMAs

// Phase 1 of a stage: the next stage's scores S_n = K_n Q^T (when HAS_NEXT)
// with the softmax weights of the current stage's scores s_c interleaved
// between the MFMAs (two, or four for d = 64, weights per MFMA).  Weights
// p = 2^(s c2 - m) are rounded to bf16 pairs for the PV product, and the row
// sum l accumulates those rounded pairs.
template <int D, bool HAS_NEXT>
__device__ __forceinline__ void qk_softmax(const char* kbase, const uint32_t (&koff)[D / 16],
                                           const bf16x8 (&qf)[D / 16], f32x16 (&sn)[2], const f32x16 (&sc)[2],
                                           float c2, float nm, bf16x8 (&pb)[4], float& l) {
  constexpr int NQK = D / 8;     // QK MFMAs per stage
  constexpr int EPM = 32 / NQK;  // weights per MFMA
  constexpr int KROW = D * 2;
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  uint32_t wv[16];
  if (HAS_NEXT) {
    sn[0] = f32x16{};
    sn[1] = f32x16{};
  }
#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    if (HAS_NEXT) {
      const int st = i >> 1, ks = i & 1;
      sn[ks] = mfma_32x32x16(as_bf16x8(ld16(kbase + koff[st] + 32 * ks * KROW)), qf[st], sn[ks]);
    }
#pragma unroll
    for (int e = 0; e < EPM; e += 2) {
      const int j = i * EPM + e, ks = j >> 4, r = j & 15;
      const float a0 = fast_exp2(fmaf(sc[ks][r], c2, nm));
      const float a1 = fast_exp2(fmaf(sc[ks][r + 1], c2, nm));
      wv[j >> 1] = pack_bf16x2(a0, a1);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv[j >> 1]), one2, l, false);
    }
  }
  if (HAS_NEXT) {
    __builtin_amdgcn_sched_group_barrier(SG_DSR, LDS_AHEAD, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VALU, 3 * EPM / 2, 0);
      if (i + LDS_AHEAD < NQK) __builtin_amdgcn_sched_group_barrier(SG_DSR, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VALU, 3 * EPM / 2, 0);
    }
  }
  // consume the weights and the row sum here (an empty asm reading them), so
  // that the compiler computes them under this phase's MFMAs instead of
  // sinking them into the PV phase
  asm volatile("" ::"v"(wv[0]), "v"(wv[1]), "v"(wv[2]), "v"(wv[3]), "v"(wv[4]), "v"(wv[5]), "v"(wv[6]), "v"(wv[7]),
               "v"(wv[8]), "v"(wv[9]), "v"(wv[10]), "v"(wv[11]), "v"(wv[12]), "v"(wv[13]), "v"(wv[14]), "v"(wv[15]),
               "v"(l));
#pragma unroll
  for (int c = 0; c < 4; ++c) pb[c] = as_bf16x8(make_uint4(wv[4 * c], wv[4 * c + 1], wv[4 * c + 2], wv[4 * c + 3]));
}

// Phase 2 of a stage: O^T += V^T P^T for the current stage, with the row
// maximum of the next stage's scores (when HAS_NEXT) interleaved; returns it
// (both lanes of a query column hold the same value).
template <int D, bool HAS_NEXT>
__device__ __forceinline__ float pv_max(const char* vbase, const uint32_t (&voff)[4], const bf16x8 (&pb)[4],
                                        f32x16 (&o)[D / 32], const f32x16 (&sn)[2]) {
  constexpr int VROW = KS * 2;
  float t = -INFINITY;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      o[ds] = mfma_32x32x16(as_bf16x8(ld16(vbase + voff[cc] + 32 * ds * VROW)), pb[cc], o[ds]);
  if (HAS_NEXT) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) t = fmaxf(t, sn[ks][r]);
    t = fmaxf(t, xor_shfl(t, 32));
  }
  __builtin_amdgcn_sched_group_barrier(SG_DSR, LDS_AHEAD, 0);
#pragma unroll
  for (int i = 0; i < 4 * (D / 32); ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    if (HAS_NEXT) __builtin_amdgcn_sched_group_barrier(SG_VALU, 2, 0);
    if (i + LDS_AHEAD < 4 * (D / 32)) __builtin_amdgcn_sched_group_barrier(SG_DSR, 1, 0);
  }
  return t;
}

// Causal mask of a stage of the diagonal block: keys after the lane's query go to -inf.
// The threshold passes through an empty asm so that the compiler computes the
// comparisons here instead of hoisting all of them out of the stage loop
// (which would keep 32 lane masks live in scalar registers).
__device__ __forceinline__ void mask_diag(f32x16 (&s)[2], int kloc0, int qloc, int lane) {
  int lim = qloc - kloc0 - 8 * (lane >> 5);   // key_of_reg(r, lane) - 8 (lane >> 5) > lim  <=>  key > query
  asm volatile("" : "+v"(lim));
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * ks + 16 * (r >> 3) + (r & 7) > lim) s[ks][r] = -INFINITY;
}

// Online-softmax bookkeeping for a stage whose score maximum (in score units) is t.
__device__ __forceinline__ void update_max(float t, float c2, float& m, float& corr, bool& any) {
  const float tmu = t * c2;
  const bool need = tmu > m + RESCALE_LOG2;
  any = __ballot(need) != 0;
  const float mn = need ? tmu : m;
  corr = fast_exp2(m - mn);
  m = mn;
}

template <int D, bool DENSE, bool OUT_BF16>
__global__ __launch_bounds__(NTHR, WG_PER_CU) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_cap,
    void* __restrict__ out, int n, int h_q, int group, Queue qd, int* __restrict__ counters, float c2) {
  using S = Stage<D>;
  // LDS: K stage buffers 0 and 1 (first and second half of a block), then V^T
  // stage buffers 0 and 1.  The V^T load runs one stage behind the K load, so
  // the next stage's K and the current stage's V^T are resident together.
  __shared__ __align__(16) char lds[2 * S::KBYTES + 2 * S::VBYTES];
  __shared__ int item;
  int x = (int)(blockIdx.x % NXCD);
  int dry = 0;   // queues found dry so far (x is the one being drained)
  const int w = wave_id(), lane = lane_id();
  const int hi = lane >> 5;
  const int qloc = 32 * w + (lane & 31);
  const int nb = n / BLK;
  const int h_kv = h_q / group;

  // per-lane LDS read offsets, the same for every stage
  uint32_t koff[S::NSTEP], voff[4];
  {
    const int krow = key_row_of_lane(lane & 31);   // + 32 ks
    const int kfix = (S::KCPR == 16) ? (krow & 15) : ((krow >> 1) & 7);
    const int vrow = lane & 31;                    // + 32 ds
    const int vfix = (vrow >> 1) & 7;
#pragma unroll
    for (int st = 0; st < S::NSTEP; ++st) koff[st] = krow * S::KROW + (((2 * st + hi) ^ kfix) * 16);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) voff[cc] = vrow * S::VROW + (((2 * cc + hi) ^ vfix) * 16);
  }
  const char* kbuf0 = lds;
  const char* kbuf1 = lds + S::KBYTES;
  const char* vbuf0 = lds + 2 * S::KBYTES;
  const char* vbuf1 = vbuf0 + S::VBYTES;
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
  const uint32_t lds0w = lds0 + (uint32_t)w * 1024u;   // this wave's first KiB of a buffer

  for (;;) {
    if (threadIdx.x == 0) item = atomicAdd(&counters[x], 1);
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(item);
    __syncthreads();
    if (u >= qd.per_queue) {
      if (++dry == NXCD) break;
      x = (x + 1) % NXCD;
      continue;
    }
    int qb;
    int64_t bh;
    if (!queue_item(qd, x, u, qb, bh)) continue;

    const int b = (int)(bh / h_q), h = (int)(bh % h_q), g = h / group;
    const char* kgb = reinterpret_cast<const char*>(k + ((size_t)b * h_kv + g) * n * D);
    const char* vgb = reinterpret_cast<const char*>(vt + ((size_t)b * h_kv + g) * (size_t)D * n);
    auto issue_k = [&](int kb, int hf, uint32_t lbuf) {
      const char* gb = kgb + (size_t)(kb * BLK + hf * KS) * D * 2;
      const uint32_t lb = lds0w + lbuf;
      dma16s<0>(kdma[0], gb, lb);
      dma16s<4096>(kdma[1], gb, lb);
      if constexpr (S::KLOADS > 2) {
        dma16s<8192>(kdma[2], gb, lb);
        dma16s<12288>(kdma[3], gb, lb);
      }
    };
    auto issue_v = [&](int kb, int hf, uint32_t lbuf) {
      const char* gb = vgb + (size_t)(kb * BLK + hf * KS) * 2;
      const uint32_t lb = lds0w + lbuf;
      dma16s<0>(vdma[0], gb, lb);
      dma16s<4096>(vdma[1], gb, lb);
      if constexpr (S::VLOADS > 2) {
        dma16s<8192>(vdma[2], gb, lb);
        dma16s<12288>(vdma[3], gb, lb);
      }
    };
    constexpr uint32_t LK0 = 0, LK1 = S::KBYTES, LV0 = 2 * S::KBYTES, LV1 = 2 * S::KBYTES + S::VBYTES;

    // Row entries: positions [t0, t1) of col_idx, read 64 at a time (one per
    // lane) with a ballot of the valid ones (block index in [0, qb]); invalid
    // entries are skipped.
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
    int64_t cb = -1;      // first position of the chunk held in cval
    int cval = -1;
    uint64_t cmask = 0;
    auto next_valid = [&](int64_t p) -> int64_t {
      if (DENSE) return p;
      for (;;) {
        if (p >= t1) return t1;
        if (cb < 0 || p >= cb + 64) {
          cb = p;
          cval = (p + lane < t1) ? col_idx[p + lane] : -1;
          cmask = __ballot(cval >= 0 && cval <= qb);
        }
        const uint64_t bits = cmask >> (int)(p - cb);
        if (bits) return p + __builtin_ctzll(bits);
        p = cb + 64;
      }
    };
    auto entry = [&](int64_t p) -> int {
      if (DENSE) return (int)p;
      return __builtin_amdgcn_readlane(cval, (int)(p - cb));
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
    float m = M_INIT, l = 0.f, corr = 1.f;
    bool any = false;

    int64_t pc = next_valid(t0);
    if (pc < t1) {
      int kb = entry(pc);
      int64_t pn = next_valid(pc + 1);
      int kbn = pn < t1 ? entry(pn) : -1;
      f32x16 sa[2], sb[2];
      bf16x8 pb[4];
      // prologue: the first half of the first block
      issue_k(kb, 0, LK0);
      vm_wait();
      __syncthreads();
      issue_k(kb, 1, LK1);
      issue_v(kb, 0, LV0);
      sa[0] = f32x16{};
      sa[1] = f32x16{};
#pragma unroll
      for (int st = 0; st < S::NSTEP; ++st)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          sa[ks] = mfma_32x32x16(as_bf16x8(ld16(kbuf0 + koff[st] + 32 * ks * S::KROW)), qf[st], sa[ks]);
      if (kb == qb) mask_diag(sa, 0, qloc, lane);
      {
        float t = -INFINITY;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int r = 0; r < 16; ++r) t = fmaxf(t, sa[ks][r]);
        t = fmaxf(t, xor_shfl(t, 32));
        update_max(t, c2, m, corr, any);
      }
      for (;;) {
        // step A: current = (kb, 0) in sa, next = (kb, 1) -> sb
        vm_wait();
        __syncthreads();
        if (kbn >= 0) issue_k(kbn, 0, LK0);
        issue_v(kb, 1, LV1);
        l *= corr;
        qk_softmax<D, true>(kbuf1, koff, qf, sb, sa, c2, -m, pb, l);
        if (any) {
#pragma unroll
          for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[ds][r] *= corr;
        }
        if (kb == qb) mask_diag(sb, KS, qloc, lane);
        update_max(pv_max<D, true>(vbuf0, voff, pb, o, sb), c2, m, corr, any);

        // step B: current = (kb, 1) in sb, next = (kbn, 0) -> sa
        vm_wait();
        __syncthreads();
        l *= corr;
        if (kbn >= 0) {
          issue_k(kbn, 1, LK1);
          issue_v(kbn, 0, LV0);
        }
        // one straight-line path whether or not a next block exists (the
        // scores and maximum computed from the stale buffer at a row's end are
        // not used), so that the accumulators stay in place across the loop
        qk_softmax<D, true>(kbuf0, koff, qf, sa, sb, c2, -m, pb, l);
        if (any) {
#pragma unroll
          for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[ds][r] *= corr;
        }
        if (kbn == qb) mask_diag(sa, 0, qloc, lane);
        const float tn = pv_max<D, true>(vbuf1, voff, pb, o, sa);
        if (kbn < 0) break;
        update_max(tn, c2, m, corr, any);
        kb = kbn;
        pc = pn;
        pn = next_valid(pc + 1);
        kbn = pn < t1 ? entry(pn) : -1;
      }
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

// ---------------------------------------------------------------------------
// d = 128: 64 query rows per wave (two 32-row tiles), one wave per SIMD.
//
// Every K and V^T operand read from LDS feeds the MFMAs of both tiles, which
// halves the operand reads per flop.  Register classes are fixed by hand:
// the S^T accumulators (read by the softmax) in VGPRs, the O^T accumulators
// and the Q operands (touched only by MFMAs) in AGPRs, so the MFMAs are
// issued as inline asm and the schedule is written out in regions fenced
// with sched_barrier: each region holds a slice of the softmax VALU work, at
// most one operand read, and one MFMA (two where a row-sum MFMA follows a PV
// MFMA).  The softmax of a stage is split
// between the QK phase (weight pairs [0, Q64_P1) of each tile) and the PV
// phase (the rest, done by the time the PV MFMAs need them, then the next
// stage's row maxima).  The row sums come from the matrix cores as well: after
// the PV MFMAs of a 16-key chunk, one 16x16x32 MFMA multiplies a constant 0/1
// selector with that chunk's weight operand, which adds the chunk's bf16
// weights of each query row into a 4-register accumulator (VGPRs) in that
// row's lanes.
//
// The compiler does not see the MFMAs inside the asm, so the wait states the
// hardware needs around them are kept by construction: a weight pair is
// written at least two regions before the PV MFMA that reads it (VALU write
// -> MFMA read needs 2), the scores and row sums are read or rescaled by VALU
// code only in later regions or after an explicit s_nop (MFMA write -> VALU
// read needs 12), and the output rescale ends with an s_nop (AGPR write ->
// MFMA read needs 2).  tests/test_isa_hazards.py checks the compiled kernel.
// ---------------------------------------------------------------------------
constexpr int Q64_THR = 128;       // two waves: one 128-row query block per workgroup
constexpr int Q64_WG_PER_CU = 2;   // four waves per CU, one per SIMD
constexpr int Q64_P1 = 10;         // weight pairs per tile computed in the QK phase (of 16)
constexpr int Q64_AHEAD = 4;       // operand reads in flight ahead of the MFMAs

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 lds16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }
// s = K Q^T tile product, s in VGPRs, q in AGPRs
__device__ __forceinline__ void mfma_s0(f32x16& s, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& s, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "a"(b));
}
// o += V^T P^T tile product, o in AGPRs
__device__ __forceinline__ void mfma_o(f32x16& o, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}
// ls += SEL W: row sums of one 16-key chunk of weights (W, the B operand of the
// PV MFMAs), ls in VGPRs, the selector in AGPRs
__device__ __forceinline__ void mfma_l(f32x4& ls, const u32x4& sel, const u32x4& w) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(ls) : "a"(sel), "v"(w));
}
// 13 wait states: covers an MFMA result read by VALU code (or its accumulator
// overwritten by VALU code) right after the MFMA
__device__ __forceinline__ void mfma_drain() {
  fence();
  asm volatile("s_nop 7\n\ts_nop 4" ::: "memory");
  fence();
}

// Barriers of the stage loop.  Every direct load of a stage is 8 instructions
// per wave, and each barrier waits for a stage load that has exactly two stage
// loads (16 instructions) issued after it, so both wait for vmcnt <= 16.
__device__ __forceinline__ void bar_top() {
  asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void bar_mid() {
  asm volatile("s_waitcnt vmcnt(16)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// max over lanes l and l ^ 32
__device__ __forceinline__ float halves_max(float t) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// sum over lanes l and l ^ 32, added in the same order in both lanes
__device__ __forceinline__ float halves_sum(float t) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A row keeps the first stage's maximum as its fixed reference when its
// Cauchy-Schwarz logit bound c2 |q| max|k| (times BOUND_SLACK, which covers
// the rounding of the norms and of the fp32 dot products) lies at most
// FIXED_SPAN (log2 units) above it: weights then stay <= 2^FIXED_SPAN and a
// row sum over up to 2^20 keys far below the fp32 range.
constexpr float FIXED_SPAN = 64.f;
constexpr float BOUND_SLACK = 1.f + 1.f / 256.f;

// Softmax state of one stage for both tiles.  Weight pair p of tile t covers
// accumulator registers 2p, 2p+1 (ks = p / 8) and becomes 32-bit word p % 4 of
// the PV operand pw[t][p / 4]; its five VALU ops are numbered k = 0..4: two
// FMAs, two exp2 and the bf16 pack.
struct Q64Soft {
  float a0[2][16], a1[2][16];
  u32x4 pw[2][4];
};

constexpr int Q64_PAIR_OPS = 5;

__device__ __forceinline__ void q64_pair_op(Q64Soft& sm, const f32x16 (&sc)[2][2], int t, int p, int k, float c2,
                                            const float (&nm)[2]) {
  const int ks = p >> 3, r = (2 * p) & 15;
  switch (k) {
    case 0: sm.a0[t][p] = fmaf(sc[t][ks][r], c2, nm[t]); break;
    case 1: sm.a1[t][p] = fmaf(sc[t][ks][r + 1], c2, nm[t]); break;
    case 2: sm.a0[t][p] = fast_exp2(sm.a0[t][p]); break;
    case 3: sm.a1[t][p] = fast_exp2(sm.a1[t][p]); break;
    default: sm.pw[t][p >> 2][p & 3] = pack_bf16x2(sm.a0[t][p], sm.a1[t][p]);
  }
}
// op q of the pair program over NP pairs from p0 of both tiles (pair-major, tiles
// alternating).  Each pair's pack is deferred into the next pair, between its two exp2: pair 0
// runs FMA, FMA, exp2, exp2; pair pp >= 1 runs FMA, FMA, exp2, pack of pair pp - 1, exp2; the
// last op packs pair NP - 1.  A pack issued right behind the exp2 it reads stalls the wave
// (and the next MFMA) on the transcendental's latency, and this order also spreads the exp2s
// evenly over the regions (about 16 VALU cycles per region, what one MFMA leaves free).
template <int NP>
__device__ __forceinline__ void q64_pair_prog(Q64Soft& sm, const f32x16 (&sc)[2][2], int p0, int q, float c2,
                                              const float (&nm)[2]) {
  int pp, k;
  if (q < 4) {
    pp = 0;
    k = q;
  } else if (q == Q64_PAIR_OPS * NP - 1) {
    pp = NP - 1;
    k = 4;
  } else {
    const int r = q - 4, slot = r % Q64_PAIR_OPS;
    pp = 1 + r / Q64_PAIR_OPS;
    if (slot == 3) {
      pp -= 1;
      k = 4;
    } else {
      k = slot < 3 ? slot : 3;
    }
  }
  q64_pair_op(sm, sc, pp & 1, p0 + (pp >> 1), k, c2, nm);
}

// QK phase.  Regions i = 0..31: MFMA i is S_n[t][ks] += K[ks][st] Q[t][st]^T
// with i = 2 (8 ks + st) + t; operand read r = 8 ks + st feeds MFMAs 2r, 2r+1.
// The read stream continues into the PV phase: reads 16..19 are its first V^T
// operands (the V^T stage is already resident).
template <bool HAS_NEXT, typename Mid>
__device__ __forceinline__ void q64_qk(const char* kbase, const char* vbase, const uint32_t (&koff)[8],
                                       const uint32_t (&voff)[4], const u32x4 (&qf)[2][8], f32x16 (&sn)[2][2],
                                       const f32x16 (&sc)[2][2], float c2, const float (&nm)[2], Q64Soft& sm,
                                       u32x4 (&op)[Q64_AHEAD + 1], Mid&& mid) {
  constexpr int KROW = 256, VROW = KS * 2;
  constexpr int NOPS = Q64_P1 * 2 * Q64_PAIR_OPS;
  auto read = [&](int r) -> u32x4 {
    if (r < 16) return lds16(kbase + koff[r & 7] + 32 * (r >> 3) * KROW);
    const int v = r - 16;
    return lds16(vbase + voff[v >> 2] + 32 * (v & 3) * VROW);
  };
#pragma unroll
  for (int r = 0; r < Q64_AHEAD; ++r) op[r % (Q64_AHEAD + 1)] = read(r);
  fence();
#pragma unroll
  for (int i = 0; i < 32; ++i) {
#pragma unroll
    for (int q = (i * NOPS) / 32; q < ((i + 1) * NOPS) / 32; ++q) q64_pair_prog<Q64_P1 * 2>(sm, sc, 0, q, c2, nm);
    const int r = i >> 1;
    // the stage's K reads are all issued; the mid-step barrier comes before the first V^T read
    if (i == 2 * (16 - Q64_AHEAD)) mid();
    if (!(i & 1)) op[(r + Q64_AHEAD) % (Q64_AHEAD + 1)] = read(r + Q64_AHEAD);
    if (HAS_NEXT) {
      const int t = i & 1, ks = r >> 3, st = r & 7;
      if (st == 0) mfma_s0(sn[t][ks], op[r % (Q64_AHEAD + 1)], qf[t][st]);
      else mfma_s(sn[t][ks], op[r % (Q64_AHEAD + 1)], qf[t][st]);
    }
    fence();
  }
  // keep the weights computed here in this phase
#pragma unroll
  for (int t = 0; t < 2; ++t)
    asm volatile("" ::"v"(sm.pw[t][0]), "v"(sm.pw[t][1]), "v"(sm.pw[t][2][0]), "v"(sm.pw[t][2][1]));
}

// PV phase.  Regions i = 0..31: MFMA i is O[t][ds] += V^T[cc][ds] P[t][cc]
// with i = 2 (4 cc + ds) + t; V^T read r = 4 cc + ds (stream index 16 + r).
// Regions 8 cc + 6 + t, after the last PV MFMA that reads P[t][cc], also add
// that chunk's weights into the row sums ls[t].  Pair ops [Q64_P1, 16) run in
// regions 0..21 (the last weight is written two regions before the first
// cc = 3 MFMA), the row maxima of S_n in 22..31.
template <bool HAS_NEXT, bool TRACK_MAX = true>
__device__ __forceinline__ void q64_pv(const char* vbase, const uint32_t (&voff)[4], f32x16 (&o)[2][4],
                                       f32x4 (&ls)[2], const u32x4& sel, const f32x16 (&sc)[2][2], float c2,
                                       const float (&nm)[2], Q64Soft& sm, const f32x16 (&sn)[2][2],
                                       float (&tmax)[2], u32x4 (&op)[Q64_AHEAD + 1]) {
  constexpr int VROW = KS * 2;
  constexpr int NOPS = (16 - Q64_P1) * 2 * Q64_PAIR_OPS;
  constexpr int NMAX = 2 * 17;
  float xm[2] = {-INFINITY, -INFINITY};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if (i < 22) {
#pragma unroll
      for (int q = (i * NOPS) / 22; q < ((i + 1) * NOPS) / 22; ++q)
        q64_pair_prog<(16 - Q64_P1) * 2>(sm, sc, Q64_P1, q, c2, nm);
    } else if (HAS_NEXT && TRACK_MAX) {
      const int j = i - 22;
#pragma unroll
      for (int q = (j * NMAX) / 10; q < ((j + 1) * NMAX) / 10; ++q) {
        const int t = q / 17, mq = q % 17;
        if (mq < 16) {
          const int ks = mq >> 3, r = (2 * mq) & 15;
          xm[t] = fmaxf(fmaxf(xm[t], sn[t][ks][r]), sn[t][ks][r + 1]);
        } else {
          tmax[t] = halves_max(xm[t]);
        }
      }
    }
    const int r = i >> 1;
    if (!(i & 1) && r + Q64_AHEAD < 16) {
      const int v = r + Q64_AHEAD;
      op[(16 + v) % (Q64_AHEAD + 1)] = lds16(vbase + voff[v >> 2] + 32 * (v & 3) * VROW);
    }
    const int t = i & 1, cc = r >> 2, ds = r & 3;
    mfma_o(o[t][ds], op[(16 + r) % (Q64_AHEAD + 1)], sm.pw[t][cc]);
    if (ds == 3) mfma_l(ls[t], sel, sm.pw[t][cc]);
    fence();
  }
}

__device__ __forceinline__ void q64_update(const float (&tmax)[2], float c2, float (&m)[2], float (&corr)[2],
                                           bool (&any)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float tmu = tmax[t] * c2;
    const bool need = tmu > m[t] + RESCALE_LOG2;
    any[t] = __ballot(need) != 0;
    const float mn = need ? tmu : m[t];
    corr[t] = fast_exp2(m[t] - mn);
    m[t] = mn;
  }
}

// O *= corr and ls *= corr for the tiles whose reference maximum was raised.
// O is scaled in asm (AGPR read, multiply, AGPR write per register) so that no
// compiler-generated code touches the AGPR accumulators inside the stage loop;
// the trailing s_nop covers the AGPR write -> MFMA accumulator read of the
// next PV MFMA.  The row sums are VGPRs, scaled by plain multiplies (their next
// MFMA is regions away).
template <typename V, int N>
__device__ __forceinline__ void agpr_scale(V& o, float c) {
#pragma unroll
  for (int r = 0; r < N; ++r) {
    float e = o[r], tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(e), "=&v"(tmp)
                 : "v"(c));
    o[r] = e;
  }
}
__device__ __forceinline__ void q64_rescale(f32x16 (&o)[2][4], f32x4 (&ls)[2], const float (&corr)[2],
                                            const bool (&any)[2]) {
  fence();
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (any[t]) {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) agpr_scale<f32x16, 16>(o[t][ds], corr[t]);
      ls[t] *= corr[t];
      asm volatile("s_nop 2" ::: "memory");
      fence();
    }
}

// Row maxima (score units) of a stage's scores, both lanes of a query column.
__device__ __forceinline__ void q64_rowmax(const f32x16 (&s)[2][2], float (&tm)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float xm = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; r += 2) xm = fmaxf(fmaxf(xm, s[t][ks][r]), s[t][ks][r + 1]);
    tm[t] = halves_max(xm);
  }
}

__device__ __forceinline__ void q64_mask(f32x16 (&s)[2][2], int kloc0, int qloc0, int lane) {
  mfma_drain();
  mask_diag(s[0], kloc0, qloc0, lane);
  mask_diag(s[1], kloc0, qloc0 + 32, lane);
  fence();
}

template <bool DENSE, bool OUT_BF16>
__global__ __launch_bounds__(Q64_THR) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_q64_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_cap,
    void* __restrict__ out, int n, int h_q, int group, Queue qd, int* __restrict__ counters,
    const float* __restrict__ kn2max, float c2) {
  constexpr int D = 128;
  using S = Stage<D>;
  // LDS: K stage buffers 0 and 1, then V^T stage buffers 0 and 1 (as in attn_kernel)
  __shared__ __align__(16) char lds[2 * S::KBYTES + 2 * S::VBYTES];
  __shared__ int item;
  int x = (int)(blockIdx.x % NXCD);
  int dry = 0;   // queues found dry so far (x is the one being drained)
  const int w = wave_id(), lane = lane_id();
  const int hi = lane >> 5;
  const int nb = n / BLK;
  const int h_kv = h_q / group;

  uint32_t koff[S::NSTEP], voff[4];
  {
    const int krow = key_row_of_lane(lane & 31);
    const int kfix = krow & 15;
    const int vrow = lane & 31;
    const int vfix = (vrow >> 1) & 7;
#pragma unroll
    for (int st = 0; st < S::NSTEP; ++st) koff[st] = krow * S::KROW + (((2 * st + hi) ^ kfix) * 16);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) voff[cc] = vrow * S::VROW + (((2 * cc + hi) ^ vfix) * 16);
  }
  const char* kbuf0 = lds;
  const char* kbuf1 = lds + S::KBYTES;
  const char* vbuf0 = lds + 2 * S::KBYTES;
  const char* vbuf1 = vbuf0 + S::VBYTES;
  // Direct loads: load i (0..7) of wave w fills LDS chunks (2i + w)*64 + lane of
  // a stage buffer.  K: row 8i + 4w + lane/16, whose swizzle alternates with
  // the parity of i.  V^T: row 16i + 8w + lane/8, one swizzle for all i.  The
  // eight per-lane byte offsets of each are kept in registers, so that all
  // loads of a stage share one scalar base address.
  uint32_t kd[8], vd[8];
  {
    const int pc = lane & 15;
    const int r0 = 4 * w + (lane >> 4), r1 = r0 + 8;
    const uint32_t kd0 = (uint32_t)(r0 * D + (pc ^ (r0 & 15)) * 8) * 2u;
    const uint32_t kd1 = (uint32_t)(r1 * D + (pc ^ (r1 & 15)) * 8) * 2u;
    const int vr0 = 8 * w + (lane >> 3);
    const uint32_t vd0 = (uint32_t)(vr0 * n + ((lane & 7) ^ ((vr0 >> 1) & 7)) * 8) * 2u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kd[i] = ((i & 1) ? kd1 : kd0) + (uint32_t)(i >> 1) * 4096u;
      vd[i] = vd0 + (uint32_t)i * 16u * (uint32_t)n * 2u;   // 16 V^T rows per load
    }
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)(char*)lds);
  const uint32_t lds0w = lds0 + (uint32_t)w * 1024u;
  // Row-sum selector, the A operand of mfma_l: 1.0 in every bf16 of lane l when
  // bit 4 of l equals bit 2 of l, else 0 (A row l % 16, weight lane group l / 16).
  // Made opaque once here, so that it stays in AGPRs instead of being rebuilt
  // before each use.
  const uint32_t sel_on = ((lane >> 4) & 1) == ((lane >> 2) & 1) ? 0x3F803F80u : 0u;
  u32x4 sel = {sel_on, sel_on, sel_on, sel_on};
  asm volatile("" : "+a"(sel));

  for (;;) {
    if (threadIdx.x == 0) item = atomicAdd(&counters[x], 1);
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(item);
    __syncthreads();
    if (u >= qd.per_queue) {
      if (++dry == NXCD) break;
      x = (x + 1) % NXCD;
      continue;
    }
    int qb;
    int64_t bh;
    if (!queue_item(qd, x, u, qb, bh)) continue;

    const int b = (int)(bh / h_q), h = (int)(bh % h_q), g = h / group;
    const char* kgb = reinterpret_cast<const char*>(k + ((size_t)b * h_kv + g) * n * D);
    const char* vgb = reinterpret_cast<const char*>(vt + ((size_t)b * h_kv + g) * (size_t)D * n);
    auto issue_k = [&](int kb, int hf, uint32_t lbuf) {
      const char* gb = kgb + (size_t)(kb * BLK + hf * KS) * D * 2;
      const uint32_t lb = lds0w + lbuf;
      dma16s<0>(kd[0], gb, lb);
      dma16s<2048>(kd[1], gb, lb);
      dma16s<4096>(kd[2], gb, lb);
      dma16s<6144>(kd[3], gb, lb);
      dma16s<8192>(kd[4], gb, lb);
      dma16s<10240>(kd[5], gb, lb);
      dma16s<12288>(kd[6], gb, lb);
      dma16s<14336>(kd[7], gb, lb);
    };
    auto issue_v = [&](int kb, int hf, uint32_t lbuf) {
      const char* gb = vgb + (size_t)(kb * BLK + hf * KS) * 2;
      const uint32_t lb = lds0w + lbuf;
      dma16s<0>(vd[0], gb, lb);
      dma16s<2048>(vd[1], gb, lb);
      dma16s<4096>(vd[2], gb, lb);
      dma16s<6144>(vd[3], gb, lb);
      dma16s<8192>(vd[4], gb, lb);
      dma16s<10240>(vd[5], gb, lb);
      dma16s<12288>(vd[6], gb, lb);
      dma16s<14336>(vd[7], gb, lb);
    };
    constexpr uint32_t LK0 = 0, LK1 = S::KBYTES, LV0 = 2 * S::KBYTES, LV1 = 2 * S::KBYTES + S::VBYTES;

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
    int64_t cb = -1;
    int cval = -1;
    uint64_t cmask = 0;
    auto next_valid = [&](int64_t p) -> int64_t {
      if (DENSE) return p;
      for (;;) {
        if (p >= t1) return t1;
        if (cb < 0 || p >= cb + 64) {
          cb = p;
          cval = (p + lane < t1) ? col_idx[p + lane] : -1;
          cmask = __ballot(cval >= 0 && cval <= qb);
        }
        const uint64_t bits = cmask >> (int)(p - cb);
        if (bits) return p + __builtin_ctzll(bits);
        p = cb + 64;
      }
    };
    auto entry = [&](int64_t p) -> int {
      if (DENSE) return (int)p;
      return __builtin_amdgcn_readlane(cval, (int)(p - cb));
    };

    const int qloc0 = 64 * w + (lane & 31);   // query row (in the block) of tile 0; tile 1 is 32 further
    u32x4 qf[2][S::NSTEP];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* qp = q + ((size_t)bh * n + (size_t)qb * BLK + qloc0 + 32 * t) * D + 8 * hi;
#pragma unroll
      for (int s = 0; s < S::NSTEP; ++s) qf[t][s] = *reinterpret_cast<const u32x4*>(qp + 16 * s);
    }
    // Squared norm of each of the wave's query rows (both lanes of a row hold
    // it), from a second read of the rows through an address the compiler
    // cannot match with qf's: read from qf, the operands would stay in VGPRs
    // and move to their AGPRs right before the first MFMAs, one instruction
    // short of the wait the hardware needs there.
    float qn2[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* qp = q + ((size_t)bh * n + (size_t)qb * BLK + qloc0 + 32 * t) * D + 8 * hi;
      asm volatile("" : "+v"(qp));
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < S::NSTEP; ++s) {
        const u32x4 x4 = *reinterpret_cast<const u32x4*>(qp + 16 * s);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 x = __builtin_bit_cast(bf16x2, x4[e]);
          acc = __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
        }
      }
      qn2[t] = halves_sum(acc);
    }
    f32x16 o[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t][i] = f32x16{};
    // Row sums: 16x16x32 accumulators whose lane l holds row l % 32 of its tile
    // (the selector row of lane l is m = l % 16; it takes the weight operand's
    // lane group g when g % 2 == (m / 4) % 2, i.e. the group holding the rows of
    // the same parity half as the output rows m of lane group l / 16).
    f32x4 ls[2] = {f32x4{}, f32x4{}};
    float m[2] = {M_INIT, M_INIT}, corr[2] = {1.f, 1.f};
    bool any[2] = {false, false};

    int64_t pc = next_valid(t0);
    if (pc < t1) {
      // Stage s = (block, half).  K(s) lives in K buffer s % 2, V^T(s) in V buffer s % 2.
      // Step s: QK of stage s+1 (phase 1), PV of stage s (phase 2).  Loads: V^T(s+1)
      // after the step's top barrier, K(s+3) after its mid barrier (once every wave
      // has read K(s+1)), so each load has a step and a half to land.  Loads past the
      // row's end are dummies (the current block), which keeps the wait counts exact.
      int kb = entry(pc);
      int64_t pn = next_valid(pc + 1);
      int kbn = pn < t1 ? entry(pn) : -1;
      int64_t pnn = kbn >= 0 ? next_valid(pn + 1) : t1;
      int kbnn = pnn < t1 ? entry(pnn) : -1;
      f32x16 sa[2][2], sb[2][2];
      Q64Soft sm;
      u32x4 op[Q64_AHEAD + 1];
      float tm[2];
      issue_k(kb, 0, LK0);
      issue_k(kb, 1, LK1);
      issue_v(kb, 0, LV0);
      bar_top();   // K(kb, 0) landed for every wave
      fence();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const u32x4 kop = lds16(kbuf0 + koff[r & 7] + 32 * (r >> 3) * S::KROW);
        if ((r & 7) == 0) {
          mfma_s0(sa[0][r >> 3], kop, qf[0][r & 7]);
          mfma_s0(sa[1][r >> 3], kop, qf[1][r & 7]);
        } else {
          mfma_s(sa[0][r >> 3], kop, qf[0][r & 7]);
          mfma_s(sa[1][r >> 3], kop, qf[1][r & 7]);
        }
      }
      fence();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // every wave has read K(kb, 0)
      issue_k(kbn >= 0 ? kbn : kb, 0, LK0);
      mfma_drain();
      if (kb == qb) {
        mask_diag(sa[0], 0, qloc0, lane);
        mask_diag(sa[1], 0, qloc0 + 32, lane);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float xm = -INFINITY;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int r = 0; r < 16; ++r) xm = fmaxf(xm, sa[t][ks][r]);
        tm[t] = halves_max(xm);
      }
      q64_update(tm, c2, m, corr, any);
      // Fixed reference maximum.  When every logit of the wave's rows is provably
      // at most FIXED_SPAN above the first stage's maximum m (Cauchy-Schwarz:
      // s <= |q| max|k|), m stays for the whole row: no stage needs its maximum,
      // a rescale test or a rescale, and the weights stay below 2^FIXED_SPAN.
      // Otherwise (a loose bound) the wave tracks its rows' maxima stage by stage
      // in a block after each step's PV phase.  Both cases run the same loop (a
      // second copy of it makes the register allocator spill).
      bool track;
      {
        const float kn2 = kn2max[(size_t)b * h_kv + g];
        bool loose = false;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float bound = c2 * __builtin_sqrtf(qn2[t] * kn2) * BOUND_SLACK;
          loose |= !(bound - m[t] <= FIXED_SPAN);
        }
        track = __ballot(loose) != 0;
        if (!track) any[0] = any[1] = false;
      }
      for (;;) {
        // step A: current = (kb, 0) in sa, next = (kb, 1) -> sb
        bar_top();                      // K(kb, 1) landed
        issue_v(kb, 1, LV1);
        {
          const float nm[2] = {-m[0], -m[1]};
          q64_qk<true>(kbuf1, vbuf0, koff, voff, qf, sb, sa, c2, nm, sm, op, [&]() {
            bar_mid();                  // V(kb, 0) landed; every wave has read K(kb, 1)
            issue_k(kbn >= 0 ? kbn : kb, 1, LK1);
          });
          q64_rescale(o, ls, corr, any);
          if (kb == qb) q64_mask(sb, KS, qloc0, lane);
          q64_pv<true, false>(vbuf0, voff, o, ls, sel, sa, c2, nm, sm, sb, tm, op);
        }
        if (track) {
          q64_rowmax(sb, tm);
          q64_update(tm, c2, m, corr, any);
        }

        // step B: current = (kb, 1) in sb, next = (kbn, 0) -> sa
        bar_top();                      // K(kbn, 0) landed
        issue_v(kbn >= 0 ? kbn : kb, 0, LV0);
        {
          const float nm[2] = {-m[0], -m[1]};
          q64_qk<true>(kbuf0, vbuf1, koff, voff, qf, sa, sb, c2, nm, sm, op, [&]() {
            bar_mid();                  // V(kb, 1) landed; every wave has read K(kbn, 0)
            issue_k(kbnn >= 0 ? kbnn : kb, 0, LK0);
          });
          q64_rescale(o, ls, corr, any);
          if (kbn == qb) q64_mask(sa, 0, qloc0, lane);
          q64_pv<true, false>(vbuf1, voff, o, ls, sel, sb, c2, nm, sm, sa, tm, op);
        }
        if (kbn < 0) break;
        if (track) {
          q64_rowmax(sa, tm);
          q64_update(tm, c2, m, corr, any);
        }
        kb = kbn;
        pn = pnn;
        kbn = kbnn;
        pnn = kbn >= 0 ? next_valid(pn + 1) : t1;
        kbnn = pnn < t1 ? entry(pnn) : -1;
      }
      mfma_drain();
    }

#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float lt = ls[t][0];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const size_t orow = (size_t)bh * n + (size_t)qb * BLK + qloc0 + 32 * t;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int d = 32 * ds + 8 * grp + 4 * hi;
          const float a0 = o[t][ds][4 * grp] * inv, a1 = o[t][ds][4 * grp + 1] * inv;
          const float a2 = o[t][ds][4 * grp + 2] * inv, a3 = o[t][ds][4 * grp + 3] * inv;
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
}

// V [bg][n][D] -> V^T [bg][D][n], 64-key tiles through LDS; also the largest
// squared norm of the tile's 64 keys, to kn2part[bg][tile].
template <int D>
__global__ __launch_bounds__(NTHR) void transpose_v_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt,
                                                           const uint16_t* __restrict__ k,
                                                           float* __restrict__ kn2part, int n) {
  __shared__ float wmax[NTHR / 64];
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
  // squared norms of the same 64 keys: the CPR threads of a key row are adjacent lanes
  const uint16_t* ksrc = k + ((size_t)bg * n + key0) * D;
  float best = 0.f;
  for (int c = threadIdx.x; c < KS * CPR; c += NTHR) {
    const uint4 u = ld16(ksrc + (size_t)(c / CPR) * D + (c % CPR) * 8);
    const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x2 x = __builtin_bit_cast(bf16x2, wds[j]);
      acc = __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
    }
#pragma unroll
    for (int msk = CPR / 2; msk >= 1; msk >>= 1) acc += xor_shfl(acc, msk);
    best = fmaxf(best, acc);
  }
  best = wave_max(best);
  if (lane_id() == 0) wmax[wave_id()] = best;
  __syncthreads();
  if (threadIdx.x == 0)
    kn2part[(size_t)bg * gridDim.x + blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// kn2max[bg] = the largest of the key tiles' squared norms of KV head bg.
__global__ __launch_bounds__(NTHR) void kn2_reduce_kernel(const float* __restrict__ kn2part,
                                                          float* __restrict__ kn2max, int tiles) {
  __shared__ float wmax[NTHR / 64];
  const int64_t bg = blockIdx.x;
  float best = 0.f;
  for (int i = threadIdx.x; i < tiles; i += NTHR) best = fmaxf(best, kn2part[(size_t)bg * tiles + i]);
  best = wave_max(best);
  if (lane_id() == 0) wmax[wave_id()] = best;
  __syncthreads();
  if (threadIdx.x == 0) kn2max[bg] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
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
// largest squared key norm per KV head and per 64-key tile of each KV head, each padded to 256 bytes
size_t kn2_bytes(const Dims& dm) {
  const size_t bg = (size_t)dm.batch * dm.h_kv;
  return ((bg * 4 + 255) & ~(size_t)255) + ((bg * (dm.n / KS) * 4 + 255) & ~(size_t)255);
}

template <int D, bool DENSE>
hipError_t attn_launch(const Dims& dm, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int64_t* row_ptr, const int32_t* col_idx, int64_t cap, void* out,
                       int out_bf16, void* ws, hipStream_t st) {
  int* counters = static_cast<int*>(ws);
  const size_t bg = (size_t)dm.batch * dm.h_kv;
  float* kn2f = reinterpret_cast<float*>(static_cast<char*>(ws) + COUNTER_BYTES);
  float* kn2part = reinterpret_cast<float*>(static_cast<char*>(ws) + COUNTER_BYTES + ((bg * 4 + 255) & ~(size_t)255));
  uint16_t* vt = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + COUNTER_BYTES + kn2_bytes(dm));
  const float c2 = LOG2E / sqrtf((float)D);
  const Queue qd = make_queue(dm.nb, dm.bh);
  const int64_t slots = (int64_t)(cu_count() * WG_PER_CU + NXCD - 1) / NXCD * NXCD;
  const int64_t items = qd.per_queue * NXCD;
  const unsigned grid = (unsigned)(items < slots ? items : slots);
  zero_counters_kernel<<<1, 64, 0, st>>>(counters);
  transpose_v_kernel<D><<<dim3(dm.n / KS, (unsigned)bg), NTHR, 0, st>>>(v, vt, k, kn2part, dm.n);
  kn2_reduce_kernel<<<(unsigned)bg, NTHR, 0, st>>>(kn2part, kn2f, dm.n / KS);
  if constexpr (D == 128) {
    const int64_t slots64 = (int64_t)(cu_count() * Q64_WG_PER_CU + NXCD - 1) / NXCD * NXCD;
    const unsigned grid64 = (unsigned)(items < slots64 ? items : slots64);
    if (out_bf16)
      attn_q64_kernel<DENSE, true><<<grid64, Q64_THR, 0, st>>>(q, k, vt, row_ptr, col_idx, cap, out, dm.n, dm.h_q,
                                                               dm.group, qd, counters, kn2f, c2);
    else
      attn_q64_kernel<DENSE, false><<<grid64, Q64_THR, 0, st>>>(q, k, vt, row_ptr, col_idx, cap, out, dm.n, dm.h_q,
                                                                dm.group, qd, counters, kn2f, c2);
  } else {
    if (out_bf16)
      attn_kernel<D, DENSE, true><<<grid, NTHR, 0, st>>>(q, k, vt, row_ptr, col_idx, cap, out, dm.n, dm.h_q,
                                                         dm.group, qd, counters, c2);
    else
      attn_kernel<D, DENSE, false><<<grid, NTHR, 0, st>>>(q, k, vt, row_ptr, col_idx, cap, out, dm.n, dm.h_q,
                                                          dm.group, qd, counters, c2);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_ws_bytes(const Dims& dm) { return COUNTER_BYTES + kn2_bytes(dm) + vt_bytes(dm); }

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
