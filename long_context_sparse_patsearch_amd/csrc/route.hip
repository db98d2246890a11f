// PatSearch on gfx950: proxy softmax of the last 128 queries against all keys,
// reduced on the fly to vertical / slash block scores and the structural mass.
//
// Method: digest page "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
// Structural-Mass-Motivated Routing", core-method section and Algorithm 2
// caption (proxy A_hat, C_struct over the first and last 128 keys, VS iff
// C_struct >= tau), and method-steps step 2 / Algorithm 3 caption (column and
// diagonal means of A_hat, block-pooled).
//
// A_hat (b x n per head) is never stored.  One pass over K computes every
// 128x128 proxy tile once (up to four query heads of a KV group per workgroup,
// so each K tile is read once for all of them) and keeps, per proxy row and
// tile, the tile's maximum logit and the sums of the row's exponentials over
// the tile's lower triangle with diagonal (in-tile key jj <= row i) and over
// its strict upper triangle, plus per row and chunk of tiles the chunk's
// maximum and normaliser.  A combine step merges the chunks into each row's
// softmax statistics in a fixed order, and a reduction then normalises the
// tile sums and adds them over the rows into L and U per key block.  Because b
// equals the block size, an entry of key block kb lies on a diagonal
// t = j + b-1-i in slash block kb when jj <= i and kb+1 otherwise, so
// p_vert[kb] = (L_kb + U_kb)/b and p_slash[kb] = (L_kb + U_{kb-1})/b.  Every
// reduction has a fixed order.
#include <math.h>

#include <mutex>

#include "../../include/crisp.h"
#include "crisp_internal.h"
#include "tile_core.hpp"

namespace crisp {

// Device scratch of crisp_route_noalloc, for callers that cannot allocate: the
// proxy passes' partial (max, sum) per chunk, the combined row statistics and
// the L/U tile sums live here instead of in a caller's workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  Every kernel of
// the routing pass writes all of the scratch it later reads, so nothing needs
// clearing between calls; calls that overlap on one GPU race on it.
static __device__ __align__(256) unsigned char scratch[CRISP_ROUTE_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

// Device address of this GPU's scratch (the current device's), looked up once
// per device: in host code the array's name is only a stand-in for the symbol.
hipError_t route_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

constexpr float LOG2E = 1.4426950408889634f;

// The proxy pass over a chunk of key tiles, for HPW query heads of one KV
// group at once: the workgroup is HPW slots of two waves, slot s holding the
// 128 proxy rows of query head split*HPW + s of the group (wave w of a slot:
// rows 64w..64w+63, as two 32-row MFMA tiles that share every K operand read
// from LDS), so each K tile staged in LDS serves every head of the slot set and
// K is read once per HPW heads.  Tiles are staged through registers two tiles
// ahead into two LDS buffers (one barrier per tile).  Slots past the group's
// last head only help stage the tiles.  The exponentials bound the kernel: per
// entry it spends one maximum (half of a max3), one fused scale-and-shift, one
// exp2 and one add, and only the diagonal 32x32 sub-tile of each row tile
// splits its entries between the lower and upper sums.
//
// Per proxy row i and key tile kb it writes the tile's maximum logit m (log2
// units) and the sums of 2^(logit - m) over the tile's lower triangle with
// diagonal (in-tile key jj <= i) and over its strict upper triangle, to
// tilep[bh][kb][3][128]; per row and chunk, the chunk's maximum and normaliser
// to part[bh][chunk][row].  One pass over K thus holds everything the block
// scores need once the rows' softmax statistics are known.
template <int D, int HPW>
__global__ __launch_bounds__(128 * HPW) void proxy_tile_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, float* __restrict__ part,
    float* __restrict__ tilep, int n, int h_q, int group, int chunk_tiles, int nchunks, float c2) {
  constexpr int NT = 128 * HPW;
  constexpr int CPR = Tile<D>::CPR;
  constexpr int KCH = BLK * CPR / NT;   // 16-byte K loads per thread per tile
  static_assert(KCH >= 1 && BLK * CPR % NT == 0, "tile staging");
  __shared__ __align__(16) uint16_t klds[2][Tile<D>::KLDS];
  const int chunk = blockIdx.x;
  const int bg = blockIdx.y;             // batch * h_kv + KV head
  const int h_kv = h_q / group;
  const int b = bg / h_kv, g = bg % h_kv;
  const int w = wave_id(), lane = lane_id();
  const int slot = w >> 1, wh = w & 1;   // two waves per head, 64 proxy rows each (two 32-row tiles)
  const int hg = blockIdx.z * HPW + slot;
  const bool active = hg < group;
  const int64_t bh = (int64_t)b * h_q + (int64_t)g * group + (active ? hg : 0);
  const int nb = n / BLK, qb = nb - 1;
  const int qloc0 = 64 * wh + (lane & 31);   // tile t: row qloc0 + 32 t
  const uint16_t* kg = k + (size_t)bg * n * D;

  bf16x8 qf[2][Tile<D>::NSTEP];
  if (active) {
    load_q_operands<D>(q + ((size_t)bh * n + (size_t)qb * BLK + 64 * wh) * D, qf[0]);
    load_q_operands<D>(q + ((size_t)bh * n + (size_t)qb * BLK + 64 * wh + 32) * D, qf[1]);
  }
  float mc[2] = {-INFINITY, -INFINITY}, lc[2] = {0.f, 0.f};

  auto load = [&](int kb, uint4 (&r)[KCH]) {
    const uint16_t* t = kg + (size_t)kb * BLK * D;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = i * NT + threadIdx.x;
      r[i] = ld16(t + (size_t)(c / CPR) * D + (c % CPR) * 8);
    }
  };
  auto store = [&](uint16_t* lds, const uint4 (&r)[KCH]) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = i * NT + threadIdx.x;
      st16(lds + (c / CPR) * Tile<D>::KSTR + (c % CPR) * 8, r[i]);
    }
  };
  // Within a 32-row tile t the rows are 32*mixblk .. 32*mixblk+31 of the proxy block, so
  // 32-key sub-tile blk lies wholly in the lower triangle (blk < mixblk), wholly in the
  // upper one (blk > mixblk) or on the diagonal (blk == mixblk): only that sub-tile needs
  // the per-entry split.
  auto compute = [&](int kb, const uint16_t* lds) {
    const uint16_t* base = lds + key_row_of_lane(lane & 31) * Tile<D>::KSTR + 8 * (lane >> 5);
    const bool diag = (kb == qb);
    float hm[2][2], hlo[2][2], hup[2][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {   // keys 64 hf .. 64 hf + 63, relative to their own maximum
      f32x16 s[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint16_t* pp = base + 32 * (2 * hf + kk) * Tile<D>::KSTR;
#pragma unroll
        for (int st = 0; st < Tile<D>::NSTEP; ++st) {
          const bf16x8 a = as_bf16x8(ld16(pp + 16 * st));   // one K read feeds both tiles
          s[0][kk] = mfma_32x32x16(a, qf[0][st], s[0][kk]);
          s[1][kk] = mfma_32x32x16(a, qf[1][st], s[1][kk]);
        }
      }
      if (diag) {   // the proxy block's own tile: keys after the row are outside the causal mask
        asm volatile("" ::: "memory");   // keep the branch: masking every tile would cost a select per entry
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * (2 * hf + kk) + key_of_reg(r, lane) > qloc0 + 32 * t) s[t][kk][r] = -INFINITY;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int mixblk = 2 * wh + t;
        float smax = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r) smax = fmaxf(smax, s[t][kk][r]);
        smax = fmaxf(smax, xor_shfl(smax, 32));
        const float tmax = smax * c2;   // c2 > 0: the maximum of the scaled logits
        // a half the causal mask hides entirely (diagonal tile, rows < 64) sums to 0
        const float nref = tmax == -INFINITY ? 0.f : -tmax;
        float lo = 0.f, up = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int blk = 2 * hf + kk;
          float bs = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(s[t][kk][r], c2, nref));
            s[t][kk][r] = e;
            bs += e;
          }
          if (blk < mixblk) {
            lo += bs;
          } else if (blk > mixblk) {
            up += bs;
          } else {
            asm volatile("" ::: "memory");   // as above: only this sub-tile takes the per-entry split
            float dlo = 0.f, dup = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              if (key_of_reg(r, lane) <= (lane & 31)) dlo += s[t][kk][r]; else dup += s[t][kk][r];
            }
            lo += dlo;
            up += dup;
          }
        }
        hm[t][hf] = tmax;
        hlo[t][hf] = lo + xor_shfl(lo, 32);
        hup[t][hf] = up + xor_shfl(up, 32);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float mt = fmaxf(hm[t][0], hm[t][1]);   // finite: key 0 of every tile is visible to every row
      const float f0 = fast_exp2(hm[t][0] - mt), f1 = fast_exp2(hm[t][1] - mt);
      const float lo = hlo[t][0] * f0 + hlo[t][1] * f1, up = hup[t][0] * f0 + hup[t][1] * f1;
      const float mn = fmaxf(mc[t], mt);
      lc[t] = lc[t] * fast_exp2(mc[t] - mn) + (lo + up) * fast_exp2(mt - mn);
      mc[t] = mn;
      if (lane < 32) {
        float* o = tilep + ((size_t)bh * nb + kb) * 3 * BLK + qloc0 + 32 * t;
        o[0] = mt;
        o[BLK] = lo;
        o[2 * BLK] = up;
      }
    }
  };

  const int kb0 = chunk * chunk_tiles, kb1 = min(nb, kb0 + chunk_tiles);
  uint4 r0[KCH], r1[KCH];
  load(kb0, r0);
  if (kb0 + 1 < kb1) load(kb0 + 1, r1);
  for (int kb = kb0; kb < kb1; kb += 2) {
    // tile kb: registers r0, buffer 0
    store(klds[0], r0);
    __syncthreads();
    if (kb + 2 < kb1) load(kb + 2, r0);
    if (active) compute(kb, klds[0]);
    if (kb + 1 >= kb1) break;
    // tile kb + 1: registers r1, buffer 1
    store(klds[1], r1);
    __syncthreads();
    if (kb + 3 < kb1) load(kb + 3, r1);
    if (active) compute(kb + 1, klds[1]);
  }
  if (active && lane < 32) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float* o = part + (((size_t)bh * nchunks + chunk) * BLK + qloc0 + 32 * t) * 2;
      o[0] = mc[t];
      o[1] = lc[t];
    }
  }
}

// Block sums of the normalised proxy: per (head, key tile kb), over the 128
// proxy rows i, L = sum_i lo_i 2^(m_i - M_i) / L_i and U likewise from up_i,
// with (M_i, 1/L_i) the rows' combined statistics.  One wave per tile, rows i
// and i + 64 in lane i, then a fixed-order butterfly.
__global__ __launch_bounds__(NTHR) void proxy_reduce_kernel(const float* __restrict__ tilep,
                                                            const float* __restrict__ stats, float* __restrict__ lu,
                                                            int nb) {
  const int64_t bh = blockIdx.y;
  const int lane = lane_id();
  const float* st = stats + (size_t)bh * BLK * 2;
  const float M0 = st[2 * lane], iL0 = st[2 * lane + 1];
  const float M1 = st[2 * (lane + 64)], iL1 = st[2 * (lane + 64) + 1];
  for (int kb = blockIdx.x * 4 + wave_id(); kb < nb; kb += gridDim.x * 4) {
    const float* t = tilep + ((size_t)bh * nb + kb) * 3 * BLK;
    const float w0 = fast_exp2(t[lane] - M0) * iL0, w1 = fast_exp2(t[lane + 64] - M1) * iL1;
    float lo = t[BLK + lane] * w0 + t[BLK + lane + 64] * w1;
    float up = t[2 * BLK + lane] * w0 + t[2 * BLK + lane + 64] * w1;
    lo = wave_sum(lo);
    up = wave_sum(up);
    if (lane == 0) {
      lu[((size_t)bh * nb + kb) * 2] = lo;
      lu[((size_t)bh * nb + kb) * 2 + 1] = up;
    }
  }
}

// Merge the per-chunk (max, sum) of every proxy row in chunk order.
__global__ __launch_bounds__(BLK) void proxy_combine_kernel(const float* __restrict__ part,
                                                            float* __restrict__ stats, int nchunks) {
  const int64_t bh = blockIdx.x;
  const int i = threadIdx.x;
  const float* p = part + (size_t)bh * nchunks * BLK * 2 + (size_t)i * 2;
  // unrolled so that the chunks' loads are in flight together (same order of operations)
  float M = -INFINITY;
#pragma unroll 16
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, p[(size_t)c * BLK * 2]);
  float L = 0.f;
#pragma unroll 16
  for (int c = 0; c < nchunks; ++c) L += p[(size_t)c * BLK * 2 + 1] * fast_exp2(p[(size_t)c * BLK * 2] - M);
  stats[((size_t)bh * BLK + i) * 2] = M;
  stats[((size_t)bh * BLK + i) * 2 + 1] = 1.f / L;
}

__global__ __launch_bounds__(NTHR) void route_finalize_kernel(
    const float* __restrict__ lu, float* __restrict__ p_vert, float* __restrict__ p_slash,
    float* __restrict__ c_struct, int8_t* __restrict__ pattern, int nb, float tau) {
  const int64_t bh = blockIdx.x;
  const float* t = lu + (size_t)bh * nb * 2;
  const float inv_b = 1.f / BLK;
  for (int kb = threadIdx.x; kb < nb; kb += NTHR) {
    const float L = t[2 * kb], U = t[2 * kb + 1];
    const float Up = kb ? t[2 * kb - 1] : 0.f;
    p_vert[(size_t)bh * nb + kb] = (L + U) * inv_b;
    p_slash[(size_t)bh * nb + kb] = (L + Up) * inv_b;
  }
  if (threadIdx.x == 0) {
    const float first = (t[0] + t[1]) * inv_b;
    const float last = (t[2 * (nb - 1)] + t[2 * (nb - 1) + 1]) * inv_b;
    const float c = first + last;
    c_struct[bh] = c;
    pattern[bh] = (c >= tau) ? 1 : 0;
  }
}

// Query heads per workgroup of the proxy pass: up to four (eight waves).
inline int proxy_hpw(int group) { return group >= 4 ? 4 : (group >= 2 ? 2 : 1); }

template <int D, int HPW>
hipError_t route_impl(const Dims& dm, float tau, const uint16_t* q, const uint16_t* k, float* c_struct,
                      int8_t* pattern, float* p_vert, float* p_slash, const RouteBufs& wb, hipStream_t st) {
  const int ct = proxy_chunk_tiles(dm), nch = proxy_num_chunks(dm);
  const float c2 = LOG2E / sqrtf((float)D);
  dim3 grid(nch, (unsigned)(dm.batch * dm.h_kv), (unsigned)((dm.group + HPW - 1) / HPW));
  proxy_tile_kernel<D, HPW><<<grid, 128 * HPW, 0, st>>>(q, k, wb.part, wb.tile, dm.n, dm.h_q, dm.group, ct, nch,
                                                         c2);
  proxy_combine_kernel<<<(unsigned)dm.bh, BLK, 0, st>>>(wb.part, wb.stats, nch);
  const unsigned rx = (unsigned)((dm.nb + 63) / 64);   // 16 tiles per wave
  proxy_reduce_kernel<<<dim3(rx, (unsigned)dm.bh), NTHR, 0, st>>>(wb.tile, wb.stats, wb.lu, dm.nb);
  route_finalize_kernel<<<(unsigned)dm.bh, NTHR, 0, st>>>(wb.lu, p_vert, p_slash, c_struct, pattern, dm.nb, tau);
  return hipGetLastError();
}

template <int D>
hipError_t route_dispatch(const Dims& dm, float tau, const uint16_t* q, const uint16_t* k, float* c_struct,
                          int8_t* pattern, float* p_vert, float* p_slash, const RouteBufs& wb, hipStream_t st) {
  switch (proxy_hpw(dm.group)) {
    case 4: return route_impl<D, 4>(dm, tau, q, k, c_struct, pattern, p_vert, p_slash, wb, st);
    case 2: return route_impl<D, 2>(dm, tau, q, k, c_struct, pattern, p_vert, p_slash, wb, st);
    default: return route_impl<D, 1>(dm, tau, q, k, c_struct, pattern, p_vert, p_slash, wb, st);
  }
}

}  // namespace

int proxy_chunk_tiles(const Dims& dm) {
  // Aim at about 1024 workgroups (of up to four query heads) per pass; at most 64 key tiles per workgroup.
  const int hpw = proxy_hpw(dm.group);
  const int64_t units = (int64_t)dm.nb * dm.batch * dm.h_kv * ((dm.group + hpw - 1) / hpw);
  int64_t ct = (units + 1023) / 1024;
  if (ct < 1) ct = 1;
  if (ct > 64) ct = 64;
  if (ct > dm.nb) ct = dm.nb;
  return (int)ct;
}

int proxy_num_chunks(const Dims& dm) {
  const int ct = proxy_chunk_tiles(dm);
  return (dm.nb + ct - 1) / ct;
}

hipError_t launch_route(const Dims& dm, float tau, const uint16_t* q, const uint16_t* k, float* c_struct,
                        int8_t* pattern, float* p_vert, float* p_slash, const RouteBufs& wb, hipStream_t st) {
  if (dm.d == 128) return route_dispatch<128>(dm, tau, q, k, c_struct, pattern, p_vert, p_slash, wb, st);
  return route_dispatch<64>(dm, tau, q, k, c_struct, pattern, p_vert, p_slash, wb, st);
}

}  // namespace crisp
