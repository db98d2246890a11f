// PatSearch on gfx950: proxy softmax of the last 128 queries against all keys,
// reduced on the fly to vertical / slash block scores and the structural mass.
//
// Method: digest page "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
// Structural-Mass-Motivated Routing", core-method section and Algorithm 2
// caption (proxy A_hat, C_struct over the first and last 128 keys, VS iff
// C_struct >= tau), and method-steps step 2 / Algorithm 3 caption (column and
// diagonal means of A_hat, block-pooled).
//
// A_hat (b x n per head) is never stored.  Pass 1 computes per proxy row the
// softmax max and normaliser over key chunks; a combine step merges chunks in
// a fixed order; pass 2 recomputes each 128x128 proxy tile, normalises it and
// sums its lower triangle with diagonal (in-tile key jj <= row i) into L and its
// strict upper triangle into U.  Because b equals the block size, an entry of
// key block kb lies on a diagonal t = j + b-1-i in slash block kb when jj <= i
// and kb+1 otherwise, so p_vert[kb] = (L_kb + U_kb)/b and
// p_slash[kb] = (L_kb + U_{kb-1})/b.  Every reduction has a fixed order.
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

template <int D>
__global__ __launch_bounds__(NTHR) void proxy_stats_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, float* __restrict__ part,
    int n, int h_q, int group, int chunk_tiles, int nchunks, float c2) {
  __shared__ __align__(16) uint16_t klds[Tile<D>::KLDS];
  const int chunk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / h_q), h = (int)(bh % h_q);
  const int h_kv = h_q / group, g = h / group;
  const int nb = n / BLK, qb = nb - 1;
  const uint16_t* qh = q + (size_t)bh * n * D;
  const uint16_t* kg = k + ((size_t)b * h_kv + g) * n * D;
  const int w = wave_id(), lane = lane_id();
  const int qloc = 32 * w + (lane & 31);

  bf16x8 qf[Tile<D>::NSTEP];
  load_q_operands<D>(qh + (size_t)(qb * BLK + 32 * w) * D, qf);

  float m = -INFINITY, l = 0.f;
  const int kb0 = chunk * chunk_tiles, kb1 = min(nb, kb0 + chunk_tiles);
  uint4 kr[Tile<D>::KCH];
  load_k_regs<D>(kg + (size_t)kb0 * BLK * D, kr);
  for (int kb = kb0; kb < kb1; ++kb) {
    store_k_lds<D>(klds, kr);
    __syncthreads();
    if (kb + 1 < kb1) load_k_regs<D>(kg + (size_t)(kb + 1) * BLK * D, kr);
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
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc += fast_exp2(s[ks][r] - mn);
    l = l * fast_exp2(m - mn) + acc;
    m = mn;
    __syncthreads();
  }
  l += xor_shfl(l, 32);
  if (lane < 32) {
    float* o = part + (((size_t)bh * nchunks + chunk) * BLK + qloc) * 2;
    o[0] = m;
    o[1] = l;
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

template <int D>
__global__ __launch_bounds__(NTHR) void proxy_pool_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ stats,
    float* __restrict__ lu, int n, int h_q, int group, int chunk_tiles, float c2) {
  __shared__ __align__(16) uint16_t klds[Tile<D>::KLDS];
  __shared__ float red[4][2];
  const int chunk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / h_q), h = (int)(bh % h_q);
  const int h_kv = h_q / group, g = h / group;
  const int nb = n / BLK, qb = nb - 1;
  const uint16_t* qh = q + (size_t)bh * n * D;
  const uint16_t* kg = k + ((size_t)b * h_kv + g) * n * D;
  const int w = wave_id(), lane = lane_id();
  const int qloc = 32 * w + (lane & 31);
  const float M = stats[((size_t)bh * BLK + qloc) * 2];
  const float invL = stats[((size_t)bh * BLK + qloc) * 2 + 1];

  bf16x8 qf[Tile<D>::NSTEP];
  load_q_operands<D>(qh + (size_t)(qb * BLK + 32 * w) * D, qf);

  const int kb0 = chunk * chunk_tiles, kb1 = min(nb, kb0 + chunk_tiles);
  uint4 kr[Tile<D>::KCH];
  load_k_regs<D>(kg + (size_t)kb0 * BLK * D, kr);
  for (int kb = kb0; kb < kb1; ++kb) {
    store_k_lds<D>(klds, kr);
    __syncthreads();
    if (kb + 1 < kb1) load_k_regs<D>(kg + (size_t)(kb + 1) * BLK * D, kr);
    f32x16 s[4];
    qk_tile<D>(klds, qf, s);
    const bool diag = (kb == qb);
    float lo = 0.f, up = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * ks + key_of_reg(r, lane);
        float p = fast_exp2(s[ks][r] * c2 - M) * invL;
        if (diag && key > qloc) p = 0.f;
        if (key <= qloc) lo += p; else up += p;
      }
    lo = wave_sum(lo);
    up = wave_sum(up);
    if (lane == 0) {
      red[w][0] = lo;
      red[w][1] = up;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float* o = lu + ((size_t)bh * nb + kb) * 2;
      o[0] = (red[0][0] + red[1][0]) + (red[2][0] + red[3][0]);
      o[1] = (red[0][1] + red[1][1]) + (red[2][1] + red[3][1]);
    }
  }
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

template <int D>
hipError_t route_impl(const Dims& dm, float tau, const uint16_t* q, const uint16_t* k, float* c_struct,
                      int8_t* pattern, float* p_vert, float* p_slash, float* ws_part, float* ws_stats,
                      float* ws_lu, hipStream_t st) {
  const int ct = proxy_chunk_tiles(dm), nch = proxy_num_chunks(dm);
  const float c2 = LOG2E / sqrtf((float)D);
  dim3 grid(nch, (unsigned)dm.bh);
  proxy_stats_kernel<D><<<grid, NTHR, 0, st>>>(q, k, ws_part, dm.n, dm.h_q, dm.group, ct, nch, c2);
  proxy_combine_kernel<<<(unsigned)dm.bh, BLK, 0, st>>>(ws_part, ws_stats, nch);
  proxy_pool_kernel<D><<<grid, NTHR, 0, st>>>(q, k, ws_stats, ws_lu, dm.n, dm.h_q, dm.group, ct, c2);
  route_finalize_kernel<<<(unsigned)dm.bh, NTHR, 0, st>>>(ws_lu, p_vert, p_slash, c_struct, pattern, dm.nb, tau);
  return hipGetLastError();
}

}  // namespace

int proxy_chunk_tiles(const Dims& dm) {
  // Aim at about 4096 workgroups per pass; at most 64 key tiles per workgroup.
  const int64_t units = (int64_t)dm.nb * dm.bh;
  int64_t ct = (units + 4095) / 4096;
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
                        int8_t* pattern, float* p_vert, float* p_slash, float* ws_part, float* ws_stats,
                        float* ws_lu, hipStream_t st) {
  if (dm.d == 128)
    return route_impl<128>(dm, tau, q, k, c_struct, pattern, p_vert, p_slash, ws_part, ws_stats, ws_lu, st);
  return route_impl<64>(dm, tau, q, k, c_struct, pattern, p_vert, p_slash, ws_part, ws_stats, ws_lu, st);
}

}  // namespace crisp
