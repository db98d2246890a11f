// Block selection on gfx950: VSIndex (sink-aware noise floor) for VS heads,
// PEIndex (pooled block map + global gamma-cumsum) for PE heads, and the
// block CSR that the attention kernel walks.
//
// Method: digest page "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
// Structural-Mass-Motivated Routing": method-steps steps 2-3, the Algorithm 3
// and Algorithm 4 captions, and the prerequisite section on the
// cumulative-coverage (gamma) threshold.
//
// The gamma-cumsum ("sort descending, accumulate until gamma") is computed
// without a sort: a three-pass radix select over the fp32 bit patterns of the
// (positive) scores finds the cut value T, the mass strictly above it and how
// many cells equal to T the prefix takes.  Masses are accumulated as unsigned
// 64-bit fixed point (2^-60 units) with integer atomics, so the result is
// exact up to the truncation of each score and independent of thread order.
// Cells equal to T are taken in flat-index order (ties to the lower index).
#include <math.h>

#include "crisp_device.hpp"
#include "crisp_internal.h"

namespace crisp {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int HBINS = 2048;
typedef unsigned long long u64;

enum { ST_PREFIX = 0, ST_ABOVE = 1, ST_NEED = 2, ST_T = 3, ST_TAKE = 4, ST_ALL = 5, ST_WORDS = 8 };

__device__ __forceinline__ u64 mass_fx(uint32_t key) {
  // score (a non-negative float) -> floor(score * 2^60); exact scaling by a power of two
  const float x = __uint_as_float(key) * 0x1p60f;
  return (u64)x;
}

__device__ __forceinline__ int64_t tri_off(int qb) { return (int64_t)qb * (qb + 1) / 2; }

// ------------------------------------------------------------------------------------------------
// Block-wide helpers (256 threads)
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  const float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}
__device__ __forceinline__ int block_count(int v, int* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  const int t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}

// ------------------------------------------------------------------------------------------------
// VSIndex: per direction, mu = max(1 - p[0] - p[N_b-1], 0)/(N_b-2); keep p > alpha*mu, at least
// kmin (top-k, ties to the lower index), then add the anchors 0 and N_b-1.
// ------------------------------------------------------------------------------------------------
constexpr int MAX_NB = 8192;   // n <= 1,048,576 tokens
constexpr int RANK_NB = 1024;  // up to this many blocks the top-k fallback ranks every block at once

__global__ __launch_bounds__(NTHR) void vs_select_kernel(
    const int8_t* __restrict__ pattern, const float* __restrict__ p_vert, const float* __restrict__ p_slash,
    uint8_t* __restrict__ vsflags, uint8_t* __restrict__ sel_mask, int nb, float alpha, int kmin) {
  __shared__ int ired[4];
  __shared__ float fv[4];
  __shared__ int fi[4];
  __shared__ uint8_t fl[MAX_NB];
  __shared__ float pv[RANK_NB];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const bool vs = pattern[bh] == 1;
  for (int dir = 0; dir < 2; ++dir) {
    uint8_t* gfl = vsflags + ((size_t)bh * 2 + dir) * nb;
    uint8_t* sm = sel_mask ? sel_mask + ((size_t)bh * 2 + dir) * nb : nullptr;
    if (!vs) {
      for (int j = tid; j < nb; j += NTHR) {
        gfl[j] = 0;
        if (sm) sm[j] = 0;
      }
      continue;
    }
    const float* p = (dir ? p_slash : p_vert) + (size_t)bh * nb;
    const float r = fmaxf((1.f - p[0]) - p[nb - 1], 0.f);
    const float mu = r / (float)(nb - 2);
    const float thr = alpha * mu;
    int c = 0;
    for (int j = tid; j < nb; j += NTHR) c += (p[j] > thr) ? 1 : 0;
    const int cnt = block_count(c, ired);
    int kk = cnt > kmin ? cnt : kmin;
    if (kk > nb) kk = nb;
    if (kk == cnt) {
      for (int j = tid; j < nb; j += NTHR) fl[j] = (p[j] > thr) ? 1 : 0;
    } else if (kk == nb) {
      for (int j = tid; j < nb; j += NTHR) fl[j] = 1;
    } else if (nb <= RANK_NB) {
      // fewer than kmin blocks above the floor: the kk blocks first in the order (score
      // descending, index ascending), i.e. those with fewer than kk blocks before them
      for (int j = tid; j < nb; j += NTHR) pv[j] = p[j];
      __syncthreads();
      for (int j = tid; j < nb; j += NTHR) {
        const float x = pv[j];
        int before = 0;
        for (int i = 0; i < nb; ++i) {
          const float y = pv[i];
          before += (y > x || (y == x && i < j)) ? 1 : 0;
        }
        fl[j] = before < kk ? 1 : 0;
      }
    } else {
      // fewer than kmin blocks above the floor: top-kmin by score, ties to the lower index
      for (int j = tid; j < nb; j += NTHR) fl[j] = 0;
      __syncthreads();
      for (int it = 0; it < kk; ++it) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int j = tid; j < nb; j += NTHR) {
          if (fl[j]) continue;
          const float x = p[j];
          if (bi == 0x7fffffff || x > bv || (x == bv && j < bi)) { bv = x; bi = j; }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
          const float ov = __shfl_xor(bv, m, 64);
          const int oi = __shfl_xor(bi, m, 64);
          if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
        }
        if (lane_id() == 0) { fv[wave_id()] = bv; fi[wave_id()] = bi; }
        __syncthreads();
        if (tid == 0) {
          float v0 = fv[0];
          int i0 = fi[0];
          for (int ww = 1; ww < 4; ++ww)
            if (fi[ww] != 0x7fffffff && (i0 == 0x7fffffff || fv[ww] > v0 || (fv[ww] == v0 && fi[ww] < i0))) {
              v0 = fv[ww];
              i0 = fi[ww];
            }
          if (i0 >= 0 && i0 < nb) fl[i0] = 1;
        }
        __syncthreads();
      }
    }
    __syncthreads();
    if (tid == 0) {
      fl[0] = 1;
      fl[nb - 1] = 1;
    }
    __syncthreads();
    for (int j = tid; j < nb; j += NTHR) {
      gfl[j] = fl[j];
      if (sm) sm[j] = fl[j];
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// PEIndex step 1: mean-pool Q (PE heads) and K (groups serving a PE head) over each 128-token block.
// ------------------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void pool_block(const uint16_t* __restrict__ src, float* __restrict__ dst, float* red) {
  constexpr int CP = D / 2;            // column pairs
  constexpr int RG = NTHR / CP;        // row groups
  constexpr int RPG = BLK / RG;        // rows per group
  const int tid = threadIdx.x;
  const int cp = tid % CP, rg = tid / CP;
  float a0 = 0.f, a1 = 0.f;
  const uint16_t* p = src + (size_t)(rg * RPG) * D + 2 * cp;
  for (int r = 0; r < RPG; ++r) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p + (size_t)r * D);
    a0 += __uint_as_float(u << 16);
    a1 += __uint_as_float(u & 0xFFFF0000u);
  }
  red[rg * D + 2 * cp] = a0;
  red[rg * D + 2 * cp + 1] = a1;
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += red[g * D + tid];
    dst[tid] = s * (1.f / BLK);
  }
}

template <int D>
__global__ __launch_bounds__(NTHR) void pool_q_kernel(const uint16_t* __restrict__ q, const int8_t* __restrict__ pattern,
                                                      float* __restrict__ qbar, int n) {
  __shared__ float red[NTHR * 2];
  const int qb = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (pattern[bh] != 0) return;
  const int nb = n / BLK;
  pool_block<D>(q + ((size_t)bh * n + (size_t)qb * BLK) * D, qbar + ((size_t)bh * nb + qb) * D, red);
}

template <int D>
__global__ __launch_bounds__(NTHR) void pool_k_kernel(const uint16_t* __restrict__ k, const int8_t* __restrict__ pattern,
                                                      float* __restrict__ kbar, int n, int h_q, int group) {
  __shared__ float red[NTHR * 2];
  const int kb = blockIdx.x;
  const int64_t bg = blockIdx.y;  // batch * h_kv + g
  const int h_kv = h_q / group;
  const int b = (int)(bg / h_kv), g = (int)(bg % h_kv);
  bool any_pe = false;
  for (int j = 0; j < group; ++j) any_pe |= pattern[(size_t)b * h_q + g * group + j] == 0;
  if (!any_pe) return;
  const int nb = n / BLK;
  pool_block<D>(k + ((size_t)bg * n + (size_t)kb * BLK) * D, kbar + ((size_t)bg * nb + kb) * D, red);
}

// ------------------------------------------------------------------------------------------------
// PEIndex step 2: block-causal pooled logits y = qbar . kbar * log2(e)/sqrt(d), 64x64 tiles (fp32).
// ------------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NTHR) void pe_logits_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                         const int8_t* __restrict__ pattern, float* __restrict__ abar,
                                                         int nb, int h_q, int group, int64_t tri, float c2) {
  __shared__ float qs[64][33];
  __shared__ float ks[64][33];
  const int64_t bh = blockIdx.y;
  if (pattern[bh] != 0) return;
  // lower-triangular tile pair (ti >= tj) from the linear id
  const int L = blockIdx.x;
  int ti = (int)((sqrtf(8.f * L + 1.f) - 1.f) * 0.5f);
  while ((ti + 1) * (ti + 2) / 2 <= L) ++ti;
  while (ti * (ti + 1) / 2 > L) --ti;
  const int tj = L - ti * (ti + 1) / 2;
  const int b = (int)(bh / h_q), h = (int)(bh % h_q);
  const int h_kv = h_q / group;
  const float* qsrc = qbar + (size_t)bh * nb * D;
  const float* ksrc = kbar + ((size_t)b * h_kv + h / group) * nb * D;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int dc = 0; dc < D; dc += 32) {
    for (int e = tid; e < 64 * 32; e += NTHR) {
      const int r = e / 32, c = e % 32;
      const int qr = ti * 64 + r, kr = tj * 64 + r;
      qs[r][c] = qr < nb ? qsrc[(size_t)qr * D + dc + c] : 0.f;
      ks[r][c] = kr < nb ? ksrc[(size_t)kr * D + dc + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = qs[4 * ty + i][kk]; bb[i] = ks[4 * tx + i][kk]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* dst = abar + (size_t)bh * tri;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qb = ti * 64 + 4 * ty + i;
    if (qb >= nb) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = tj * 64 + 4 * tx + j;
      if (kb <= qb) dst[tri_off(qb) + kb] = acc[i][j] * c2;
    }
  }
}

// PEIndex step 3: row softmax over kb <= qb, then x = A_bar / N_b (in place).
__global__ __launch_bounds__(NTHR) void pe_softmax_kernel(const int8_t* __restrict__ pattern, float* __restrict__ abar,
                                                          int nb, int64_t tri) {
  __shared__ float red[4];
  const int qb = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (pattern[bh] != 0) return;
  float* row = abar + (size_t)bh * tri + tri_off(qb);
  const int len = qb + 1;
  // Loads four strides at a time so that each thread has four in flight; every thread still adds
  // its entries in index order.
  float m = -INFINITY;
  for (int j0 = threadIdx.x; j0 < len; j0 += 4 * NTHR) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = j0 + u * NTHR < len ? row[j0 + u * NTHR] : -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) m = fmaxf(m, v[u]);
  }
  m = block_max(m, red);
  float s = 0.f;
  for (int j0 = threadIdx.x; j0 < len; j0 += 4 * NTHR) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = j0 + u * NTHR < len ? row[j0 + u * NTHR] : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j0 + u * NTHR < len) s += fast_exp2(v[u] - m);
  }
  s = block_sum(s, red);
  const float fnb = (float)nb;
  for (int j = threadIdx.x; j < len; j += NTHR) row[j] = fast_exp2(row[j] - m) / s / fnb;
}

// ------------------------------------------------------------------------------------------------
// gamma-cumsum as a radix select over the score bits (three passes: 11, 11, 10 bits).
// ------------------------------------------------------------------------------------------------
__global__ void zero_u64_kernel(u64* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void pe_state_init_kernel(const int8_t* __restrict__ pattern, u64* __restrict__ state, int64_t bh_total,
                                     u64 need) {
  const int64_t bh = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (bh >= bh_total) return;
  u64* s = state + bh * ST_WORDS;
  s[ST_PREFIX] = 0;
  s[ST_ABOVE] = 0;
  s[ST_NEED] = need;
  s[ST_T] = 0;
  s[ST_TAKE] = 0;
  s[ST_ALL] = 0;
}

__device__ __forceinline__ void pass_bits(int pass, int& shift, int& width) {
  shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
  width = pass == 2 ? 10 : 11;
}

// Adds to the LDS histogram lm, by this pass's digit, the masses of the cells keys[e] for
// e = e0, e0 + NTHR, ... < e1 (filter: only those whose bits above the digit equal prefix).  Eight
// loads are in flight per thread.  A thread adds its cells' masses in a register while they fall in
// the same bucket and flushes the run with one LDS atomic when the bucket changes: on a smooth map
// most lanes of a wave hit the same bucket, and one atomic per cell would serialise on it.  The
// sums are exact integers, so the grouping does not change them.
__device__ __forceinline__ void hist_cells(const uint32_t* __restrict__ keys, int64_t e0, int64_t e1, bool filter,
                                           int shift, int pshift, uint32_t dmask, uint32_t prefix, u64* lm) {
  constexpr int U = 8;
  uint32_t run_dig = 0;
  u64 run_mass = 0;
  for (int64_t e = e0; e < e1; e += U * NTHR) {
    uint32_t kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kv[u] = e + u * NTHR < e1 ? keys[e + u * NTHR] : 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t key = kv[u];
      if (e + u * NTHR >= e1 || (filter && (key >> pshift) != prefix)) continue;
      const uint32_t dig = (key >> shift) & dmask;
      if (dig != run_dig) {
        if (run_mass) atomicAdd(&lm[run_dig], run_mass);
        run_dig = dig;
        run_mass = 0;
      }
      run_mass += mass_fx(key);
    }
  }
  if (run_mass) atomicAdd(&lm[run_dig], run_mass);
}

constexpr int HIST_CHUNK = 65536;

__global__ __launch_bounds__(NTHR) void pe_hist_kernel(const int8_t* __restrict__ pattern, const float* __restrict__ abar,
                                                       const u64* __restrict__ state, u64* __restrict__ hmass,
                                                       int64_t tri, int pass) {
  __shared__ u64 lm[HBINS];
  const int64_t bh = blockIdx.y;
  if (pattern[bh] != 0) return;
  const u64* st = state + bh * ST_WORDS;
  if (st[ST_ALL]) return;
  int shift, width;
  pass_bits(pass, shift, width);
  const int pshift = shift + width;                  // bits above this pass's digit
  const uint32_t prefix = (uint32_t)st[ST_PREFIX];
  for (int i = threadIdx.x; i < HBINS; i += NTHR) lm[i] = 0;
  __syncthreads();
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(abar + (size_t)bh * tri);
  const int64_t e0 = (int64_t)blockIdx.x * HIST_CHUNK;
  const int64_t e1 = e0 + HIST_CHUNK < tri ? e0 + HIST_CHUNK : tri;
  const uint32_t dmask = (1u << width) - 1u;
  hist_cells(keys, e0 + threadIdx.x, e1, pass > 0, shift, pshift, dmask, prefix, lm);
  __syncthreads();
  u64* gm = hmass + bh * HBINS;
  for (int i = threadIdx.x; i < HBINS; i += NTHR)
    if (lm[i]) atomicAdd(&gm[i], lm[i]);
}

// Run by one full wave: the first bucket, from the top (nbk - 1) down, at which the running mass
// reaches rem.  Lane j sums its buckets nbk-1-per*j down to nbk-per*(j+1) (per = nbk / 64),
// starting at a lane-rotated offset so that the wave's LDS reads fall in distinct banks; an
// inclusive prefix over the lanes finds the lane that crosses rem, and that lane walks its own
// buckets.  Returns false on every lane when all buckets together stay below rem; otherwise lane
// `owner` gets the bucket (`found`) and the mass of the buckets above it (`above`).  The same
// bucket and mass as a walk from the top over all buckets: the sums are exact integers.
__device__ __forceinline__ bool wave_bucket_search(const u64* lm, int nbk, u64 rem, int lane, int& owner, int& found,
                                                   u64& above) {
  const int per = nbk / 64, top = nbk - 1 - per * lane;
  u64 own = 0;
  for (int i = 0; i < per; ++i) own += lm[top - (i + lane) % per];
  u64 incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const u64 v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  const u64 hit = __ballot(incl >= rem);
  if (hit == 0) return false;
  owner = __builtin_ctzll(hit);
  if (lane == owner) {
    u64 cum = incl - own;
    int f = top - per + 1;
    for (int i = 0; i < per; ++i) {
      if (cum + lm[top - i] >= rem) {
        f = top - i;
        break;
      }
      cum += lm[top - i];
    }
    found = f;
    above = cum;
  }
  return true;
}

// Reads the head's histogram of this pass and clears it for the next one (a head whose
// histogram is never filled again, VS or already decided, keeps a cleared one).
__global__ __launch_bounds__(NTHR) void pe_find_kernel(const int8_t* __restrict__ pattern, u64* __restrict__ hmass,
                                                       u64* __restrict__ state, int pass) {
  __shared__ u64 lm[HBINS];
  const int64_t bh = blockIdx.x;
  if (pattern[bh] != 0) return;
  u64* st = state + bh * ST_WORDS;
  if (st[ST_ALL]) return;
  for (int i = threadIdx.x; i < HBINS; i += NTHR) {
    lm[i] = hmass[bh * HBINS + i];
    hmass[bh * HBINS + i] = 0;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int shift, width;
  pass_bits(pass, shift, width);
  const u64 need = st[ST_NEED] - st[ST_ABOVE];
  int owner = 0, found = 0;
  u64 cum = 0;
  if (!wave_bucket_search(lm, 1 << width, need, lane, owner, found, cum)) {
    // the whole map sums to less than gamma: keep every cell
    if (lane == 0) {
      st[ST_ALL] = 1;
      st[ST_T] = 0;
      st[ST_TAKE] = ~0ull;
    }
    return;
  }
  if (lane != owner) return;
  st[ST_PREFIX] = (st[ST_PREFIX] << width) | (u64)found;
  st[ST_ABOVE] += cum;
  if (pass == 2) {
    const uint32_t T = (uint32_t)st[ST_PREFIX];
    st[ST_T] = T;
    const u64 rem = st[ST_NEED] - st[ST_ABOVE];
    const u64 mt = mass_fx(T);
    st[ST_TAKE] = mt ? (rem + mt - 1) / mt : ~0ull;
  }
}

// ------------------------------------------------------------------------------------------------
// Per-row PEIndex (variant): the gamma-cumsum inside each row of the pooled map, as the same
// three-pass radix select run over one row per workgroup in LDS.  need = gamma / N_b in the
// fixed point (a row of x = A_bar / N_b sums to 1 / N_b).  rowst[r] = {T, take}: the row keeps
// its cells above T and its first `take` cells equal to T (~0: all of them).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(NTHR) void pe_row_select_kernel(const int8_t* __restrict__ pattern,
                                                             const float* __restrict__ abar, u64* __restrict__ rowst,
                                                             int nb, int64_t tri, u64 need) {
  __shared__ u64 lm[HBINS];
  __shared__ u64 sh[3];   // prefix, mass above, done
  const int qb = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (pattern[bh] != 0) return;
  const int64_t r = bh * nb + qb;
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(abar + (size_t)bh * tri + tri_off(qb));
  const int len = qb + 1;
  const int tid = threadIdx.x, lane = lane_id();
  if (tid == 0) { sh[0] = 0; sh[1] = 0; sh[2] = 0; }
  for (int pass = 0; pass < 3; ++pass) {
    int shift, width;
    pass_bits(pass, shift, width);
    const int pshift = shift + width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = tid; i < HBINS; i += NTHR) lm[i] = 0;
    __syncthreads();
    const uint32_t prefix = (uint32_t)sh[0];
    hist_cells(keys, tid, len, pass > 0, shift, pshift, dmask, prefix, lm);
    __syncthreads();
    if (tid < 64) {
      int owner = 0, found = 0;
      u64 cum = 0;
      if (!wave_bucket_search(lm, 1 << width, need - sh[1], lane, owner, found, cum)) {
        if (lane == 0) sh[2] = 1;   // the row sums to less than gamma: keep it all
      } else if (lane == owner) {
        sh[0] = (sh[0] << width) | (u64)found;
        sh[1] += cum;
      }
    }
    __syncthreads();
    if (sh[2]) break;
  }
  if (tid == 0) {
    if (sh[2]) {
      rowst[2 * r] = 0;
      rowst[2 * r + 1] = ~0ull;
    } else {
      const uint32_t T = (uint32_t)sh[0];
      const u64 rem = need - sh[1];
      const u64 mt = mass_fx(T);
      rowst[2 * r] = T;
      rowst[2 * r + 1] = mt ? (rem + mt - 1) / mt : ~0ull;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// CSR: count per row, per-head tie allocation (PE), exclusive scan, fill.
// ------------------------------------------------------------------------------------------------
// Whether VS row qb keeps tile (qb, kb): tile (qb, kb) lies on block diagonal qb - kb, i.e. in
// selected slash block nb-1-(qb-kb), or with the band in the slash block of diagonal qb-kb-1
// (nb-(qb-kb)), whose tokens reach this tile.  Every read stays in bounds for any kb (indices are
// clamped), so a caller can issue several without branches; kb > qb is never kept.
__device__ __forceinline__ bool vs_cell(const uint8_t* vert, const uint8_t* slash, int nb, int qb, int kb, int band) {
  const int kc = kb < qb ? kb : qb;
  const int kd = kc < qb ? kc : qb - 1;
  const uint8_t v = vert[kc], s0 = slash[nb - 1 - qb + kc], s1 = slash[nb - qb + kd];
  return kb <= qb && (v | s0 | (band && kb < qb && s1));
}

// The CSR passes read a row 64 * CSR_U entries at a time (CSR_U loads in flight per lane).
constexpr int CSR_U = 4;

__global__ __launch_bounds__(64) void row_count_kernel(const int8_t* __restrict__ pattern, const uint8_t* __restrict__ vsflags,
                                                       const float* __restrict__ abar, const u64* __restrict__ state,
                                                       int64_t* __restrict__ rowcnt, int32_t* __restrict__ eqcnt,
                                                       int32_t* __restrict__ seltake, int nb, int64_t tri, int band,
                                                       const u64* __restrict__ rowst) {
  const int64_t r = blockIdx.x;
  const int64_t bh = r / nb;
  const int qb = (int)(r % nb);
  const int lane = threadIdx.x;
  if (pattern[bh] == 1) {
    const uint8_t* vert = vsflags + (size_t)bh * 2 * nb;
    const uint8_t* slash = vert + nb;
    int cnt = 0;
    for (int kb0 = 0; kb0 <= qb; kb0 += 64 * CSR_U) {
      bool sel[CSR_U];
#pragma unroll
      for (int u = 0; u < CSR_U; ++u) sel[u] = vs_cell(vert, slash, nb, qb, kb0 + 64 * u + lane, band);
#pragma unroll
      for (int u = 0; u < CSR_U; ++u) cnt += __popcll(__ballot(sel[u]));
    }
    if (lane == 0) { rowcnt[r] = cnt; eqcnt[r] = 0; seltake[r] = 0; }
    return;
  }
  const uint32_t T = rowst ? (uint32_t)rowst[2 * r] : (uint32_t)state[bh * ST_WORDS + ST_T];
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(abar + (size_t)bh * tri + tri_off(qb));
  int gt = 0, eq = 0;
  for (int kb0 = 0; kb0 <= qb; kb0 += 64 * CSR_U) {
    uint32_t kv[CSR_U];
#pragma unroll
    for (int u = 0; u < CSR_U; ++u) kv[u] = keys[min(kb0 + 64 * u + lane, qb)];
#pragma unroll
    for (int u = 0; u < CSR_U; ++u) {
      const bool valid = kb0 + 64 * u + lane <= qb;
      gt += __popcll(__ballot(valid && kv[u] > T));
      eq += __popcll(__ballot(valid && kv[u] == T));
    }
  }
  if (lane == 0) {
    const uint32_t dk = keys[qb];
    if (rowst) {
      // per-row cut: the row's own ties, in block order; the diagonal is the row's last cell
      const u64 take = rowst[2 * r + 1];
      const int tk = take >= (u64)eq ? eq : (int)take;
      const bool diag_sel = dk > T || (dk == T && eq <= tk);
      rowcnt[r] = gt + tk + (diag_sel ? 0 : 1);
      eqcnt[r] = eq;
      seltake[r] = tk;
    } else {
      rowcnt[r] = gt;
      eqcnt[r] = eq;
      seltake[r] = dk > T ? 2 : (dk == T ? 1 : 0);   // class of the diagonal cell, resolved by pe_ties_kernel
    }
  }
}

// Allocates the cells equal to T to rows in flat order and finishes the PE row counts.
__global__ __launch_bounds__(NTHR) void pe_ties_kernel(const int8_t* __restrict__ pattern, const u64* __restrict__ state,
                                                       int64_t* __restrict__ rowcnt, const int32_t* __restrict__ eqcnt,
                                                       int32_t* __restrict__ seltake, int nb) {
  __shared__ int64_t part[NTHR];
  const int64_t bh = blockIdx.x;
  if (pattern[bh] != 0) return;
  const u64 take = state[bh * ST_WORDS + ST_TAKE];
  const int tid = threadIdx.x;
  const int per = (nb + NTHR - 1) / NTHR;
  const int r0 = tid * per, r1 = min(nb, r0 + per);
  int64_t loc = 0;
  for (int qb = r0; qb < r1; ++qb) loc += eqcnt[bh * nb + qb];
  part[tid] = loc;
  __syncthreads();
  if (tid == 0) {
    int64_t acc = 0;
    for (int i = 0; i < NTHR; ++i) { const int64_t v = part[i]; part[i] = acc; acc += v; }
  }
  __syncthreads();
  int64_t before = part[tid];
  for (int qb = r0; qb < r1; ++qb) {
    const int64_t r = bh * nb + qb;
    const int64_t eq = eqcnt[r];
    int64_t tk;
    if (take == ~0ull) tk = eq;
    else {
      const int64_t left = (int64_t)take - before;
      tk = left <= 0 ? 0 : (left < eq ? left : eq);
    }
    const int cls = seltake[r];
    const bool diag_sel = cls == 2 || (cls == 1 && tk == eq);
    rowcnt[r] = rowcnt[r] + tk + (diag_sel ? 0 : 1);
    seltake[r] = (int32_t)tk;
    before += eq;
  }
}

constexpr int SCAN_PER = 1024;   // elements per scan block (256 threads x 4)

__global__ __launch_bounds__(NTHR) void scan_blocks_kernel(const int64_t* __restrict__ cnt, int64_t* __restrict__ part, int64_t n) {
  __shared__ int64_t red[NTHR];
  const int64_t base = (int64_t)blockIdx.x * SCAN_PER;
  int64_t s = 0;
  for (int i = 0; i < 4; ++i) {
    const int64_t e = base + threadIdx.x * 4 + i;
    if (e < n) s += cnt[e];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = NTHR / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(NTHR) void scan_top_kernel(int64_t* __restrict__ part, int64_t nblk) {
  __shared__ int64_t seg[NTHR];
  const int tid = threadIdx.x;
  const int64_t per = (nblk + NTHR - 1) / NTHR;
  const int64_t b0 = tid * per, b1 = b0 + per < nblk ? b0 + per : nblk;
  int64_t s = 0;
  for (int64_t i = b0; i < b1; ++i) s += part[i];
  seg[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int64_t acc = 0;
    for (int i = 0; i < NTHR; ++i) { const int64_t v = seg[i]; seg[i] = acc; acc += v; }
    part[nblk] = acc;
  }
  __syncthreads();
  int64_t acc = seg[tid];
  for (int64_t i = b0; i < b1; ++i) { const int64_t v = part[i]; part[i] = acc; acc += v; }
}

__global__ __launch_bounds__(NTHR) void scan_apply_kernel(const int64_t* __restrict__ cnt, const int64_t* __restrict__ part,
                                                          int64_t* __restrict__ row_ptr, int64_t n, int64_t nblk) {
  __shared__ int64_t red[NTHR];
  const int64_t base = (int64_t)blockIdx.x * SCAN_PER;
  int64_t v[4];
  int64_t s = 0;
  for (int i = 0; i < 4; ++i) {
    const int64_t e = base + threadIdx.x * 4 + i;
    v[i] = e < n ? cnt[e] : 0;
    s += v[i];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  // inclusive Hillis-Steele scan over the 256 thread sums
  for (int o = 1; o < NTHR; o <<= 1) {
    const int64_t add = (int)threadIdx.x >= o ? red[threadIdx.x - o] : 0;
    __syncthreads();
    red[threadIdx.x] += add;
    __syncthreads();
  }
  int64_t acc = part[blockIdx.x] + red[threadIdx.x] - s;
  for (int i = 0; i < 4; ++i) {
    const int64_t e = base + threadIdx.x * 4 + i;
    if (e < n) row_ptr[e] = acc;
    acc += v[i];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[n] = part[nblk];
}

__global__ __launch_bounds__(64) void fill_kernel(const int8_t* __restrict__ pattern, const uint8_t* __restrict__ vsflags,
                                                  const float* __restrict__ abar, const u64* __restrict__ state,
                                                  const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ seltake,
                                                  int32_t* __restrict__ col_idx, int nb, int64_t tri, int band,
                                                  const u64* __restrict__ rowst) {
  const int64_t r = blockIdx.x;
  const int64_t bh = r / nb;
  const int qb = (int)(r % nb);
  const int lane = threadIdx.x;
  const u64 below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int32_t* out = col_idx + row_ptr[r];
  int pos = 0;
  if (pattern[bh] == 1) {
    const uint8_t* vert = vsflags + (size_t)bh * 2 * nb;
    const uint8_t* slash = vert + nb;
    for (int kb0 = 0; kb0 <= qb; kb0 += 64 * CSR_U) {
      bool sel[CSR_U];
#pragma unroll
      for (int u = 0; u < CSR_U; ++u) sel[u] = vs_cell(vert, slash, nb, qb, kb0 + 64 * u + lane, band);
#pragma unroll
      for (int u = 0; u < CSR_U; ++u) {
        const u64 bal = __ballot(sel[u]);
        if (sel[u]) out[pos + __popcll(bal & below)] = kb0 + 64 * u + lane;
        pos += __popcll(bal);
      }
    }
    return;
  }
  const uint32_t T = rowst ? (uint32_t)rowst[2 * r] : (uint32_t)state[bh * ST_WORDS + ST_T];
  const int take = seltake[r];
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(abar + (size_t)bh * tri + tri_off(qb));
  int ties = 0;
  for (int kb0 = 0; kb0 <= qb; kb0 += 64 * CSR_U) {
    uint32_t kv[CSR_U];
#pragma unroll
    for (int u = 0; u < CSR_U; ++u) kv[u] = keys[min(kb0 + 64 * u + lane, qb)];
#pragma unroll
    for (int u = 0; u < CSR_U; ++u) {
      const int kb = kb0 + 64 * u + lane;
      const bool valid = kb <= qb;
      const uint32_t key = kv[u];
      const bool eq = valid && key == T;
      const u64 beq = __ballot(eq);
      const int eqrank = ties + __popcll(beq & below);
      const bool sel = valid && (key > T || (eq && eqrank < take) || kb == qb);
      const u64 bal = __ballot(sel);
      if (sel) out[pos + __popcll(bal & below)] = kb;
      pos += __popcll(bal);
      ties += __popcll(beq);
    }
  }
}

template <int D>
hipError_t select_impl(const Dims& dm, float alpha, float gamma, int kmin, const uint16_t* q, const uint16_t* k,
                       const int8_t* pattern, const float* p_vert, const float* p_slash, int64_t* row_ptr,
                       int32_t* col_idx, uint8_t* sel_mask, const SelectWs& ws, hipStream_t st, int vs_rule,
                       int band, int pe_rows) {
  const int nb = dm.nb;
  const unsigned bh = (unsigned)dm.bh;
  if (vs_rule == VS_GAMMA_CUMSUM) {
    const hipError_t e = launch_flex_vs(dm, gamma, kmin, pattern, p_vert, p_slash, ws.vsflags, sel_mask, st);
    if (e != hipSuccess) return e;
  } else if (vs_rule == VS_MEDIAN_FLOOR) {
    const hipError_t e = launch_median_vs(dm, alpha, kmin, pattern, p_vert, p_slash, ws.vsflags, sel_mask, st);
    if (e != hipSuccess) return e;
  } else {
    vs_select_kernel<<<bh, NTHR, 0, st>>>(pattern, p_vert, p_slash, ws.vsflags, sel_mask, nb, alpha, kmin);
  }
  pool_q_kernel<D><<<dim3(nb, bh), NTHR, 0, st>>>(q, pattern, ws.qbar, dm.n);
  pool_k_kernel<D><<<dim3(nb, (unsigned)(dm.batch * dm.h_kv)), NTHR, 0, st>>>(k, pattern, ws.kbar, dm.n, dm.h_q, dm.group);
  const int tiles = (nb + 63) / 64;
  const int pairs = tiles * (tiles + 1) / 2;
  const float c2 = LOG2E / sqrtf((float)D);
  pe_logits_kernel<D><<<dim3(pairs, bh), NTHR, 0, st>>>(ws.qbar, ws.kbar, pattern, ws.abar, nb, dm.h_q, dm.group, dm.tri, c2);
  pe_softmax_kernel<<<dim3(nb, bh), NTHR, 0, st>>>(pattern, ws.abar, nb, dm.tri);
  const u64* rowst = nullptr;
  if (pe_rows) {
    const u64 need_row = (u64)ceil((double)gamma / (double)nb * 0x1p60);
    pe_row_select_kernel<<<dim3(nb, bh), NTHR, 0, st>>>(pattern, ws.abar, ws.pe_rowst, nb, dm.tri, need_row);
    rowst = ws.pe_rowst;
    row_count_kernel<<<(unsigned)dm.rows, 64, 0, st>>>(pattern, ws.vsflags, ws.abar, ws.pe_state, ws.rowcnt, ws.eqcnt,
                                                        ws.seltake, nb, dm.tri, band, rowst);
  } else {
    const u64 need = (u64)ceil((double)gamma * 0x1p60);
    pe_state_init_kernel<<<(bh + 255) / 256, 256, 0, st>>>(pattern, ws.pe_state, dm.bh, need);
    const unsigned hchunks = (unsigned)((dm.tri + HIST_CHUNK - 1) / HIST_CHUNK);
    zero_u64_kernel<<<256, 256, 0, st>>>(ws.hist_mass, dm.bh * HBINS);   // later passes: cleared by pe_find
    for (int pass = 0; pass < 3; ++pass) {
      pe_hist_kernel<<<dim3(hchunks, bh), NTHR, 0, st>>>(pattern, ws.abar, ws.pe_state, ws.hist_mass, dm.tri, pass);
      pe_find_kernel<<<bh, NTHR, 0, st>>>(pattern, ws.hist_mass, ws.pe_state, pass);
    }
    row_count_kernel<<<(unsigned)dm.rows, 64, 0, st>>>(pattern, ws.vsflags, ws.abar, ws.pe_state, ws.rowcnt, ws.eqcnt,
                                                        ws.seltake, nb, dm.tri, band, nullptr);
    pe_ties_kernel<<<bh, NTHR, 0, st>>>(pattern, ws.pe_state, ws.rowcnt, ws.eqcnt, ws.seltake, nb);
  }
  const int64_t nblk = (dm.rows + SCAN_PER - 1) / SCAN_PER;
  scan_blocks_kernel<<<(unsigned)nblk, NTHR, 0, st>>>(ws.rowcnt, ws.scan_part, dm.rows);
  scan_top_kernel<<<1, NTHR, 0, st>>>(ws.scan_part, nblk);
  scan_apply_kernel<<<(unsigned)nblk, NTHR, 0, st>>>(ws.rowcnt, ws.scan_part, row_ptr, dm.rows, nblk);
  fill_kernel<<<(unsigned)dm.rows, 64, 0, st>>>(pattern, ws.vsflags, ws.abar, ws.pe_state, row_ptr, ws.seltake, col_idx,
                                                nb, dm.tri, band, rowst);
  return hipGetLastError();
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t select_ws_layout(const Dims& dm, SelectWs* ws, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  SelectWs w{};
  w.vsflags = (uint8_t*)take((size_t)dm.bh * 2 * dm.nb);
  w.qbar = (float*)take((size_t)dm.bh * dm.nb * dm.d * 4);
  w.kbar = (float*)take((size_t)dm.batch * dm.h_kv * dm.nb * dm.d * 4);
  w.abar = (float*)take((size_t)dm.bh * dm.tri * 4);
  w.hist_mass = (unsigned long long*)take((size_t)dm.bh * HBINS * 8);
  w.pe_state = (unsigned long long*)take((size_t)dm.bh * ST_WORDS * 8);
  w.rowcnt = (int64_t*)take((size_t)dm.rows * 8);
  w.eqcnt = (int32_t*)take((size_t)dm.rows * 4);
  w.seltake = (int32_t*)take((size_t)dm.rows * 4);
  w.scan_part = (int64_t*)take((size_t)((dm.rows + SCAN_PER - 1) / SCAN_PER + 1) * 8);
  w.pe_rowst = (unsigned long long*)take((size_t)dm.rows * 16);
  if (ws) *ws = w;
  return off;
}

hipError_t launch_select(const Dims& dm, float alpha, float gamma, int kmin_blocks, const uint16_t* q, const uint16_t* k,
                         const int8_t* pattern, const float* p_vert, const float* p_slash, int64_t* row_ptr,
                         int32_t* col_idx, uint8_t* sel_mask, const SelectWs& ws, hipStream_t st, int vs_rule,
                         int band, int pe_rows) {
  if (dm.d == 128)
    return select_impl<128>(dm, alpha, gamma, kmin_blocks, q, k, pattern, p_vert, p_slash, row_ptr, col_idx, sel_mask,
                            ws, st, vs_rule, band, pe_rows);
  return select_impl<64>(dm, alpha, gamma, kmin_blocks, q, k, pattern, p_vert, p_slash, row_ptr, col_idx, sel_mask, ws,
                         st, vs_rule, band, pe_rows);
}

}  // namespace crisp
