// The FlexPrefill baseline path on gfx950: the JSD router and the gamma-cumsum
// VS budget rule that CRISP replaces (PEIndex and the attention are shared).
//
// Method: digest page "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
// Structural-Mass-Motivated Routing", the prerequisite sections on
// Jensen-Shannon divergence and on the cumulative-coverage (gamma) threshold.
//
// Router: a_hat is the proxy's block-pooled distribution (p_vert of
// crisp_route); a_bar is the softmax over key blocks of the mean of the last
// 128 queries against each block's mean key, scaled by 1/sqrt(d).  The head is
// VS iff D_JS(a_hat, a_bar) >= tau (natural log).  VS budget: per direction,
// the shortest prefix of the scores sorted descending (ties to the lower
// index) whose sum reaches gamma, clipped to [k_min, N_b], plus the anchor
// blocks 0 and N_b-1 — the format crisp_select's VS flags use.
#include <math.h>

#include "crisp_device.hpp"
#include "crisp_internal.h"

namespace crisp {

namespace {

constexpr int MAX_NB = 8192;   // n <= 1,048,576 tokens

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  const double t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

__device__ __forceinline__ float block_max_f32(float v, float* red) {
  v = wave_max(v);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  const float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}

// kbar[bg][kb][:] = mean of the 128 key rows of block kb (every KV group).
template <int D>
__global__ __launch_bounds__(NTHR) void flex_pool_k_kernel(const uint16_t* __restrict__ k, float* __restrict__ kbar,
                                                           int n) {
  __shared__ float part[NTHR];
  const int kb = blockIdx.x;
  const int64_t bg = blockIdx.y;
  const int nb = n / BLK;
  constexpr int SPLIT = NTHR / D;   // row groups per dimension
  const int dim = threadIdx.x % D, grp = threadIdx.x / D;
  const uint16_t* src = k + ((size_t)bg * n + (size_t)kb * BLK) * D + dim;
  // rows grp, grp + SPLIT, ... in that order; sixteen loads in flight per thread
  constexpr int PER = BLK / SPLIT, U = 16;
  static_assert(PER % U == 0, "row batches");
  float s = 0.f;
  for (int j0 = 0; j0 < PER; j0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = bf16_to_f32(src[(size_t)(grp + SPLIT * (j0 + u)) * D]);
#pragma unroll
    for (int u = 0; u < U; ++u) s += v[u];
  }
  part[threadIdx.x] = s;
  __syncthreads();
  if (grp == 0) {
    float t = part[dim];
    for (int g2 = 1; g2 < SPLIT; ++g2) t += part[g2 * D + dim];
    kbar[((size_t)bg * nb + kb) * D + dim] = t * (1.f / BLK);
  }
}

// One workgroup per (batch, query head): a_bar, D_JS(p_vert, a_bar), the route.
template <int D>
__global__ __launch_bounds__(NTHR) void flex_route_kernel(const uint16_t* __restrict__ q, const float* __restrict__ kbar,
                                                          const float* __restrict__ p_vert, float* __restrict__ jsd,
                                                          int8_t* __restrict__ pattern, int n, int h_q, int group,
                                                          float tau, float scale) {
  __shared__ float qh[D];
  __shared__ float part[NTHR];
  __shared__ float ab[MAX_NB];
  __shared__ float fred[4];
  __shared__ double dred[4];
  const int64_t bh = blockIdx.x;
  const int nb = n / BLK;
  const int h_kv = h_q / group;
  const int b = (int)(bh / h_q), h = (int)(bh % h_q);
  const int64_t bg = (int64_t)b * h_kv + h / group;
  const int tid = threadIdx.x;
  // mean of the last 128 query rows
  {
    constexpr int SPLIT = NTHR / D;
    const int dim = tid % D, grp = tid / D;
    const uint16_t* src = q + ((size_t)bh * n + (size_t)(n - BLK)) * D + dim;
    float s = 0.f;
    for (int r = grp; r < BLK; r += SPLIT) s += bf16_to_f32(src[(size_t)r * D]);
    part[tid] = s;
    __syncthreads();
    if (grp == 0) {
      float t = part[dim];
      for (int g2 = 1; g2 < SPLIT; ++g2) t += part[g2 * D + dim];
      qh[dim] = t * (1.f / BLK);
    }
    __syncthreads();
  }
  // pooled logits and their softmax over all key blocks
  const float* kg = kbar + (size_t)bg * nb * D;
  float mx = -INFINITY;
  for (int j = tid; j < nb; j += NTHR) {
    const float* kr = kg + (size_t)j * D;
    float s = 0.f;
#pragma unroll 8
    for (int c = 0; c < D; ++c) s = fmaf(qh[c], kr[c], s);
    s *= scale;
    ab[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = block_max_f32(mx, fred);
  double sum = 0.0;
  for (int j = tid; j < nb; j += NTHR) {
    const float e = expf(ab[j] - mx);
    ab[j] = e;
    sum += (double)e;
  }
  sum = block_sum_f64(sum, dred);
  const double inv = 1.0 / sum;
  // D_JS = 1/2 sum p log(p/m) + 1/2 sum a log(a/m), m = (p + a)/2; zero terms vanish
  const float* p = p_vert + (size_t)bh * nb;
  double acc = 0.0;
  for (int j = tid; j < nb; j += NTHR) {
    const double pj = (double)p[j], aj = (double)ab[j] * inv;
    const double m = 0.5 * (pj + aj);
    if (pj > 0.0) acc += 0.5 * pj * log(pj / m);
    if (aj > 0.0) acc += 0.5 * aj * log(aj / m);
  }
  acc = block_sum_f64(acc, dred);
  if (tid == 0) {
    jsd[bh] = (float)acc;
    pattern[bh] = acc >= (double)tau ? 1 : 0;
  }
}

// Bitonic sort of np (a power of two) (score, index) pairs in LDS into score
// descending, index ascending order; every thread of the workgroup calls it.
__device__ __forceinline__ void sort_desc(float* sv, int* si, int np) {
  const int tid = threadIdx.x;
  for (int kk = 2; kk <= np; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < np; i += NTHR) {
        const int l = i ^ jj;
        if (l > i) {
          const float a = sv[i], c = sv[l];
          const int ia = si[i], ic = si[l];
          const bool l_first = c > a || (c == a && ic < ia);   // element l belongs before element i
          const bool up = (i & kk) == 0;
          if (up ? l_first : !l_first) {
            sv[i] = c;
            sv[l] = a;
            si[i] = ic;
            si[l] = ia;
          }
        }
      }
      __syncthreads();
    }
  }
}

// One workgroup per (batch, query head): VS flags of both directions by the
// noise floor with mu = the median of the N_b - 2 non-anchor scores (the
// variant of the digest's Table 9): keep p > alpha mu, at least k_min blocks
// (top-k, ties to the lower index), plus the anchors (PE heads: all zero).
__global__ __launch_bounds__(NTHR) void median_vs_kernel(const int8_t* __restrict__ pattern,
                                                         const float* __restrict__ p_vert,
                                                         const float* __restrict__ p_slash,
                                                         uint8_t* __restrict__ vsflags, uint8_t* __restrict__ sel_mask,
                                                         int nb, float alpha, int kmin) {
  __shared__ float sv[MAX_NB];
  __shared__ int si[MAX_NB];
  __shared__ uint8_t fl[MAX_NB];
  __shared__ float thr_s;
  __shared__ int cnt_s;
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const bool vs = pattern[bh] == 1;
  int np = 1;
  while (np < nb) np <<= 1;
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
    for (int j = tid; j < np; j += NTHR) {
      sv[j] = j < nb ? p[j] : -INFINITY;
      si[j] = j < nb ? j : 0x7fffffff;
    }
    for (int j = tid; j < nb; j += NTHR) fl[j] = 0;
    if (tid == 0) cnt_s = 0;
    __syncthreads();
    sort_desc(sv, si, np);
    if (tid == 0) {
      // ranks (m-1)/2 and m/2 among the non-anchor blocks, m = nb - 2, in sorted order
      const int m = nb - 2, lo = (m - 1) / 2, hi = m / 2;
      float vlo = 0.f, vhi = 0.f;
      int seen = 0;
      for (int t = 0; t < nb && seen <= hi; ++t) {
        const int j = si[t];
        if (j == 0 || j == nb - 1) continue;
        if (seen == lo) vlo = sv[t];
        if (seen == hi) vhi = sv[t];
        ++seen;
      }
      const float mu = lo == hi ? vlo : 0.5f * (vlo + vhi);
      thr_s = alpha * mu;
    }
    __syncthreads();
    const float thr = thr_s;
    int c = 0;
    for (int j = tid; j < nb; j += NTHR) c += p[j] > thr ? 1 : 0;
    atomicAdd(&cnt_s, c);
    __syncthreads();
    int take = cnt_s > kmin ? cnt_s : kmin;
    if (take > nb) take = nb;
    for (int t = tid; t < take; t += NTHR)
      if (si[t] < nb) fl[si[t]] = 1;
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

// One workgroup per (batch, query head): VS flags of both directions by the
// gamma-cumsum rule (PE heads: all zero).
__global__ __launch_bounds__(NTHR) void flex_vs_kernel(const int8_t* __restrict__ pattern,
                                                       const float* __restrict__ p_vert,
                                                       const float* __restrict__ p_slash, uint8_t* __restrict__ vsflags,
                                                       uint8_t* __restrict__ sel_mask, int nb, double gamma, int kmin) {
  __shared__ float sv[MAX_NB];
  __shared__ int si[MAX_NB];
  __shared__ double csum[NTHR];
  __shared__ uint8_t fl[MAX_NB];
  __shared__ int cut;
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const bool vs = pattern[bh] == 1;
  int np = 1;
  while (np < nb) np <<= 1;
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
    for (int j = tid; j < np; j += NTHR) {
      sv[j] = j < nb ? p[j] : -INFINITY;
      si[j] = j < nb ? j : 0x7fffffff;
    }
    for (int j = tid; j < nb; j += NTHR) fl[j] = 0;
    if (tid == 0) cut = nb;
    __syncthreads();
    sort_desc(sv, si, np);
    // inclusive prefix sums in fp64 over the sorted scores: the first position reaching gamma
    const int per = (np + NTHR - 1) / NTHR;
    const int lo = tid * per, hi = lo + per < nb ? lo + per : nb;
    double s = 0.0;
    for (int t = lo; t < hi; ++t) s += (double)sv[t];
    csum[tid] = s;
    __syncthreads();
    if (tid == 0) {
      double run = 0.0;
      for (int t = 0; t < NTHR; ++t) {
        const double c = csum[t];
        csum[t] = run;   // exclusive prefix of the chunks
        run += c;
      }
    }
    __syncthreads();
    {
      double run = csum[tid];
      for (int t = lo; t < hi; ++t) {
        run += (double)sv[t];
        if (run >= gamma) {
          atomicMin(&cut, t + 1);
          break;
        }
      }
    }
    __syncthreads();
    int take = cut > kmin ? cut : kmin;
    if (take > nb) take = nb;
    for (int t = tid; t < take; t += NTHR)
      if (si[t] < nb) fl[si[t]] = 1;   // (a NaN score could let padding sort early)
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

}  // namespace

size_t flex_route_ws_bytes(const Dims& dm) { return (size_t)dm.batch * dm.h_kv * dm.nb * dm.d * sizeof(float); }

hipError_t launch_flex_route(const Dims& dm, float tau, const uint16_t* q, const uint16_t* k, const float* p_vert,
                             float* jsd, int8_t* pattern, float* kbar, hipStream_t st) {
  const float scale = 1.f / sqrtf((float)dm.d);
  const dim3 pg((unsigned)dm.nb, (unsigned)(dm.batch * dm.h_kv));
  if (dm.d == 128) {
    flex_pool_k_kernel<128><<<pg, NTHR, 0, st>>>(k, kbar, dm.n);
    flex_route_kernel<128><<<(unsigned)dm.bh, NTHR, 0, st>>>(q, kbar, p_vert, jsd, pattern, dm.n, dm.h_q, dm.group,
                                                            tau, scale);
  } else {
    flex_pool_k_kernel<64><<<pg, NTHR, 0, st>>>(k, kbar, dm.n);
    flex_route_kernel<64><<<(unsigned)dm.bh, NTHR, 0, st>>>(q, kbar, p_vert, jsd, pattern, dm.n, dm.h_q, dm.group,
                                                           tau, scale);
  }
  return hipGetLastError();
}

hipError_t launch_median_vs(const Dims& dm, float alpha, int kmin_blocks, const int8_t* pattern, const float* p_vert,
                            const float* p_slash, uint8_t* vsflags, uint8_t* sel_mask, hipStream_t st) {
  median_vs_kernel<<<(unsigned)dm.bh, NTHR, 0, st>>>(pattern, p_vert, p_slash, vsflags, sel_mask, dm.nb, alpha,
                                                     kmin_blocks);
  return hipGetLastError();
}

hipError_t launch_flex_vs(const Dims& dm, float gamma, int kmin_blocks, const int8_t* pattern, const float* p_vert,
                          const float* p_slash, uint8_t* vsflags, uint8_t* sel_mask, hipStream_t st) {
  flex_vs_kernel<<<(unsigned)dm.bh, NTHR, 0, st>>>(pattern, p_vert, p_slash, vsflags, sel_mask, dm.nb, (double)gamma,
                                                   kmin_blocks);
  return hipGetLastError();
}

}  // namespace crisp
