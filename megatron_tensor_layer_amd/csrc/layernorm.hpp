// LayerNorm of token rows for the sequence-parallel region of the layer
// ("parallelism" blog post, "Sequence parallelism: the parts TP leaves
// behind": LayerNorm, the bias after the row-parallel product and the residual
// add run on each rank's own slice of the sequence), fused with the bias +
// residual add that precedes it, and its backward.
//
//   forward:  v = x + residual + bias (rounded to the storage type: the value
//             the backward reads back); mean and biased variance of v over the
//             row's h features; y = (v - mean) rstd gamma + beta,
//             rstd = 1 / sqrt(var + eps)
//   backward: x_hat = (v - mean) rstd, g = dy gamma,
//             dx = rstd (g - mean(g) - x_hat mean(g x_hat)) + dresid,
//             dgamma = sum over rows of dy x_hat, dbeta = sum over rows of dy
//
// Bandwidth-bound: each row is read once into registers (packed, 16 bytes a
// chunk) and the reductions over the row run on the registers. TPR threads
// share a row: one wave for rows of up to 512 chunks (h <= 4096 in bf16), else
// the whole 256-thread workgroup. Reductions are fixed trees (wave butterfly,
// then the four waves in order), so results do not depend on timing.
#pragma once

#include "tp_common.hpp"

namespace tpl {

struct LnFwdArgs {
  const void *x, *bias, *resid, *gamma, *beta;
  void *sum_out, *y;
  float* stats;  // [rows, 2]: mean, rstd
  long rows;
  int h;
  float eps;
};

struct LnBwdArgs {
  const void *dy, *v, *gamma, *dresid;
  const float* stats;
  void *dx, *dgamma, *dbeta;
  long rows;
  int h;
};

namespace ln {

// Sums of two values over the TPR threads of a row; every thread gets the
// same pair (a butterfly adds the same two partials on both partners).
template <int TPR>
__device__ __forceinline__ float2 row_sum2(float2 v, float2* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    v.x += __shfl_xor(v.x, o, 64);
    v.y += __shfl_xor(v.y, o, 64);
  }
  if constexpr (TPR == 64) {
    return v;
  } else {
    static_assert(TPR == 256, "a row takes one wave or the whole workgroup");
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return make_float2((red[0].x + red[1].x) + (red[2].x + red[3].x), (red[0].y + red[1].y) + (red[2].y + red[3].y));
  }
}

// Count, mean and sum of squared deviations of each thread's values,
// combined over the row's TPR threads by the pairwise update of Chan, Golub
// and LeVeque (n = na + nb, mean = (na ma + nb mb) / n,
// M2 = M2a + M2b + (mb - ma)^2 na nb / n), written symmetrically in the two
// partners so that every thread ends with bit-identical moments. One
// reduction round: the variance needs no second pass over the row.
__device__ __forceinline__ void chan_merge(float& n, float& m, float& q, float nb, float mb, float qb) {
  const float nn = n + nb;
  if (nn > 0.0f) {
    const float d = mb - m;
    const float mm = (n * m + nb * mb) / nn;
    q = (q + qb) + d * d * (n * nb / nn);
    m = mm;
  }
  n = nn;
}

template <int TPR>
__device__ __forceinline__ void row_moments(float& n, float& m, float& q, float4* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float nb = __shfl_xor(n, o, 64), mb = __shfl_xor(m, o, 64), qb = __shfl_xor(q, o, 64);
    chan_merge(n, m, q, nb, mb, qb);
  }
  if constexpr (TPR == 256) {
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float4(n, m, q, 0.0f);
    __syncthreads();
    float n0 = red[0].x, m0 = red[0].y, q0 = red[0].z;
    float n2 = red[2].x, m2 = red[2].y, q2 = red[2].z;
    chan_merge(n0, m0, q0, red[1].x, red[1].y, red[1].z);
    chan_merge(n2, m2, q2, red[3].x, red[3].y, red[3].z);
    chan_merge(n0, m0, q0, n2, m2, q2);
    n = n0; m = m0; q = q0;
  }
}

template <typename T>
__device__ __forceinline__ void unpack(const uint4& u, float f[Elt<T>::VEC]) {
  loadv<T, Elt<T>::VEC>(reinterpret_cast<const T*>(&u), f);
}

template <typename T>
__device__ __forceinline__ uint4 pack(const float f[Elt<T>::VEC]) {
  uint4 u;
  storev<T, Elt<T>::VEC>(reinterpret_cast<T*>(&u), f);
  return u;
}

}  // namespace ln

// One row per TPR threads; NC = most 16-byte chunks a thread holds. Every
// load of the row (and of bias, gamma, beta) is issued before the first
// reduction, so the row costs one memory round trip and one barrier round.
template <typename T, int TPR, int NC>
__global__ void __launch_bounds__(256) ln_fwd_kernel(const LnFwdArgs a) {
  constexpr int VEC = Elt<T>::VEC, RPW = 256 / TPR;
  __shared__ float4 red[4];
  const long row = (long)blockIdx.x * RPW + threadIdx.x / TPR;
  const int lane = threadIdx.x % TPR;
  if (row >= a.rows) return;  // only with TPR = 64, whose reductions need no barrier
  const int nch = a.h / VEC;
  const long base = row * a.h;
  const T* x = static_cast<const T*>(a.x) + base;
  const T* rs = a.resid ? static_cast<const T*>(a.resid) + base : nullptr;
  const T* bs = static_cast<const T*>(a.bias);
  const T* gm = static_cast<const T*>(a.gamma);
  const T* bt = static_cast<const T*>(a.beta);
  uint4 pv[NC], pr[NC], pb[NC], pg[NC], pt[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * TPR;
    if (ch < nch) {
      pv[c] = *reinterpret_cast<const uint4*>(x + ch * VEC);
      if (rs) pr[c] = *reinterpret_cast<const uint4*>(rs + ch * VEC);
      if (bs) pb[c] = *reinterpret_cast<const uint4*>(bs + ch * VEC);
      if (gm) {
        pg[c] = *reinterpret_cast<const uint4*>(gm + ch * VEC);
        pt[c] = *reinterpret_cast<const uint4*>(bt + ch * VEC);
      }
    }
  }
  float cnt = 0.0f, s = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * TPR;
    if (ch < nch) {
      float v[VEC];
      ln::unpack<T>(pv[c], v);
      if (rs) {
        float r[VEC];
        ln::unpack<T>(pr[c], r);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] += r[e];
      }
      if (bs) {
        float b[VEC];
        ln::unpack<T>(pb[c], b);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] += b[e];
      }
      pv[c] = ln::pack<T>(v);  // rounded once: the normalised value is the stored one
      if (a.sum_out) *reinterpret_cast<uint4*>(static_cast<T*>(a.sum_out) + base + ch * VEC) = pv[c];
      ln::unpack<T>(pv[c], v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) s += v[e];
      cnt += (float)VEC;
    }
  }
  if (!gm) return;  // add only (uniform over the workgroup)
  // this thread's mean and squared deviations, then the row's
  float m = cnt > 0.0f ? s / cnt : 0.0f, q = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (lane + c * TPR < nch) {
      float v[VEC];
      ln::unpack<T>(pv[c], v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float dv = v[e] - m;
        q += dv * dv;
      }
    }
  }
  ln::row_moments<TPR>(cnt, m, q, red);
  const float mean = m, rstd = 1.0f / sqrtf(q / (float)a.h + a.eps);
  T* y = static_cast<T*>(a.y) + base;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * TPR;
    if (ch < nch) {
      float v[VEC], g[VEC], b[VEC];
      ln::unpack<T>(pv[c], v);
      ln::unpack<T>(pg[c], g);
      ln::unpack<T>(pt[c], b);
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = (v[e] - mean) * rstd * g[e] + b[e];
      storev<T, VEC>(y + ch * VEC, v);
    }
  }
  if (lane == 0) *reinterpret_cast<float2*>(a.stats + 2 * row) = make_float2(mean, rstd);
}

// dx of one row per TPR threads: all loads first, one barrier round for
// the two row sums.
template <typename T, int TPR, int NC>
__global__ void __launch_bounds__(256) ln_bwd_dx_kernel(const LnBwdArgs a) {
  constexpr int VEC = Elt<T>::VEC, RPW = 256 / TPR;
  __shared__ float2 red[4];
  const long row = (long)blockIdx.x * RPW + threadIdx.x / TPR;
  const int lane = threadIdx.x % TPR;
  if (row >= a.rows) return;
  const int nch = a.h / VEC;
  const long base = row * a.h;
  const float2 st = *reinterpret_cast<const float2*>(a.stats + 2 * row);
  const float mean = st.x, rstd = st.y;
  const T* dy = static_cast<const T*>(a.dy) + base;
  const T* vv = static_cast<const T*>(a.v) + base;
  const T* gm = static_cast<const T*>(a.gamma);
  const T* dr = a.dresid ? static_cast<const T*>(a.dresid) + base : nullptr;
  uint4 pd[NC], pv[NC], pg[NC], pr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * TPR;
    if (ch < nch) {
      pd[c] = *reinterpret_cast<const uint4*>(dy + ch * VEC);
      pv[c] = *reinterpret_cast<const uint4*>(vv + ch * VEC);
      pg[c] = *reinterpret_cast<const uint4*>(gm + ch * VEC);
      if (dr) pr[c] = *reinterpret_cast<const uint4*>(dr + ch * VEC);
    }
  }
  float2 sum = make_float2(0.0f, 0.0f);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (lane + c * TPR < nch) {
      float d[VEC], v[VEC], g[VEC];
      ln::unpack<T>(pd[c], d);
      ln::unpack<T>(pv[c], v);
      ln::unpack<T>(pg[c], g);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float gg = d[e] * g[e];
        sum.x += gg;
        sum.y += gg * ((v[e] - mean) * rstd);
      }
    }
  }
  const float2 tot = ln::row_sum2<TPR>(sum, red);
  const float inv_h = 1.0f / (float)a.h;
  const float m1 = tot.x * inv_h, m2 = tot.y * inv_h;
  T* dx = static_cast<T*>(a.dx) + base;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * TPR;
    if (ch < nch) {
      float d[VEC], v[VEC], g[VEC], o[VEC];
      ln::unpack<T>(pd[c], d);
      ln::unpack<T>(pv[c], v);
      ln::unpack<T>(pg[c], g);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float xh = (v[e] - mean) * rstd;
        o[e] = rstd * (d[e] * g[e] - m1 - xh * m2);
      }
      if (dr) {
        float r[VEC];
        ln::unpack<T>(pr[c], r);
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] += r[e];
      }
      storev<T, VEC>(dx + ch * VEC, o);
    }
  }
}

// dgamma and dbeta: column sums over the rows, CT threads across VEC columns
// each, RG row groups, then a fixed tree over the row groups in LDS.
template <typename T>
__global__ void __launch_bounds__(256) ln_bwd_dparam_kernel(const LnBwdArgs a) {
  constexpr int VEC = Elt<T>::VEC, CT = 8, RG = 256 / CT, W = CT * VEC;
  const int ct = threadIdx.x % CT, rg = threadIdx.x / CT;
  const int col = (blockIdx.x * CT + ct) * VEC;
  float ag[VEC], ab[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) ag[e] = ab[e] = 0.0f;
  if (col < a.h) {
    constexpr int U = 8;  // rows in flight per thread
    const T* dy = static_cast<const T*>(a.dy) + col;
    const T* vv = static_cast<const T*>(a.v) + col;
    for (long r0 = rg; r0 < a.rows; r0 += (long)U * RG) {
      uint4 pd[U], pv[U];
      float2 st[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const long r = r0 + (long)u * RG;
        if (r < a.rows) {
          pd[u] = *reinterpret_cast<const uint4*>(dy + r * a.h);
          pv[u] = *reinterpret_cast<const uint4*>(vv + r * a.h);
          st[u] = *reinterpret_cast<const float2*>(a.stats + 2 * r);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (r0 + (long)u * RG < a.rows) {
          float d[VEC], v[VEC];
          ln::unpack<T>(pd[u], d);
          ln::unpack<T>(pv[u], v);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            ag[e] += d[e] * ((v[e] - st[u].x) * st[u].y);
            ab[e] += d[e];
          }
        }
      }
    }
  }
  __shared__ float red[RG][2 * W + 1];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    red[rg][ct * VEC + e] = ag[e];
    red[rg][W + ct * VEC + e] = ab[e];
  }
  __syncthreads();
  for (int k = RG / 2; k >= 1; k /= 2) {
    for (int i = threadIdx.x; i < k * 2 * W; i += 256) red[i / (2 * W)][i % (2 * W)] += red[i / (2 * W) + k][i % (2 * W)];
    __syncthreads();
  }
  if (threadIdx.x < 2 * W) {
    const int j = threadIdx.x % W, c = blockIdx.x * W + j;
    if (c < a.h) Elt<T>::st(static_cast<T*>(threadIdx.x < W ? a.dgamma : a.dbeta) + c, red[0][threadIdx.x]);
  }
}

}  // namespace tpl
