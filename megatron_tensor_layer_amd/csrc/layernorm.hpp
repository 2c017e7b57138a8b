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
// chunk) and both reductions over the row run on the registers. TPR threads
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

// Sum over the TPR threads of a row; every thread gets the same value.
template <int TPR>
__device__ __forceinline__ float row_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if constexpr (TPR == 64) {
    return v;
  } else {
    static_assert(TPR == 256, "a row takes one wave or the whole workgroup");
    __syncthreads();  // the previous reduction has read red
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
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

// One row per TPR threads; NC = most 16-byte chunks a thread holds.
template <typename T, int TPR, int NC>
__global__ void __launch_bounds__(256) ln_fwd_kernel(const LnFwdArgs a) {
  constexpr int VEC = Elt<T>::VEC, RPW = 256 / TPR;
  __shared__ float red[4];
  const long row = (long)blockIdx.x * RPW + threadIdx.x / TPR;
  const int lane = threadIdx.x % TPR;
  if (row >= a.rows) return;  // only with TPR = 64, whose reductions need no barrier
  const int nch = a.h / VEC;
  const long base = row * a.h;
  const T* x = static_cast<const T*>(a.x) + base;
  const T* rs = a.resid ? static_cast<const T*>(a.resid) + base : nullptr;
  const T* bs = static_cast<const T*>(a.bias);
  uint4 pv[NC];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * TPR;
    if (ch < nch) {
      float v[VEC];
      loadv<T, VEC>(x + ch * VEC, v);
      if (rs) {
        float r[VEC];
        loadv<T, VEC>(rs + ch * VEC, r);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] += r[e];
      }
      if (bs) {
        float b[VEC];
        loadv<T, VEC>(bs + ch * VEC, b);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] += b[e];
      }
      pv[c] = ln::pack<T>(v);  // rounded once: the normalised value is the stored one
      if (a.sum_out) *reinterpret_cast<uint4*>(static_cast<T*>(a.sum_out) + base + ch * VEC) = pv[c];
      ln::unpack<T>(pv[c], v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) s += v[e];
    }
  }
  if (!a.gamma) return;  // add only (uniform over the workgroup)
  const float inv_h = 1.0f / (float)a.h;
  const float mean = ln::row_sum<TPR>(s, red) * inv_h;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (lane + c * TPR < nch) {
      float v[VEC];
      ln::unpack<T>(pv[c], v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float dv = v[e] - mean;
        q += dv * dv;
      }
    }
  }
  const float var = ln::row_sum<TPR>(q, red) * inv_h;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  const T* gm = static_cast<const T*>(a.gamma);
  const T* bt = static_cast<const T*>(a.beta);
  T* y = static_cast<T*>(a.y) + base;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * TPR;
    if (ch < nch) {
      float v[VEC], g[VEC], b[VEC];
      ln::unpack<T>(pv[c], v);
      loadv<T, VEC>(gm + ch * VEC, g);
      loadv<T, VEC>(bt + ch * VEC, b);
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = (v[e] - mean) * rstd * g[e] + b[e];
      storev<T, VEC>(y + ch * VEC, v);
    }
  }
  if (lane == 0) {
    a.stats[2 * row] = mean;
    a.stats[2 * row + 1] = rstd;
  }
}

// dx of one row per TPR threads.
template <typename T, int TPR, int NC>
__global__ void __launch_bounds__(256) ln_bwd_dx_kernel(const LnBwdArgs a) {
  constexpr int VEC = Elt<T>::VEC, RPW = 256 / TPR;
  __shared__ float red[4];
  const long row = (long)blockIdx.x * RPW + threadIdx.x / TPR;
  const int lane = threadIdx.x % TPR;
  if (row >= a.rows) return;
  const int nch = a.h / VEC;
  const long base = row * a.h;
  const float mean = a.stats[2 * row], rstd = a.stats[2 * row + 1];
  const T* dy = static_cast<const T*>(a.dy) + base;
  const T* vv = static_cast<const T*>(a.v) + base;
  const T* gm = static_cast<const T*>(a.gamma);
  uint4 pd[NC], pv[NC];
  float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * TPR;
    if (ch < nch) {
      pd[c] = *reinterpret_cast<const uint4*>(dy + ch * VEC);
      pv[c] = *reinterpret_cast<const uint4*>(vv + ch * VEC);
      float d[VEC], v[VEC], g[VEC];
      ln::unpack<T>(pd[c], d);
      ln::unpack<T>(pv[c], v);
      loadv<T, VEC>(gm + ch * VEC, g);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float gg = d[e] * g[e];
        s1 += gg;
        s2 += gg * ((v[e] - mean) * rstd);
      }
    }
  }
  const float inv_h = 1.0f / (float)a.h;
  const float m1 = ln::row_sum<TPR>(s1, red) * inv_h;
  const float m2 = ln::row_sum<TPR>(s2, red) * inv_h;
  const T* dr = a.dresid ? static_cast<const T*>(a.dresid) + base : nullptr;
  T* dx = static_cast<T*>(a.dx) + base;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * TPR;
    if (ch < nch) {
      float d[VEC], v[VEC], g[VEC], o[VEC];
      ln::unpack<T>(pd[c], d);
      ln::unpack<T>(pv[c], v);
      loadv<T, VEC>(gm + ch * VEC, g);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float xh = (v[e] - mean) * rstd;
        o[e] = rstd * (d[e] * g[e] - m1 - xh * m2);
      }
      if (dr) {
        float r[VEC];
        loadv<T, VEC>(dr + ch * VEC, r);
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
    const T* dy = static_cast<const T*>(a.dy) + col;
    const T* vv = static_cast<const T*>(a.v) + col;
    for (long r = rg; r < a.rows; r += RG) {
      float d[VEC], v[VEC];
      loadv<T, VEC>(dy + r * a.h, d);
      loadv<T, VEC>(vv + r * a.h, v);
      const float2 st = *reinterpret_cast<const float2*>(a.stats + 2 * r);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        ag[e] += d[e] * ((v[e] - st.x) * st.y);
        ab[e] += d[e];
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
