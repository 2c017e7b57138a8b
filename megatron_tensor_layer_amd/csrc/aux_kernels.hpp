// Bandwidth-bound kernels of the layer: causal scaled softmax (the scale is
// applied by the score GEMM), the softmax-backward row terms, bias-gradient
// column sums and the stand-in all-reduce. All reductions run in a fixed
// order (wavefront butterflies and fixed LDS trees), so results are
// bit-reproducible run to run.
#pragma once

#include "tp_common.hpp"

namespace tpl {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Causal softmax, one wavefront per row (paper-graph page, "Computation
// Optimizations": the causal mask is implicit inside the softmax reduction,
// no mask tensor is read). Row q of batch z reads S[z, q, 0..q] (fp32, already
// scaled by 1/sqrt(d)) and writes P[z, q, k] = exp(S - max) / sum for k <= q,
// zeros for q < k < min(s, roundup(q+1, pad)) so that every tile of P the
// causal GEMMs read is defined. Rows are held in registers: s <= 64*4*MAXC.
// ---------------------------------------------------------------------------
template <typename T, int MAXC>
__global__ void __launch_bounds__(256) causal_softmax_kernel(const float* __restrict__ S, T* __restrict__ P,
                                                             long rows, int s, int pad) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int q = (int)(row % s);
  const float* src = S + row * (long)s;
  T* dst = P + row * (long)s;
  const int n = q + 1;
  const int wend = min(s, ((q + pad) / pad) * pad);

  float x[MAXC][4];
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int k = (c * 64 + lane) * 4;
    if (k < n) {
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[c][e] = (k + e < n) ? v[e] : -INFINITY;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[c][e] = -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, x[c][e]);
  }
  mx = wave_max(mx);
  float sum = 0.0f;
  const float L2E = 1.4426950408889634f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ev = exp2f((x[c][e] - mx) * L2E);  // exp(-inf) = 0 for masked keys
      x[c][e] = ev;
      sum += ev;
    }
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int k = (c * 64 + lane) * 4;
    if (k < wend) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = x[c][e] * inv;
      Elt<T>::store4(dst + k, o);
    }
  }
}

// Rows longer than 64*4*MAXC: two passes over S (online max / sum, then write).
template <typename T>
__global__ void __launch_bounds__(256) causal_softmax_long_kernel(const float* __restrict__ S, T* __restrict__ P,
                                                                  long rows, int s, int pad) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int q = (int)(row % s);
  const float* src = S + row * (long)s;
  T* dst = P + row * (long)s;
  const int n = q + 1;
  const int wend = min(s, ((q + pad) / pad) * pad);
  const float L2E = 1.4426950408889634f;
  float mx = -INFINITY, sum = 0.0f;
  for (int k = lane; k < n; k += 64) {
    const float v = src[k];
    const float nm = fmaxf(mx, v);
    sum = sum * exp2f((mx - nm) * L2E) + exp2f((v - nm) * L2E);
    mx = nm;
  }
  // combine the lanes' (max, sum) pairs
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(mx, o, 64), os = __shfl_xor(sum, o, 64);
    const float nm = fmaxf(mx, om);
    const float a = (mx == -INFINITY) ? 0.0f : sum * exp2f((mx - nm) * L2E);
    const float b = (om == -INFINITY) ? 0.0f : os * exp2f((om - nm) * L2E);
    sum = a + b;
    mx = nm;
  }
  const float inv = 1.0f / sum;
  for (int k = lane; k < wend; k += 64) {
    const float pv = (k < n) ? exp2f((src[k] - mx) * L2E) * inv : 0.0f;
    Elt<T>::st(dst + k, pv);
  }
}

// ---------------------------------------------------------------------------
// D[z, q] = sum_c dC[q*b+beta, j*d+c] * C[q*b+beta, j*d+c],  z = beta*a_r + j.
// Equals rowsum(P * dP) of the softmax backward because C = P V.
// One thread per (token row, head).
// ---------------------------------------------------------------------------
// C is read in fp32 (the unrounded P V accumulator), so D matches the row
// sums of P * dP that the dS epilogue subtracts it from.
template <typename T>
__global__ void __launch_bounds__(256) rowdot_kernel(const T* __restrict__ dC, const float* __restrict__ C,
                                                     float* __restrict__ D, int Trows, int b, int ar, int d, int s) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)Trows * ar) return;
  const int row = (int)(idx / ar), j = (int)(idx - (idx / ar) * ar);
  const long ld = (long)ar * d;
  const T* x = dC + row * ld + (long)j * d;
  const float* y = C + row * ld + (long)j * d;
  float acc = 0.0f;
  for (int c = 0; c < d; c += 4) {
    float u[4], v[4];
    Elt<T>::load4(x + c, u);
    Elt<float>::load4(y + c, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += u[e] * v[e];
  }
  const int sigma = row / b, beta = row - (row / b) * b;
  D[((long)beta * ar + j) * s + sigma] = acc;
}

// ---------------------------------------------------------------------------
// out[n] = sum_r X[r, n]: bias gradients. Block = 8 column threads (16 bytes
// each) x 32 row groups; row groups are combined by a fixed LDS tree.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) colsum_kernel(const T* __restrict__ X, T* __restrict__ out, int R, int N, long ld) {
  constexpr int VEC = Elt<T>::VEC;
  const int ct = threadIdx.x & 7, rg = threadIdx.x >> 3;
  const int col = (blockIdx.x * 8 + ct) * VEC;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
  if (col < N) {
    for (int r = rg; r < R; r += 32) {
      const T* p = X + (long)r * ld + col;
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        float v[4];
        Elt<T>::load4(p + e, v);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[e + u] += v[u];
      }
    }
  }
  __shared__ float red[32][8 * VEC + 1];
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[rg][ct * VEC + e] = acc[e];
  __syncthreads();
  for (int w = 16; w > 0; w >>= 1) {
    if (rg < w) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) red[rg][ct * VEC + e] += red[rg + w][ct * VEC + e];
    }
    __syncthreads();
  }
  if (rg == 0 && col < N) {
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      float v[4] = {red[0][ct * VEC + e], red[0][ct * VEC + e + 1], red[0][ct * VEC + e + 2], red[0][ct * VEC + e + 3]};
      Elt<T>::store4(out + col + e, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Stand-in all-reduce followed by the fused bias + residual add:
//   out[r, c] = sum_k part[k, r, c] (rank order, fp32) + bias[c] + resid[r, c]
// bias and resid may be null. Rounded once to the output type.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) reduce_partials_kernel(const T* __restrict__ part, const T* __restrict__ bias,
                                                              const T* __restrict__ resid, T* __restrict__ out,
                                                              long rows, long cols, int t) {
  const long n = rows * cols;
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < t; ++r) {
    float v[4];
    Elt<T>::load4(part + (long)r * n + i, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  if (bias) {
    float v[4];
    Elt<T>::load4(bias + (i % cols), v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  if (resid) {
    float v[4];
    Elt<T>::load4(resid + i, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  Elt<T>::store4(out + i, acc);
}

}  // namespace tpl
