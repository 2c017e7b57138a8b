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
// Equals rowsum(P * dP) of the softmax backward because C = P V. C is read in
// fp32 (the unrounded P V accumulator), so D matches the row sums of P * dP
// that the dS epilogue subtracts it from.
// One block per token row: the threads form the products of 4-element chunks
// of the row (coalesced), park the chunk sums in LDS, and thread j then adds
// head j's chunks in order. Heads are taken ROWDOT_LDS * 4 / d at a time.
// ---------------------------------------------------------------------------
constexpr int ROWDOT_LDS = 4096;  // chunk sums per pass
template <typename T>
__global__ void __launch_bounds__(256) rowdot_kernel(const T* __restrict__ dC, const float* __restrict__ C,
                                                     float* __restrict__ D, int b, int ar, int d, int s) {
  __shared__ float part[ROWDOT_LDS];
  const int row = blockIdx.x;
  const long ld = (long)ar * d;
  const T* x = dC + row * ld;
  const float* y = C + row * ld;
  const int cpd = d / 4;                     // chunks per head
  const int hpp = ROWDOT_LDS / cpd;          // heads per pass
  const int sigma = row / b, beta = row - (row / b) * b;
  for (int h0 = 0; h0 < ar; h0 += hpp) {
    const int nh = min(hpp, ar - h0);
    const int nc = nh * cpd;
    for (int c = threadIdx.x; c < nc; c += 256) {
      float u[4], v[4];
      Elt<T>::load4(x + (long)h0 * d + 4 * c, u);
      Elt<float>::load4(y + (long)h0 * d + 4 * c, v);
      part[c] = (u[0] * v[0] + u[1] * v[1]) + (u[2] * v[2] + u[3] * v[3]);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nh; j += 256) {
      float acc = 0.0f;
      for (int c = 0; c < cpd; ++c) acc += part[j * cpd + c];
      D[((long)beta * ar + h0 + j) * s + sigma] = acc;
    }
    __syncthreads();
  }
}

// rowdot_kernel fused with the fixed-order split-K sum that produces dC (the
// output projection's input gradient, split along K): per token row, each
// 4-element chunk is the sum of the splits' fp32 partials (split order),
// stored as bf16 dC, and the rounded values enter the same chunk products and
// per-head sums as in rowdot_kernel, so D is bitwise the unfused result.
// part: splits planes of T x (ar d) fp32; dC row pitch ar d.
__global__ void __launch_bounds__(256) splitk_rowdot_kernel(const float* __restrict__ part, int splits,
                                                            bf16_t* __restrict__ dC, const float* __restrict__ C,
                                                            float* __restrict__ D, int T, int b, int ar, int d,
                                                            int s) {
  __shared__ float red[ROWDOT_LDS];
  const int row = blockIdx.x;
  const long ld = (long)ar * d;
  const int cpd = d / 4;
  const int hpp = ROWDOT_LDS / cpd;
  const int sigma = row / b, beta = row - (row / b) * b;
  for (int h0 = 0; h0 < ar; h0 += hpp) {
    const int nh = min(hpp, ar - h0);
    const int nc = nh * cpd;
    for (int c = threadIdx.x; c < nc; c += 256) {
      const long off = (long)row * ld + (long)h0 * d + 4 * c;
      float u[4] = {0.f, 0.f, 0.f, 0.f}, v[4];
      // pieces in order, two loads in flight per step
      int k = 0;
      for (; k + 2 <= splits; k += 2) {
        float x[4], y[4];
        Elt<float>::load4(part + (long)k * T * ld + off, x);
        Elt<float>::load4(part + (long)(k + 1) * T * ld + off, y);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = (u[e] + x[e]) + y[e];
      }
      if (k < splits) {
        float x[4];
        Elt<float>::load4(part + (long)k * T * ld + off, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] += x[e];
      }
      Elt<bf16_t>::store4(dC + off, u);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = bf2f(f2bf(u[e]));
      Elt<float>::load4(C + off, v);
      red[c] = (u[0] * v[0] + u[1] * v[1]) + (u[2] * v[2] + u[3] * v[3]);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nh; j += 256) {
      float acc = 0.0f;
      for (int c = 0; c < cpd; ++c) acc += red[j * cpd + c];
      D[((long)beta * ar + h0 + j) * s + sigma] = acc;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// out[n] = sum_r X[r, n]: bias gradients in one fixed-order pass. A block owns
// 8 x VEC columns (8 column threads of 16 bytes: a 128-byte row piece) over all
// R rows. Its NT/8 row groups each sum rows rg, rg + NT/8, ... with 16 loads in
// flight per thread (64 KB per 256-thread block, enough to cover HBM latency
// with one block per CU), then a fixed LDS tree adds the groups and the result
// is rounded once.
// ---------------------------------------------------------------------------
template <typename T, int NT>
__global__ void __launch_bounds__(NT) colsum_kernel(const T* __restrict__ X, T* __restrict__ out, int R, int N,
                                                    long ld) {
  constexpr int VEC = Elt<T>::VEC, CT = 8, RG = NT / CT, W = CT * VEC, U = 16;
  const int ct = threadIdx.x % CT, rg = threadIdx.x / CT;
  const int col = (blockIdx.x * CT + ct) * VEC;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
  if (col < N) {
    int r = rg;
    for (; r + (U - 1) * RG < R; r += U * RG) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const uint4*>(X + (long)(r + RG * u) * ld + col);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float f[VEC];
        Elt<T>::load4(reinterpret_cast<const T*>(&v[u]), f);
        if constexpr (VEC == 8) Elt<T>::load4(reinterpret_cast<const T*>(&v[u]) + 4, f + 4);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += f[e];
      }
    }
    for (; r < R; r += RG) {
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
  __shared__ float red[RG][W + 1];
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[rg][ct * VEC + e] = acc[e];
  __syncthreads();
  for (int h = RG / 2; h >= 1; h /= 2) {  // fixed tree over the row groups
    for (int i = threadIdx.x; i < h * W; i += NT) red[i / W][i % W] += red[i / W + h][i % W];
    __syncthreads();
  }
  if (threadIdx.x < W) {
    const int c = blockIdx.x * W + threadIdx.x;
    if (c < N) Elt<T>::st(out + c, red[0][threadIdx.x]);
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
