// Flash-style causal self-attention of one rank's heads on gfx950 (bf16 MFMA,
// fp32 softmax), forward and backward, without materialising any s x s
// matrix.
//
// The method is the attention block of the "parallelism" blog ("Tensor
// parallelism: split every matrix", "Attention") with the causal mask of its
// "Context parallelism" section, evaluated with the running-max softmax of
// "How the softmax stays exact: the online softmax": each query keeps a
// running maximum m and running sum l of exponentials; when a new block of
// keys raises the maximum, the partial sum and the partial context are
// rescaled by exp(m_old - m_new), so the final result equals the plain
// softmax exactly (up to rounding).
//
// Per (sequence beta, head j) pair z:  S = Q K^T / sqrt(d),  P = softmax(S)
// over keys k <= query i,  C = P V.  Backward, with D_i = sum_k P_ik dP_ik =
// dC_i . C_i:  dP = dC V^T,  dS = P (dP - D) / sqrt(d),  dV = P^T dC,
// dQ = dS K,  dK = dS^T Q.
//
// Scores: S = Qh Kh^T + Qh Kl^T + Ql Kh^T, where Qh, Kh are the bf16 Q, K and
// Ql, Kl their bf16 rounding residuals (written by the QKV GEMM epilogue):
// three MFMA passes keep about 16 mantissa bits of the logits, which the
// peaked softmax rows of wide layers need.
//
// Kernels (64-lane waves of 32 query or key rows each):
//   fa_fwd8_kernel   : 256 queries, 8 waves (d <= 128): keys in tiles of 64
//                      staged in LDS (Kh, Kl, V; double buffered, 96 KB at
//                      d = 128); two waves share each SIMD, so one wave's
//                      softmax arithmetic and waits overlap the other's MFMAs;
//                      writes C (bf16 and fp32) and the log2-domain
//                      log-sum-exp. fa_fwd_kernel: the same with 4 waves and
//                      128 queries, for d = 160 (more live state per wave).
//   fa_bwd_dkv_kernel: 128 keys (32 per wave); queries in tiles of 64 (Qh,
//                      Ql, dC + LSE and D); accumulates dK, dV.
//   fa_bwd_dq_kernel : 128 queries; keys in tiles of 64; dQ (fa_bwd_dq2_kernel:
//                      single-buffered, two workgroups per CU, Q's low part
//                      kept in LDS rather than registers).
// dQ has its own kernel (recomputing P and dP) so that every gradient is a
// fixed-order sum: no atomics, bitwise reproducible.
//
// Work items. Causality makes the tile ranges of the blocks very unequal
// (the last query block sees s / 64 key tiles, the first two), and a few
// heads per rank give only a couple of hundred blocks, so each range is cut
// into chunks of at most ct tiles, one workgroup each; blocks with several
// chunks leave fp32 partials that a combine kernel merges in chunk order.
// The (head, item) list is dealt to the 8 XCDs in contiguous runs, so the
// workgroups of one head share its K, V (or Q, dC) in one L2.
//
// Register layouts. The MFMA is issued with the "column" operand first
// (mma16(bfrag, afrag, acc)), so a 32x32 accumulator gives lane l the row
// l % 32 and the 16 columns 8 jj + 4 g + e (g = l / 32, jj, e < 4). A row's
// softmax statistics then need one exchange between lanes l and l ^ 32.
// When such an accumulator (rows x keys) becomes the left operand of the
// next product (a reduction over keys), its 16-key step kk uses the lane's
// own registers 8 (kk % 2) .. 8 (kk % 2) + 7 as the 8 k-slots: slot 8 g + e
// holds key 16 kk + 4 g + e and slot 8 g + 4 + e key 16 kk + 8 + 4 g + e. The
// right operand (keys x columns, staged in LDS) is read with
// ds_read_b64_tr_b16 in that same key order, so no lane exchange is needed:
// the sum over keys does not depend on their order.
//
// LDS tiles: 64 rows x DP columns (DP = d rounded up to 64) as DP / 64 panels
// of 64 rows x 128 bytes. The 16-byte chunk c of row r sits at position
// c ^ asw(r). asw(r) takes 8 distinct values on the even rows and on the odd
// rows of every 16, so 16-byte fragment reads of 16 consecutive rows hit 16
// distinct bank groups; rows 4a and 4a + 2 (and 4a + 1, 4a + 3) differ in
// bit 2 of asw, so a transposed read (4 consecutive rows x 32 bytes per 16
// lanes, two such groups per 32 lanes) is conflict free as well. asw uses
// row bits 1-3 only, so every fragment address is a per-lane offset computed
// once plus a compile-time constant.
#pragma once

#include <type_traits>

#include "gemm_direct.hpp"

namespace tpl {

struct FaArgs {
  const bf16_t* qkv;     // [T, q3]: this rank's Q | K | V, token (sigma, beta) at row sigma * b + beta
  const bf16_t* qkv_lo;  // [T, 2 hr]: bf16 rounding residuals of Q | K
  bf16_t* ctx;           // [T, hr]: context C, head j at columns j d
  float* ctx32;          // [T, hr]: C in fp32 (for D of the backward)
  float* lse;            // [z, s]: log-sum-exp of each query's scores, base 2, scores in log2 units
  const bf16_t* dctx;    // [T, hr]: dC
  const float* dsum;     // [z, s]: D = rowsum(dC * C)
  bf16_t* dqkv;          // [T, q3]: dQ | dK | dV
  float* part;           // fp32 partial results of the chunks of split blocks
  int s, b, ar, d, hr, q3, z;
  int ct;     // 64-row tiles per chunk (even)
  int items;  // work items per head of the launched kernel
  float sl2;  // log2(e) / sqrt(d)
  float sc;   // 1 / sqrt(d)
};

namespace fa {

constexpr int BQ = 128;  // queries (dq) or keys (dkv) per block: 4 waves x 32
constexpr int BQF = 256; // queries per block of the forward kernel with 8 waves (d <= 128)
constexpr int BT = 64;   // rows per staged LDS tile

__host__ __device__ inline int asw(int r) { return ((r & 2) << 1) | ((r >> 2) & 3); }

// ---- work items -------------------------------------------------------------

struct Item {
  int blk, c, nch, t0, t1;  // block, chunk, chunks of the block, tile range [t0, t1)
};
// Tile range of a block of bq rows: keys [0, end of its queries) for query
// blocks, queries [its first key, s) for key blocks.
__host__ __device__ inline void block_range(int blk, int s, bool keyblocks, int& t0, int& t1, int bq = BQ) {
  const int ntot = (s + BT - 1) / BT, qe = (blk + 1) * bq < s ? (blk + 1) * bq : s;
  t0 = keyblocks ? blk * (bq / BT) : 0;
  t1 = keyblocks ? ntot : (qe + BT - 1) / BT;
}
// Item idx of one head: blocks heaviest first, each cut into chunks.
__host__ __device__ inline Item item_of(int idx, int s, int ct, bool keyblocks, int bq = BQ) {
  const int nblk = (s + bq - 1) / bq;
  for (int j = 0; j < nblk; ++j) {
    const int blk = keyblocks ? j : nblk - 1 - j;
    int t0, t1;
    block_range(blk, s, keyblocks, t0, t1, bq);
    const int nch = (t1 - t0 + ct - 1) / ct;
    if (idx < nch) {
      const int e = t0 + (idx + 1) * ct;
      return {blk, idx, nch, t0 + idx * ct, e < t1 ? e : t1};
    }
    idx -= nch;
  }
  return {-1, 0, 0, 0, 0};
}
__host__ __device__ inline int items_per_head(int s, int ct, bool keyblocks, int bq = BQ) {
  const int nblk = (s + bq - 1) / bq;
  int n = 0;
  for (int blk = 0; blk < nblk; ++blk) {
    int t0, t1;
    block_range(blk, s, keyblocks, t0, t1, bq);
    n += (t1 - t0 + ct - 1) / ct;
  }
  return n;
}
// Workgroup L -> (head z, item): the z * items list in contiguous runs per
// XCD (workgroups are dealt to the 8 XCDs round-robin); a bijection of
// [0, z * items).
__device__ __forceinline__ void xcd_item(int L, int zs, int items, int& z, int& idx) {
  const int W = zs * items, per = W >> 3, rem = W & 7, x = L & 7, k = L >> 3;
  const int i = x * per + min(x, rem) + k;
  z = i / items;
  idx = i - z * items;
}
// fp32 slot of (z, block, chunk): bq rows x d per accumulated matrix
__host__ __device__ inline long part_slot(int z, int blk, int c, int s, int ct, int d, int bq = BQ) {
  const int nblk = (s + bq - 1) / bq, ncmax = ((s + BT - 1) / BT + ct - 1) / ct;
  return (((long)z * nblk + blk) * ncmax + c) * (long)bq * d;
}

// ---- LDS tiles ----------------------------------------------------------------

// Loader of one 64-row x DP-column tile of a token-major matrix into LDS
// with global_load_lds_dwordx4 (1 KB per wave-wide instruction: 8 rows of
// one panel). Offsets are relative to the tile's first row; a tile that
// crosses the sequence end repeats its last valid row, and columns >= d
// repeat column 0: in bounds, and only ever multiplied into outputs that are
// masked or never stored.
template <int DP, int NW = 4>
struct Tile {
  static constexpr int PANELS = DP / 64;
  static constexpr int BYTES = PANELS * 8192;
  static constexpr int U4 = BYTES / 16;             // uint4 per tile
  static constexpr int PER_WAVE = PANELS * 8 / NW;  // loads per wave (NW waves)
  static_assert(PER_WAVE * NW == PANELS * 8, "the tile's loads split evenly over the waves");
  uint32_t off[PER_WAVE];
  __device__ __forceinline__ void init(int rows, long ld, int d, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int inst = wave * PER_WAVE + i;  // panel inst / 8, row group inst % 8
      const int rr = (inst & 7) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ asw(rr);
      int col = (inst >> 3) * 64 + c * 8;
      if (col >= d) col = 0;
      off[i] = (uint32_t)(((long)min(rr, rows - 1) * ld + col) * 2);
    }
  }
  __device__ __forceinline__ void issue(const bf16_t* base, uint4* lds, int wave) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) load_lds16(base, off[i], lds + (wave * PER_WAVE + i) * 64);
  }
};

// Per-lane byte offsets of the fragment reads of a tile.
//  r16[kq]   : 16-byte read of row 32 bb + l % 32, columns 8 (2 ks + g) ..,
//              ks % 4 = kq; + (ks / 4) 8192 + bb 4096.
//  tr[o][h]  : transposed read for output columns 32 nb + l % 32 (nb % 2 = o)
//              and rows 16 kk + 4 g + {0..3} (h = 0) or + 8 (h = 1);
//              + (nb / 2) 8192 + kk 2048. Within a 16-lane group,
//              ds_read_b64_tr_b16 hands lane i element i % 4 of the 8-byte
//              pieces addressed by lanes 4c + i / 4.
struct LaneOff {
  uint32_t r16[4];
  uint32_t tr[2][2];
  __device__ __forceinline__ void init(int lane) {
    const int r32 = lane & 31, g = lane >> 5, y = g ^ asw(r32);
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) r16[kq] = (uint32_t)(r32 * 128 + (((2 * kq) ^ y) << 4));
    const int G = lane >> 4, i = lane & 15;
    const int colL = 16 * (G & 1) + 4 * (i & 3), kL = 4 * (G >> 1) + (i >> 2), cL = colL >> 3;
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = kL + 8 * h;
        tr[o][h] = (uint32_t)(k * 128 + (((4 * o + cL) ^ asw(k)) << 4) + 2 * (colL & 7));
      }
  }
};

__device__ __forceinline__ uint4 lds16(const uint4* t, uint32_t off) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(t) + off);
}
__device__ __forceinline__ uint4 frag16(const uint4* t, const LaneOff& lo, int ks, int bb) {
  return lds16(t, lo.r16[ks & 3] + (uint32_t)((ks >> 2) * 8192 + bb * 4096));
}
__device__ __forceinline__ uint4 frag_tr(const uint4* t, const LaneOff& lo, int kk, int nb) {
  const uint32_t c = (uint32_t)((nb >> 1) * 8192 + kk * 2048);
  const uint2 a = read_tr(t, lo.tr[nb & 1][0] + c);
  const uint2 b = read_tr(t, lo.tr[nb & 1][1] + c);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// ---- register helpers ---------------------------------------------------------

// Left-operand fragment (bf16, round to nearest even) of 16-key step kk from
// a 32-column block of fp32 accumulators: registers 8 half .. 8 half + 7.
__device__ __forceinline__ uint4 pack_frag(const f32x16_t& a, int half) {
  const f32x4_t x = {a[8 * half], a[8 * half + 1], a[8 * half + 2], a[8 * half + 3]};
  const f32x4_t y = {a[8 * half + 4], a[8 * half + 5], a[8 * half + 6], a[8 * half + 7]};
  const bf16x4_t bx = __builtin_convertvector(x, bf16x4_t), by = __builtin_convertvector(y, bf16x4_t);
  const bf16x8_t v = {bx[0], bx[1], bx[2], bx[3], by[0], by[1], by[2], by[3]};
  return __builtin_bit_cast(uint4, v);
}

__device__ __forceinline__ void zero(f32x16_t& a) {
#pragma unroll
  for (int e = 0; e < 16; ++e) a[e] = 0.0f;
}

// v combined with the value of lane l ^ 32 (the other half of the row's
// columns), in the same order on both lanes (the operations are
// commutative): v_permlane32_swap exchanges the two 32-lane halves between
// two registers in the VALU, without an LDS round trip.
// (Written as assembly: the compiler's builtin for this instruction loses its
// second result. The s_nop covers the wait states the instruction needs after
// a VALU write of its operands.)
__device__ __forceinline__ void halves(float v, float& lo, float& hi) {
  lo = v;
  hi = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
__device__ __forceinline__ float max32(float v) {
  float lo, hi;
  halves(v, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum32(float v) {
  float lo, hi;
  halves(v, lo, hi);
  return lo + hi;
}

// Column (within a 64-wide tile) of accumulator register e of block bb.
__device__ __forceinline__ int acc_col(int bb, int e, int g) { return 32 * bb + 8 * (e >> 2) + 4 * g + (e & 3); }

// Growth of a row's running maximum (log2 units) that the forward pass
// tolerates before rescaling: with a stale maximum m the exponentials are at
// most 2^TAU, exact in fp32 and bf16 alike, and since l and C accumulate
// against the same m the final C / l is unchanged.
constexpr float TAU = 8.0f;

// acc[bb] += sum over the KS 16-wide steps of  X_row . Y_row  for the three
// split products (Xh Yh + Xh Yl + Xl Yh), Y rows 32 bb + l % 32 of two LDS
// tiles (high and low parts), X in registers. Fragment reads run one step
// ahead of the MFMAs; the scheduling barriers keep the compiler from hoisting
// every read of the tile (which would exhaust the VGPRs).
template <int KS>
__device__ __forceinline__ void split_scores(const uint4* Lh, const uint4* Ll, const LaneOff& lo,
                                             const uint4 (&xh)[KS], const uint4 (&xl)[KS], f32x16_t (&acc)[2]) {
  uint4 fh[2][2], fl[2][2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    fh[0][bb] = frag16(Lh, lo, 0, bb);
    fl[0][bb] = frag16(Ll, lo, 0, bb);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        fh[cur ^ 1][bb] = frag16(Lh, lo, ks + 1, bb);
        fl[cur ^ 1][bb] = frag16(Ll, lo, ks + 1, bb);
      }
    }
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      mma16(fh[cur][bb], xh[ks], acc[bb], bf16_t{});
      mma16(fl[cur][bb], xh[ks], acc[bb], bf16_t{});
      mma16(fh[cur][bb], xl[ks], acc[bb], bf16_t{});
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// split_scores with the low part of X read per step from this lane's LDS
// slots (xl_lds[64 ks], 16 bytes each) instead of registers.
template <int KS>
__device__ __forceinline__ void split_scores_lds(const uint4* Lh, const uint4* Ll, const LaneOff& lo,
                                                 const uint4 (&xh)[KS], const uint4* xl_lds, f32x16_t (&acc)[2]) {
  uint4 fh[2][2], fl[2][2], xl[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    fh[0][bb] = frag16(Lh, lo, 0, bb);
    fl[0][bb] = frag16(Ll, lo, 0, bb);
  }
  xl[0] = xl_lds[0];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        fh[cur ^ 1][bb] = frag16(Lh, lo, ks + 1, bb);
        fl[cur ^ 1][bb] = frag16(Ll, lo, ks + 1, bb);
      }
      xl[cur ^ 1] = xl_lds[64 * (ks + 1)];
    }
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      mma16(fh[cur][bb], xh[ks], acc[bb], bf16_t{});
      mma16(fl[cur][bb], xh[ks], acc[bb], bf16_t{});
      mma16(fh[cur][bb], xl[cur], acc[bb], bf16_t{});
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// acc[bb] += sum over KS steps of X_row . Y_row (one product), Y from LDS.
template <int KS>
__device__ __forceinline__ void row_products(const uint4* L, const LaneOff& lo, const uint4 (&x)[KS],
                                             f32x16_t (&acc)[2]) {
  uint4 f[2][2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) f[0][bb] = frag16(L, lo, 0, bb);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) f[cur ^ 1][bb] = frag16(L, lo, ks + 1, bb);
    }
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) mma16(f[cur][bb], x[ks], acc[bb], bf16_t{});
    __builtin_amdgcn_sched_barrier(0);
  }
}

// row_products with f(ks) called after the MFMAs of each step (inside its
// scheduling region): independent VALU work placed there runs while the
// matrix pipe works through those MFMAs.
template <int KS, class F>
__device__ __forceinline__ void row_products_with(const uint4* L, const LaneOff& lo, const uint4 (&x)[KS],
                                                  f32x16_t (&acc)[2], F&& f) {
  uint4 fr[2][2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) fr[0][bb] = frag16(L, lo, 0, bb);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) fr[cur ^ 1][bb] = frag16(L, lo, ks + 1, bb);
    }
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) mma16(fr[cur][bb], x[ks], acc[bb], bf16_t{});
    f(ks);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// out[nb] += P . Y over the tile's 64 rows, P given as fp32 accumulators
// p[2] (rows x 64, converted to bf16 here) and Y (64 x NB*32) read
// transposed from LDS, one 16-row step ahead.
template <int NB>
__device__ __forceinline__ void tr_products(const uint4* L, const LaneOff& lo, const f32x16_t (&p)[2],
                                            f32x16_t (&out)[NB]) {
  uint4 y[2][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) y[0][nb] = frag_tr(L, lo, 0, nb);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < 4) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) y[cur ^ 1][nb] = frag_tr(L, lo, kk + 1, nb);
    }
    const uint4 pf = pack_frag(p[kk >> 1], kk & 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) mma16(y[cur][nb], pf, out[nb], bf16_t{});
    __builtin_amdgcn_sched_barrier(0);
  }
}

// tr_products with f(kk) called after the MFMAs of each 16-row step.
template <int NB, class F>
__device__ __forceinline__ void tr_products_with(const uint4* L, const LaneOff& lo, const f32x16_t (&p)[2],
                                                 f32x16_t (&out)[NB], F&& f) {
  uint4 y[2][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) y[0][nb] = frag_tr(L, lo, 0, nb);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < 4) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) y[cur ^ 1][nb] = frag_tr(L, lo, kk + 1, nb);
    }
    const uint4 pf = pack_frag(p[kk >> 1], kk & 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) mma16(y[cur][nb], pf, out[nb], bf16_t{});
    f(kk);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Fragments of 32 rows x d of a token-major matrix straight from HBM into
// registers: lane l holds row r, columns 16 ks + 8 g .. + 7.
template <int KS>
__device__ __forceinline__ void load_rows(const bf16_t* base, long ld, int r, int g, uint4 (&f)[KS]) {
  const bf16_t* p = base + (long)r * ld + 8 * g;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) f[ks] = *reinterpret_cast<const uint4*>(p + 16 * ks);
}

// Makes the compiler complete the loads of these registers here. The tile
// loads of the main loops are inline assembly the compiler does not track;
// a register load still pending at a loop's first use would make it wait
// for vmcnt(0) inside the loop, which also drains the next tile's prefetch
// on every iteration.
template <int KS>
__device__ __forceinline__ void settle(uint4 (&f)[KS]) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(f[ks].x), "+v"(f[ks].y), "+v"(f[ks].z), "+v"(f[ks].w));
}
__device__ __forceinline__ void settle(float& x) { asm volatile("" : "+v"(x)); }

// 32 rows x 32 NB accumulator columns of one wave to fp32 partial slots in
// register order (float4 index ((wave NB + nb) 4 + jj) 64 + lane): every
// wave-wide store is 1 KB contiguous.
template <int NB>
__device__ __forceinline__ void part_store(float* slot, const f32x16_t (&o)[NB], int wave, int lane) {
  float4* p = reinterpret_cast<float4*>(slot) + wave * NB * 256 + lane;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      p[(nb * 4 + jj) * 64] = make_float4(o[nb][4 * jj], o[nb][4 * jj + 1], o[nb][4 * jj + 2], o[nb][4 * jj + 3]);
}

// Row-major bf16 (and optionally fp32) store of a wave's 32 rows x 32 NB
// accumulators times f at dst (this lane's row), columns 32 nb + 8 jj + 4 g.
template <int NB>
__device__ __forceinline__ void rows_store(bf16_t* dst, float* dst32, const f32x16_t (&o)[NB], float f, int g) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[nb][4 * jj + e] * f;
      const int col = 32 * nb + 8 * jj + 4 * g;
      Elt<bf16_t>::store4(dst + col, v);
      if (dst32) Elt<float>::store4(dst32 + col, v);
    }
}

}  // namespace fa

// ---------------------------------------------------------------------------
// forward: 1-D grid of z * items workgroups; one item = one chunk of key
// tiles of a block of 128 queries
// ---------------------------------------------------------------------------
// NW waves of 32 queries each: a block is 32 NW queries; one workgroup per
// CU, the next key tile loads while this one is computed (double-buffered).
// With NW = 8 two waves share each SIMD, so one's softmax arithmetic and
// waits overlap the other's MFMAs, and every staged key tile serves 256
// queries.
template <int D, int NW>
__device__ __forceinline__ void fa_fwd_body(const FaArgs& a, uint4* lds) {
  constexpr int DP = (D + 63) / 64 * 64, KS = D / 16, NB = D / 32, BQW = 32 * NW;
  using TL = fa::Tile<DP, NW>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int z, idx;
  fa::xcd_item(blockIdx.x, a.z, a.items, z, idx);
  const int beta = z / a.ar, head = z - (z / a.ar) * a.ar;
  const fa::Item it = fa::item_of(idx, a.s, a.ct, false, BQW);
  const int q0 = it.blk * BQW;
  const long ld = (long)a.b * a.q3, ldl = (long)a.b * 2 * a.hr;
  const bf16_t* Qh = a.qkv + (long)beta * a.q3 + head * a.d;
  const bf16_t* Kh = Qh + a.hr;
  const bf16_t* Vv = Qh + 2 * a.hr;
  const bf16_t* Ql = a.qkv_lo + (long)beta * 2 * a.hr + head * a.d;
  const bf16_t* Kl = Ql + a.hr;
  const int r32 = lane & 31, g = lane >> 5;
  const int qrow = q0 + 32 * wave + r32;
  uint4 qh[KS], ql[KS];
  fa::load_rows<KS>(Qh, ld, min(qrow, a.s - 1), g, qh);
  fa::load_rows<KS>(Ql, ldl, min(qrow, a.s - 1), g, ql);
  fa::settle(qh);
  fa::settle(ql);
  fa::LaneOff lo;
  lo.init(lane);
  TL tk, tl;  // offsets of full tiles
  tk.init(fa::BT, ld, a.d, wave, lane);
  tl.init(fa::BT, ldl, a.d, wave, lane);

  f32x16_t o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) fa::zero(o[nb]);
  float m = -INFINITY, l = 0.0f;  // every row sees its chunk's first key (chunks start at multiples of BQW)
  // key tiles this wave's rows can see (none if all its rows are past s)
  const int wt = q0 + 32 * wave < a.s ? min(it.t1, cdiv(min(a.s, q0 + 32 * wave + 32), fa::BT)) : 0;

  auto issue = [&](int t, int buf) {
    uint4* L = lds + buf * 3 * TL::U4;
    const long r0 = (long)fa::BT * t;
    if (r0 + fa::BT <= a.s) {
      tk.issue(Kh + r0 * ld, L, wave);
      tl.issue(Kl + r0 * ldl, L + TL::U4, wave);
      tk.issue(Vv + r0 * ld, L + 2 * TL::U4, wave);
    } else {  // the tile crosses the sequence end
      TL ek, el;
      ek.init(a.s - (int)r0, ld, a.d, wave, lane);
      el.init(a.s - (int)r0, ldl, a.d, wave, lane);
      ek.issue(Kh + r0 * ld, L, wave);
      el.issue(Kl + r0 * ldl, L + TL::U4, wave);
      ek.issue(Vv + r0 * ld, L + 2 * TL::U4, wave);
    }
  };
  auto compute = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    const uint4* Lk = lds + BUF * 3 * TL::U4;
    if (t < wt) {
      f32x16_t sacc[2];
      fa::zero(sacc[0]);
      fa::zero(sacc[1]);
      fa::split_scores<KS>(Lk, Lk + TL::U4, lo, qh, ql, sacc);
      // causal mask (key > query) and the sequence end, on tiles that reach them
      if (fa::BT * t + fa::BT - 1 > q0 + 32 * wave || fa::BT * t + fa::BT > a.s) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = fa::BT * t + fa::acc_col(bb, e, g);
            if (key > qrow || key >= a.s) sacc[bb][e] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[bb][e]);
      mx = fa::max32(mx) * a.sl2;  // row maximum of the tile, log2 units
      const bool grow = mx > m + fa::TAU;      // (true on the chunk's first tile: m = -inf)
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? mx : m;
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
        m = mn;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[nb][e] *= alpha;
      }
      float rs = 0.0f;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[bb][e], a.sl2, -m));
          sacc[bb][e] = p;
          rs += p;
        }
      l += fa::sum32(rs);
      fa::tr_products<NB>(Lk + 2 * TL::U4, lo, sacc, o);
    }
  };
  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    if (t + 1 < it.t1) issue(t + 1, BUF ^ 1);
    compute(bufc, t);
    wait_loads();
    __syncthreads();
  };
  issue(it.t0, 0);
  wait_loads();
  __syncthreads();
  for (int t = it.t0; t < it.t1; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < it.t1) step(std::integral_constant<int, 1>{}, t + 1);
  }

  if (it.nch > 1) {  // partial: unnormalised C, running maximum and sum
    fa::part_store<NB>(a.part + fa::part_slot(z, it.blk, it.c, a.s, a.ct, D, BQW), o, wave, lane);
    if (g == 0) {
      float2* ml = reinterpret_cast<float2*>(a.part + fa::part_slot(a.z, 0, 0, a.s, a.ct, D, BQW));
      ml[fa::part_slot(z, it.blk, it.c, a.s, a.ct, 1, BQW) + 32 * wave + r32] = make_float2(m, l);
    }
  } else if (qrow < a.s) {
    const long trow = (long)qrow * a.b + beta;
    fa::rows_store<NB>(a.ctx + trow * a.hr + head * a.d, a.ctx32 + trow * a.hr + head * a.d, o, 1.0f / l, g);
    if (g == 0) a.lse[(long)z * a.s + qrow] = m + __log2f(l);
  }
}

// 4 waves, 128-query blocks (d = 160: more live state than two waves per
// SIMD can hold)
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) fa_fwd_kernel(const FaArgs a) {
  __shared__ __attribute__((aligned(1024))) uint4 lds[2 * 3 * fa::Tile<(D + 63) / 64 * 64>::U4];
  fa_fwd_body<D, 4>(a, lds);
}
// 8 waves, 256-query blocks (d <= 128)
template <int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) fa_fwd8_kernel(const FaArgs a) {
  __shared__ __attribute__((aligned(1024))) uint4 lds[2 * 3 * fa::Tile<(D + 63) / 64 * 64>::U4];
  fa_fwd_body<D, 8>(a, lds);
}

// Forward combine: grid (blocks * NW * D / 32, z), one float4 of a block's
// 32 NW x D context per thread, in the partials' register order. For a query
// block split into chunks c with partials (C_c, m_c, l_c): M = max m_c,
// w_c = 2^(m_c - M), C = sum w_c C_c / sum w_c l_c, LSE = M + log2(sum w_c
// l_c), in chunk order.
template <int D, int NW>
__global__ void __launch_bounds__(256) fa_fwd_combine_kernel(const FaArgs a) {
  constexpr int NB = D / 32, PER = NW * D / 32, BQW = 32 * NW;
  const int blk = blockIdx.x / PER, z = blockIdx.y, beta = z / a.ar, head = z - (z / a.ar) * a.ar;
  int t0, t1;
  fa::block_range(blk, a.s, false, t0, t1, BQW);
  const int nch = cdiv(t1 - t0, a.ct);
  if (nch <= 1) return;
  const int j = (blockIdx.x - blk * PER) * 256 + threadIdx.x;  // float4 index in register order
  const int wave = j / (NB * 256), rem = j - wave * (NB * 256), nb = rem >> 8, jj = (rem >> 6) & 3,
            lane = rem & 63;
  const int r = 32 * wave + (lane & 31), qrow = blk * BQW + r;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (qrow < a.s) {  // (rows past the sequence end: nothing to combine)
    const float2* ml = reinterpret_cast<const float2*>(a.part + fa::part_slot(a.z, 0, 0, a.s, a.ct, D, BQW));
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, ml[fa::part_slot(z, blk, c, a.s, a.ct, 1, BQW) + r].x);
    float L = 0.0f;
    // chunks in order; all of a chunk pair's loads go out before its sums
    auto part4 = [&](int c) {
      return reinterpret_cast<const float4*>(a.part + fa::part_slot(z, blk, c, a.s, a.ct, D, BQW))[j];
    };
    auto add = [&](const float2 x, const float4 p) {
      const float w = __builtin_amdgcn_exp2f(x.x - M);
      L += w * x.y;
      v[0] += w * p.x; v[1] += w * p.y; v[2] += w * p.z; v[3] += w * p.w;
    };
    int c = 0;
    for (; c + 2 <= nch; c += 2) {
      const float2 x0 = ml[fa::part_slot(z, blk, c, a.s, a.ct, 1, BQW) + r];
      const float2 x1 = ml[fa::part_slot(z, blk, c + 1, a.s, a.ct, 1, BQW) + r];
      const float4 p0 = part4(c), p1 = part4(c + 1);
      add(x0, p0);
      add(x1, p1);
    }
    if (c < nch) add(ml[fa::part_slot(z, blk, c, a.s, a.ct, 1, BQW) + r], part4(c));
    const float inv = 1.0f / L;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= inv;
    if (nb == 0 && jj == 0 && lane < 32) a.lse[(long)z * a.s + qrow] = M + __log2f(L);
  }
  // The block's 1024 values are 32 rows x 32 columns; in register order a
  // store instruction would write 16 bytes to each of 32 rows. Staged
  // through LDS, 8 consecutive threads write one row's 32 columns.
  __shared__ float4 st[32][8];
  const int c4 = 2 * jj + (lane >> 5);
  st[lane & 31][c4] = make_float4(v[0], v[1], v[2], v[3]);
  __syncthreads();
  const int rr = threadIdx.x >> 3, cc = threadIdx.x & 7;
  const int qrow2 = blk * BQW + 32 * wave + rr;
  if (qrow2 < a.s) {
    const float4 x = st[rr][cc];
    const float w4[4] = {x.x, x.y, x.z, x.w};
    const long trow2 = (long)qrow2 * a.b + beta;
    const int col2 = head * a.d + 32 * nb + 4 * cc;
    Elt<bf16_t>::store4(a.ctx + trow2 * a.hr + col2, w4);
    Elt<float>::store4(a.ctx32 + trow2 * a.hr + col2, w4);
  }
}

// ---------------------------------------------------------------------------
// backward, dK and dV: 1-D grid of z * items; one item = one chunk of query
// tiles of a block of 128 keys (key blocks first-to-last: the first sees
// every query)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
fa_bwd_dkv_kernel(const FaArgs a) {
  constexpr int DP = (D + 63) / 64 * 64, KS = D / 16, NB = D / 32;
  using TL = fa::Tile<DP>;
  constexpr int STAGE = 3 * TL::U4 + 32;  // Qh, Ql, dC tiles + 64 LSE + 64 D (floats)
  __shared__ __attribute__((aligned(1024))) uint4 lds[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int z, idx;
  fa::xcd_item(blockIdx.x, a.z, a.items, z, idx);
  const int beta = z / a.ar, head = z - (z / a.ar) * a.ar;
  const fa::Item it = fa::item_of(idx, a.s, a.ct, true);
  const int k0 = it.blk * fa::BQ;
  const long ld = (long)a.b * a.q3, ldl = (long)a.b * 2 * a.hr, ldc = (long)a.b * a.hr;
  const bf16_t* Qh = a.qkv + (long)beta * a.q3 + head * a.d;
  const bf16_t* Kh = Qh + a.hr;
  const bf16_t* Vv = Qh + 2 * a.hr;
  const bf16_t* Ql = a.qkv_lo + (long)beta * 2 * a.hr + head * a.d;
  const bf16_t* Kl = Ql + a.hr;
  const bf16_t* dC = a.dctx + (long)beta * a.hr + head * a.d;
  const float* lse = a.lse + (long)z * a.s;
  const float* dsum = a.dsum + (long)z * a.s;
  const int r32 = lane & 31, g = lane >> 5;
  const int krow = k0 + 32 * wave + r32;
  uint4 kh[KS], kl[KS], vf[KS];
  fa::load_rows<KS>(Kh, ld, min(krow, a.s - 1), g, kh);
  fa::load_rows<KS>(Kl, ldl, min(krow, a.s - 1), g, kl);
  fa::load_rows<KS>(Vv, ld, min(krow, a.s - 1), g, vf);
  fa::settle(kh);
  fa::settle(kl);
  fa::settle(vf);
  fa::LaneOff lo;
  lo.init(lane);
  TL tq, tl, td;
  tq.init(fa::BT, ld, a.d, wave, lane);
  tl.init(fa::BT, ldl, a.d, wave, lane);
  td.init(fa::BT, ldc, a.d, wave, lane);

  f32x16_t dk[NB], dv[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    fa::zero(dk[nb]);
    fa::zero(dv[nb]);
  }
  const int kmin = k0 + 32 * wave;  // smallest key of this wave

  auto issue = [&](int t, int buf) {
    uint4* L = lds + buf * STAGE;
    const long r0 = (long)fa::BT * t;
    if (r0 + fa::BT <= a.s) {
      tq.issue(Qh + r0 * ld, L, wave);
      tl.issue(Ql + r0 * ldl, L + TL::U4, wave);
      td.issue(dC + r0 * ldc, L + 2 * TL::U4, wave);
    } else {  // the tile crosses the sequence end
      TL eq, el, ed;
      eq.init(a.s - (int)r0, ld, a.d, wave, lane);
      el.init(a.s - (int)r0, ldl, a.d, wave, lane);
      ed.init(a.s - (int)r0, ldc, a.d, wave, lane);
      eq.issue(Qh + r0 * ld, L, wave);
      el.issue(Ql + r0 * ldl, L + TL::U4, wave);
      ed.issue(dC + r0 * ldc, L + 2 * TL::U4, wave);
    }
    // LSE and D of the tile's 64 queries (16 bytes per lane; s is a multiple
    // of 4, chunks past the sequence end repeat its last chunk: finite, and
    // only ever multiplied by a masked zero)
    if (wave == 0 && lane < 16) {
      const uint32_t q = (uint32_t)min(fa::BT * t + 4 * lane, a.s - 4);
      load_lds16(reinterpret_cast<const bf16_t*>(lse), q * 4u, L + 3 * TL::U4);
      load_lds16(reinterpret_cast<const bf16_t*>(dsum), q * 4u, L + 3 * TL::U4 + 16);
    }
  };
  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    if (t + 1 < it.t1) issue(t + 1, BUF ^ 1);
    const uint4* Lq = lds + BUF * STAGE;
    const uint4* Ld = Lq + 2 * TL::U4;
    const float* Lf = reinterpret_cast<const float*>(Lq + 3 * TL::U4);
    if (kmin < a.s && fa::BT * t + fa::BT - 1 >= kmin) {  // some query of the tile sees a key of this wave
      f32x16_t st[2];
      fa::zero(st[0]);
      fa::zero(st[1]);
      fa::split_scores<KS>(Lq, Lq + TL::U4, lo, kh, kl, st);
      // P^T (keys x queries), visible iff key <= query < s.  Tiles clear of
      // the diagonal and the sequence end take the unmasked form (a runtime
      // per-element mask would become one branch per element).
      auto expo = [&](auto masked, int i) {
        const int bb = i >> 4, e = i & 15;
        const int c = fa::acc_col(bb, e, g);
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[bb][e], a.sl2, -Lf[c]));
        if constexpr (decltype(masked)::value) {
          const int q = fa::BT * t + c;
          st[bb][e] = (q < krow || q >= a.s) ? 0.0f : p;
        } else {
          st[bb][e] = p;
        }
      };
      const bool edge = fa::BT * t < kmin + 32 || fa::BT * t + fa::BT > a.s;
      // dS^T = P^T (dP^T - D) / sqrt(d), in place of dP^T
      f32x16_t dp[2];
      auto dsi = [&](int i) {
        const int bb = i >> 4, e = i & 15;
        const int c = fa::acc_col(bb, e, g);
        dp[bb][e] = st[bb][e] * a.sc * (dp[bb][e] - Lf[64 + c]);
      };
      fa::zero(dp[0]);
      fa::zero(dp[1]);
      if constexpr (D <= 128) {
        // dP^T = V dC^T does not depend on the scores, so its MFMAs go first
        // with the exponentials spread over its steps, and dS^T is formed
        // under the MFMAs of dV += P^T dC: the VALU work runs while the
        // matrix pipe is busy instead of between the products.
        constexpr int EPS = (32 + KS - 1) / KS;  // exponentials per dP^T step
        auto run = [&](auto masked) {
          fa::row_products_with<KS>(Ld, lo, vf, dp, [&](int ks) {
#pragma unroll
            for (int j = 0; j < EPS; ++j)
              if (ks * EPS + j < 32) expo(masked, ks * EPS + j);
          });
        };
        if (edge) run(std::true_type{});
        else run(std::false_type{});
        fa::tr_products_with<NB>(Ld, lo, st, dv, [&](int kk) {
#pragma unroll
          for (int j = 0; j < 8; ++j) dsi(kk * 8 + j);
        });
      } else {
        // d = 160: the registers leave no room to hold dP^T through dV's
        // products, so the steps run in dependency order.
        auto run = [&](auto masked) {
#pragma unroll
          for (int i = 0; i < 32; ++i) expo(masked, i);
        };
        if (edge) run(std::true_type{});
        else run(std::false_type{});
        fa::tr_products<NB>(Ld, lo, st, dv);  // dV += P^T dC
        fa::row_products<KS>(Ld, lo, vf, dp);  // dP^T = V dC^T
#pragma unroll
        for (int i = 0; i < 32; ++i) dsi(i);
      }
      fa::tr_products<NB>(Lq, lo, dp, dk);  // dK += dS^T Qh
    }
    wait_loads();
    __syncthreads();
  };
  issue(it.t0, 0);
  wait_loads();
  __syncthreads();
  for (int t = it.t0; t < it.t1; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < it.t1) step(std::integral_constant<int, 1>{}, t + 1);
  }

  if (it.nch > 1) {  // partials: dK then dV
    float* slot = a.part + 2 * fa::part_slot(z, it.blk, it.c, a.s, a.ct, D);
    fa::part_store<NB>(slot, dk, wave, lane);
    fa::part_store<NB>(slot + fa::BQ * D, dv, wave, lane);
  } else if (krow < a.s) {
    const long trow = (long)krow * a.b + beta;
    bf16_t* dK = a.dqkv + trow * a.q3 + a.hr + head * a.d;
    fa::rows_store<NB>(dK, nullptr, dk, 1.0f, g);
    fa::rows_store<NB>(dK + a.hr, nullptr, dv, 1.0f, g);
  }
}

// ---------------------------------------------------------------------------
// backward, dQ: items as in the forward pass
// ---------------------------------------------------------------------------
template <int D, int NBUF, bool QLDS = false>
__device__ __forceinline__ void fa_dq_body(const FaArgs& a, uint4* lds, uint4* qlo_lds = nullptr) {
  constexpr int DP = (D + 63) / 64 * 64, KS = D / 16, NB = D / 32;
  using TL = fa::Tile<DP>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int z, idx;
  fa::xcd_item(blockIdx.x, a.z, a.items, z, idx);
  const int beta = z / a.ar, head = z - (z / a.ar) * a.ar;
  const fa::Item it = fa::item_of(idx, a.s, a.ct, false);
  const int q0 = it.blk * fa::BQ;
  const long ld = (long)a.b * a.q3, ldl = (long)a.b * 2 * a.hr, ldc = (long)a.b * a.hr;
  const bf16_t* Qh = a.qkv + (long)beta * a.q3 + head * a.d;
  const bf16_t* Kh = Qh + a.hr;
  const bf16_t* Vv = Qh + 2 * a.hr;
  const bf16_t* Ql = a.qkv_lo + (long)beta * 2 * a.hr + head * a.d;
  const bf16_t* Kl = Ql + a.hr;
  const bf16_t* dC = a.dctx + (long)beta * a.hr + head * a.d;
  const int r32 = lane & 31, g = lane >> 5;
  const int qrow = q0 + 32 * wave + r32;
  const int qc = min(qrow, a.s - 1);
  uint4 qh[KS], ql[KS], dof[KS];
  fa::load_rows<KS>(Qh, ld, qc, g, qh);
  fa::load_rows<KS>(Ql, ldl, qc, g, ql);
  fa::load_rows<KS>(dC, ldc, qc, g, dof);
  float lse = a.lse[(long)z * a.s + qc];
  float dsum = a.dsum[(long)z * a.s + qc];
  fa::settle(qh);
  fa::settle(ql);
  fa::settle(dof);
  fa::settle(lse);
  fa::settle(dsum);
  // (single-buffered, two workgroups per CU: Q's low part waits in LDS, which
  // frees its registers for the loop)
  uint4* const xl_lds = QLDS ? qlo_lds + wave * KS * 64 + lane : nullptr;
  if constexpr (QLDS) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xl_lds[64 * ks] = ql[ks];
  }
  fa::LaneOff lo;
  lo.init(lane);
  TL tk, tl;
  tk.init(fa::BT, ld, a.d, wave, lane);
  tl.init(fa::BT, ldl, a.d, wave, lane);

  f32x16_t dq[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) fa::zero(dq[nb]);
  const int wt = q0 + 32 * wave < a.s ? min(it.t1, cdiv(min(a.s, q0 + 32 * wave + 32), fa::BT)) : 0;

  auto issue = [&](int t, int buf) {
    uint4* L = lds + buf * 3 * TL::U4;
    const long r0 = (long)fa::BT * t;
    if (r0 + fa::BT <= a.s) {
      tk.issue(Kh + r0 * ld, L, wave);
      tl.issue(Kl + r0 * ldl, L + TL::U4, wave);
      tk.issue(Vv + r0 * ld, L + 2 * TL::U4, wave);
    } else {  // the tile crosses the sequence end
      TL ek, el;
      ek.init(a.s - (int)r0, ld, a.d, wave, lane);
      el.init(a.s - (int)r0, ldl, a.d, wave, lane);
      ek.issue(Kh + r0 * ld, L, wave);
      el.issue(Kl + r0 * ldl, L + TL::U4, wave);
      ek.issue(Vv + r0 * ld, L + 2 * TL::U4, wave);
    }
  };
  auto compute = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    const uint4* Lk = lds + BUF * 3 * TL::U4;
    if (t < wt) {
      f32x16_t sacc[2], dp[2];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        fa::zero(sacc[bb]);
        fa::zero(dp[bb]);
      }
      if constexpr (QLDS) fa::split_scores_lds<KS>(Lk, Lk + TL::U4, lo, qh, xl_lds, sacc);
      else fa::split_scores<KS>(Lk, Lk + TL::U4, lo, qh, ql, sacc);
      fa::row_products<KS>(Lk + 2 * TL::U4, lo, dof, dp);  // dP = dC V^T
      // dS = P (dP - D) / sqrt(d), P = 0 for key > query or key >= s
      const bool edge = fa::BT * t + fa::BT - 1 > q0 + 32 * wave || fa::BT * t + fa::BT > a.s;
      // (with Q's low part in LDS the registers allow a second, mask-free loop
      // for tiles clear of the diagonal, as in the dK/dV kernel)
      if (!QLDS || edge) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = fa::BT * t + fa::acc_col(bb, e, g);
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[bb][e], a.sl2, -lse));
            const float v = p * a.sc * (dp[bb][e] - dsum);
            dp[bb][e] = (edge && (key > qrow || key >= a.s)) ? 0.0f : v;
          }
      } else {  // clear of the diagonal and the sequence end: no mask
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[bb][e], a.sl2, -lse));
            dp[bb][e] = p * a.sc * (dp[bb][e] - dsum);
          }
      }
      fa::tr_products<NB>(Lk, lo, dp, dq);  // dQ += dS Kh
    }
  };
  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    if (t + 1 < it.t1) issue(t + 1, BUF ^ 1);
    compute(bufc, t);
    wait_loads();
    __syncthreads();
  };
  if constexpr (NBUF == 2) {
    issue(it.t0, 0);
    wait_loads();
    __syncthreads();
    for (int t = it.t0; t < it.t1; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < it.t1) step(std::integral_constant<int, 1>{}, t + 1);
    }
  } else {
    for (int t = it.t0; t < it.t1; ++t) {
      issue(t, 0);
      wait_loads();
      __syncthreads();
      compute(std::integral_constant<int, 0>{}, t);
      __syncthreads();
    }
  }

  if (it.nch > 1) {
    fa::part_store<NB>(a.part + fa::part_slot(z, it.blk, it.c, a.s, a.ct, D), dq, wave, lane);
  } else if (qrow < a.s) {
    const long trow = (long)qrow * a.b + beta;
    fa::rows_store<NB>(a.dqkv + trow * a.q3 + head * a.d, nullptr, dq, 1.0f, g);
  }
}

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
fa_bwd_dq_kernel(const FaArgs a) {
  __shared__ __attribute__((aligned(1024))) uint4 lds[2 * 3 * fa::Tile<(D + 63) / 64 * 64>::U4];
  fa_dq_body<D, 2>(a, lds);
}
template <int D>
__global__ void __launch_bounds__(256, 2) fa_bwd_dq2_kernel(const FaArgs a) {
  __shared__ __attribute__((aligned(1024))) uint4 lds[3 * fa::Tile<(D + 63) / 64 * 64>::U4];
  __shared__ __attribute__((aligned(16))) uint4 qlo[4 * (D / 16) * 64];
  fa_dq_body<D, 1, true>(a, lds, qlo);
}

// Backward combine: grid (blocks * D / 8, z), one float4 per thread per
// matrix, in the partials' register order. Sums the chunk partials of split
// blocks in chunk order: KEYS = false, dQ (query blocks); KEYS = true, dK and
// dV (key blocks).
template <int D, bool KEYS>
__global__ void __launch_bounds__(256) fa_bwd_combine_kernel(const FaArgs a) {
  constexpr int NB = D / 32, PER = D / 8, MATS = KEYS ? 2 : 1;
  const int blk = blockIdx.x / PER, z = blockIdx.y, beta = z / a.ar, head = z - (z / a.ar) * a.ar;
  int t0, t1;
  fa::block_range(blk, a.s, KEYS, t0, t1);
  const int nch = cdiv(t1 - t0, a.ct);
  if (nch <= 1) return;
  const int j = (blockIdx.x - blk * PER) * 256 + threadIdx.x;
  const int wave = j / (NB * 256), rem = j - wave * (NB * 256), nb = rem >> 8, jj = (rem >> 6) & 3,
            lane = rem & 63;
  const int row = blk * fa::BQ + 32 * wave + (lane & 31);
  // the block's values are 32 rows x 32 columns of each matrix; they are
  // staged through LDS so that 8 consecutive threads store one row's 32
  // columns (in register order a store would write 8 bytes to each of 32 rows)
  __shared__ float4 st[32][8];
  const int rr = threadIdx.x >> 3, cc = threadIdx.x & 7;
  const int row2 = blk * fa::BQ + 32 * wave + rr;
  const long trow2 = (long)row2 * a.b + beta;
  const int col2 = head * a.d + 32 * nb + 4 * cc;
#pragma unroll
  for (int mat = 0; mat < MATS; ++mat) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (row < a.s) {
      // chunks in order, two loads in flight per step
      auto part4 = [&](int c) {
        return reinterpret_cast<const float4*>(a.part + MATS * fa::part_slot(z, blk, c, a.s, a.ct, D) +
                                               mat * fa::BQ * D)[j];
      };
      int c = 0;
      for (; c + 2 <= nch; c += 2) {
        const float4 x = part4(c), y = part4(c + 1);
        v[0] = (v[0] + x.x) + y.x; v[1] = (v[1] + x.y) + y.y; v[2] = (v[2] + x.z) + y.z; v[3] = (v[3] + x.w) + y.w;
      }
      if (c < nch) {
        const float4 x = part4(c);
        v[0] += x.x; v[1] += x.y; v[2] += x.z; v[3] += x.w;
      }
    }
    if (mat > 0) __syncthreads();  // the previous matrix's stores have read st
    st[lane & 31][2 * jj + (lane >> 5)] = make_float4(v[0], v[1], v[2], v[3]);
    __syncthreads();
    if (row2 < a.s) {
      const float4 x = st[rr][cc];
      const float w4[4] = {x.x, x.y, x.z, x.w};
      Elt<bf16_t>::store4(a.dqkv + trow2 * a.q3 + (KEYS ? (1 + mat) * a.hr : 0) + col2, w4);
    }
  }
}

}  // namespace tpl
