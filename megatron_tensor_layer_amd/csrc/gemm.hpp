// MFMA GEMM for gfx950: C = epilogue(op(A) * op(B)), bf16 or fp32 operands,
// fp32 accumulation, LDS-staged double-buffered tiles, fused epilogues.
//
// Design (CDNA4, 64-wide waves):
//  * A block computes a BM x BN tile with WM x WN waves; each wave owns a
//    (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles
//    (v_mfma_f32_32x32x16_bf16 for bf16, v_mfma_f32_32x32x2_f32 for fp32).
//  * Both operands are staged in LDS "K-contiguous": one 128-byte LDS row
//    holds BK = 64 bf16 (32 fp32) consecutive k of one m (or n) index, so an
//    MFMA fragment (8 bf16 / 4 fp32 consecutive k of one row) is a single
//    16-byte LDS read. The eight 16-byte chunks of a row are XOR-swizzled by
//    (row & 7), which makes both the fragment reads and the stores
//    bank-conflict free.
//  * An operand stored K-contiguous in HBM (e.g. X in X W, or W in dY W^T) is
//    copied chunk by chunk. An operand stored M/N-contiguous (W in X W, both
//    operands of a weight gradient X^T dY) is read as VECxVEC element blocks
//    (VEC rows of k, 16 bytes along m/n each) and transposed in registers
//    before the LDS store, so the LDS layout and the inner loop are the same
//    for every operand orientation.
//  * fp32 MFMA pairs lanes 0-31 / 32-63 with k = 0 / 1 of each 32x32x2 step;
//    feeding element e of a 4-float chunk to step e makes one 16-byte
//    fragment cover 8 k values in 4 steps. A and B use the same k order, so
//    the sum over k is unchanged.
//  * The MFMA is issued with the B fragment as its first operand, which puts
//    one output row m and four consecutive columns n in each lane: epilogues
//    load bias / residual / aux values and store results 4 elements at a time.
//  * Tiles are ordered in groups of GM tile-rows and remapped so that
//    consecutive tiles land on the same XCD (workgroups are dealt to the 8
//    XCDs round-robin), so co-resident blocks share A and B panels in L2.
//  * Causal (lower-triangular) tile sets and causal K ranges serve the
//    attention products; split-K writes fp32 partials reduced in a fixed
//    order by a second kernel (no atomics, deterministic).
#pragma once

#include "tp_common.hpp"

namespace tpl {

enum EpiKind : int {
  EPI_LINEAR = 0,       // C = alpha*acc (+ bias[n]) (+ resid[m,n])
  EPI_BIAS_GELU = 1,    // U = acc + bias[n] -> C;  GELU(U) -> C2
  EPI_GELU_BWD = 2,     // C = acc * gelu'(aux[m,n])
  EPI_SOFTMAX_BWD = 3,  // C = (n <= m) ? alpha * aux[m,n] * (acc - rowv[m]) : 0
  EPI_PARTIAL = 4,      // split-K: fp32 partial[split, m, n] = acc
  EPI_BIAS_SPLIT = 5,   // V = acc + bias[n] -> C (bf16); for n < c2_cols also the
                        // rounding residual V - bf16(V) -> C2 (bf16, row pitch ldc2)
  EPI_DUAL_F32 = 6,     // C = acc (storage type) and C2 = acc (fp32), same layout
  EPI_SK_PART = 7       // fp32 accumulator fragment of a stream-K unit, tile-row-major
};

enum KMode : int {
  K_FULL = 0,   // k in [0, K)
  K_LOWER = 1,  // k in [0, min(K, m0 + BM))   (causal: key <= query)
  K_UPPER = 2   // k in [m0, K)                 (causal: query >= key)
};

struct GemmArgs {
  int M, N, K;
  int zdiv;              // batch z -> (z1, z2) = (z / zdiv, z % zdiv)
  int tiles_m, tiles_n;  // set by the launcher
  int tri;               // 1: only tiles with tile_n <= tile_m (BM == BN)
  int kmode;
  int splits, k_chunk;   // split-K (EPI_PARTIAL pass)
  int group_m;           // tile-rows per ordering group
  int no_xcd;            // 1: tile index is used as given (the launch maps blocks to XCDs itself);
                         // 2: as 1, and stream-K tiles (index >= skm_base) are placed by the skm_* map
  int skm_base, skm_col0;  // first stream-K tile index; first tile-column of the stream-K region
  int skm_br, skm_bc;      // tiles of one XCD: a block of skm_br x skm_bc tiles
  int skm_q, skm_gr, skm_gc;  // runs of one K phase: skm_q groups of skm_gr x skm_gc tiles per block
  int xcd_br, xcd_bc, xcd_g;  // > 0: XCD x takes one xcd_br x xcd_bc block of tiles (blocks laid out
                             // row-major over the tile grid), walked in strips of xcd_g tile-rows
  int kseg, kseg_len;    // kseg = 3: K runs over (A,B), (A,B2), (A2,B), each kseg_len long
  int c2_cols;           // EPI_BIAS_SPLIT: columns that get a residual in C2
  const void* A; long lda, a_s1, a_s2;
  const void* B; long ldb, b_s1, b_s2;
  const void* A2;  // second halves of split operands: same strides as A / B
  const void* B2;
  void* C; long ldc, c_s1, c_s2;
  void* C2; long ldc2;
  const void* bias;
  const void* resid; long ldr;
  const void* aux; long ldx, x_s1, x_s2;
  const float* rowv; long r_s1, r_s2;
  float alpha;
  float* part;
  void* csum;  // direct bf16 kernel, grouped launches: bf16 [N] sum over k of B[k, n] (tiles of tile-row 0)
};

// Stream-K launch plan (direct bf16 kernel, batch 1). Blocks [0, dp_tiles)
// compute whole tiles; the remaining sk_tiles tiles' K iterations (iters of
// BK each per tile) are laid end to end and cut into `units` runs of c
// iterations, one run per block. A run that covers only part of a tile
// stores its fp32 fragment in slot (unit - first unit of the tile) of that
// tile's f slots; the fix-up kernel sums the slots in order and applies the
// epilogue. dp_tiles and units are multiples of 8 (one run of blocks per XCD).
struct SkPlan {
  int dp_tiles, sk_tiles, iters, c, units, f;
  float* part;
};

template <typename T_, int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  using T = T_;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int VEC = Elt<T>::VEC;
  static constexpr int BK = 8 * VEC;  // one 128-byte LDS row
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static constexpr int LDS_BYTES = 2 * (BM + BN) * 128;
};

// ---------------------------------------------------------------------------
// global -> LDS loaders
//
// Each thread owns fixed 16-byte chunks of the BM x BK (BN x BK) tile; their
// element offsets relative to the tile's k origin are computed once. Rows
// beyond M (N) are clamped to the last valid row: they only feed output rows
// (columns) that are never stored. k beyond the K range must read as zero;
// that happens only in a ragged last K tile, handled by a uniform branch.
// ---------------------------------------------------------------------------

// Operand stored K-contiguous: element (row, k) at base[row*ld + k].
template <typename T, int R, int NT>
struct KLoader {
  static constexpr int VEC = Elt<T>::VEC;
  static constexpr int BK = 8 * VEC;
  static constexpr int TOTAL = R * 8;  // 16-byte chunks in an R x BK tile
  static_assert(TOTAL % NT == 0, "tile rows must cover the threads");
  static constexpr int CH = TOTAL / NT;
  static constexpr int LOADS = CH, STORES = CH;  // global loads / LDS stores per tile
  uint32_t off[CH];
  uint4 v[CH];

  __device__ __forceinline__ void init(long ld, int row0, int rlim, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * NT;
      const int row = min(row0 + (c >> 3), rlim - 1);
      off[i] = (uint32_t)((long)row * ld + (c & 7) * VEC);
    }
  }
  // base = operand origin advanced to the tile's first k; kvalid = k range
  // left (> 0). TAIL: chunks at k >= kvalid read the tile's first chunk of the
  // row (always in bounds) and are replaced by zeros.
  template <bool TAIL>
  __device__ __forceinline__ void load(const T* base, long ld, int kvalid, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if constexpr (!TAIL) {
        v[i] = *reinterpret_cast<const uint4*>(base + off[i]);
      } else {
        const int kc = ((tid + i * NT) & 7) * VEC;
        const bool ok = kc < kvalid;
        const uint4 x = *reinterpret_cast<const uint4*>(base + (off[i] - (ok ? 0 : kc)));
        v[i] = ok ? x : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * NT;
      const int r = c >> 3, kc = c & 7;
      lds[r * 8 + (kc ^ (r & 7))] = v[i];
    }
  }
  __device__ __forceinline__ static const T* advance(const T* base, long ld, int k) { return base + k; }
};

__device__ __forceinline__ uint32_t dw(const uint4& x, int q) {
  return q == 0 ? x.x : (q == 1 ? x.y : (q == 2 ? x.z : x.w));
}

// in[r] = 8 bf16 (k = r, mn = 0..7)  ->  out[j] = 8 bf16 (k = 0..7, mn = j)
__device__ __forceinline__ void transpose_blk(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = dw(in[2 * q], j >> 1), hi = dw(in[2 * q + 1], j >> 1);
      w[q] = (j & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u) : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    out[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// in[r] = 4 fp32 (k = r, mn = 0..3)  ->  out[j] = 4 fp32 (k = 0..3, mn = j)
__device__ __forceinline__ void transpose_blk(const uint4 (&in)[4], uint4 (&out)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = make_uint4(dw(in[0], j), dw(in[1], j), dw(in[2], j), dw(in[3], j));
}

// Operand stored M/N-contiguous: element (mn, k) at base[k*ld + mn]. A thread
// loads VEC rows of k x 16 bytes of mn and transposes them in registers.
template <typename T, int R, int NT>
struct MNLoader {
  static constexpr int VEC = Elt<T>::VEC;
  static constexpr int BK = 8 * VEC;
  static constexpr int TOTAL = (R / VEC) * 8;  // VEC x VEC blocks in an R x BK tile
  static constexpr int BPT = (TOTAL + NT - 1) / NT;
  static constexpr int LOADS = BPT * VEC, STORES = BPT * VEC;
  uint32_t off[BPT];
  uint4 v[BPT][VEC];

  __device__ __forceinline__ void init(long ld, int mn0, int mnlim, int tid) {
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int c = min(tid + b * NT, TOTAL - 1);
      const int kc = c & 7;
      const int mn = min(mn0 + (c >> 3) * VEC, mnlim - VEC);
      off[b] = (uint32_t)((long)(kc * VEC) * ld + mn);
    }
  }
  template <bool TAIL>
  __device__ __forceinline__ void load(const T* base, long ld, int kvalid, int tid) {
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int kc = (min(tid + b * NT, TOTAL - 1) & 7) * VEC;
#pragma unroll
      for (int r = 0; r < VEC; ++r) {
        if constexpr (!TAIL) {
          v[b][r] = *reinterpret_cast<const uint4*>(base + r * ld + off[b]);
        } else {
          // rows k >= kvalid read row 0 of the tile (in bounds) and become zeros
          const bool ok = kc + r < kvalid;
          const uint4 x = *reinterpret_cast<const uint4*>(base + (ok ? r * ld + off[b] : off[b] - (long)kc * ld));
          v[b][r] = ok ? x : make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int c = tid + b * NT;
      if (TOTAL % NT == 0 || c < TOTAL) {
        const int kc = c & 7, mb = c >> 3;
        uint4 w[VEC];
        transpose_blk(v[b], w);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int row = mb * VEC + j;
          lds[row * 8 + (kc ^ (row & 7))] = w[j];
        }
      }
    }
  }
  __device__ __forceinline__ static const T* advance(const T* base, long ld, int k) { return base + (long)k * ld; }
};

template <bool KMAJ, typename T, int R, int NT>
struct LoaderSel {
  using type = KLoader<T, R, NT>;
};
template <typename T, int R, int NT>
struct LoaderSel<false, T, R, NT> {
  using type = MNLoader<T, R, NT>;
};

// ---------------------------------------------------------------------------
// MFMA step on one 16-byte fragment pair
// ---------------------------------------------------------------------------

__device__ __forceinline__ void mma16(const uint4& bfrag, const uint4& afrag, f32x16_t& acc, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bfrag),
                                                __builtin_bit_cast(bf16x8_t, afrag), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(const uint4& bfrag, const uint4& afrag, f32x16_t& acc, float) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(bfrag.x), __uint_as_float(afrag.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(bfrag.y), __uint_as_float(afrag.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(bfrag.z), __uint_as_float(afrag.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(bfrag.w), __uint_as_float(afrag.w), acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// epilogue on 4 consecutive columns of one row
// ---------------------------------------------------------------------------

// V = 4 or 8 consecutive columns col..col+V-1 of one row (V divides N).
template <int EPI, typename T, typename TO, int V = 4>
__device__ __forceinline__ void epi_apply(const GemmArgs& p, int z1, int z2, int row, int col, float v[V], int split) {
  if constexpr (EPI == EPI_PARTIAL) {
    storev<float, V>(p.part + ((long)split * p.M + row) * (long)p.N + col, v);
    return;
  } else {
    if constexpr (EPI == EPI_LINEAR) {
      if (p.alpha != 1.0f) {
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] *= p.alpha;
      }
      if (p.bias) {
        float bb[V];
        loadv<T, V>(static_cast<const T*>(p.bias) + col, bb);
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] += bb[e];
      }
      if (p.resid) {
        float rr[V];
        loadv<T, V>(static_cast<const T*>(p.resid) + (long)row * p.ldr + col, rr);
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] += rr[e];
      }
    } else if constexpr (EPI == EPI_BIAS_GELU) {
      float bb[V];
      loadv<T, V>(static_cast<const T*>(p.bias) + col, bb);
      float g[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        v[e] += bb[e];
        g[e] = gelu_f(v[e]);
      }
      storev<T, V>(static_cast<T*>(p.C2) + (long)row * p.ldc2 + col, g);
    } else if constexpr (EPI == EPI_GELU_BWD) {
      float u[V];
      loadv<T, V>(static_cast<const T*>(p.aux) + (long)row * p.ldx + col, u);
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] *= gelu_grad_f(u[e]);
    } else if constexpr (EPI == EPI_BIAS_SPLIT) {
      float bb[V];
      loadv<T, V>(static_cast<const T*>(p.bias) + col, bb);
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] += bb[e];
      if (col < p.c2_cols) {
        float lo[V];
#pragma unroll
        for (int e = 0; e < V; ++e) lo[e] = v[e] - bf2f(f2bf(v[e]));
        storev<T, V>(static_cast<T*>(p.C2) + (long)row * p.ldc2 + col, lo);
      }
    } else if constexpr (EPI == EPI_DUAL_F32) {
      storev<float, V>(static_cast<float*>(p.C2) + z1 * p.c_s1 + z2 * p.c_s2 + (long)row * p.ldc + col, v);
    } else if constexpr (EPI == EPI_SOFTMAX_BWD) {
      float pp[V];
      loadv<T, V>(static_cast<const T*>(p.aux) + z1 * p.x_s1 + z2 * p.x_s2 + (long)row * p.ldx + col, pp);
      const float D = p.rowv[z1 * p.r_s1 + z2 * p.r_s2 + row];
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = (col + e <= row) ? p.alpha * pp[e] * (v[e] - D) : 0.0f;
    }
    storev<TO, V>(static_cast<TO*>(p.C) + z1 * p.c_s1 + z2 * p.c_s2 + (long)row * p.ldc + col, v);
  }
}

// ---------------------------------------------------------------------------
// instruction interleaving hints (sched_group_barrier masks: 0x008 MFMA,
// 0x020 global read, 0x100 LDS read, 0x200 LDS write)
// ---------------------------------------------------------------------------

template <int N, int MASK>
__device__ __forceinline__ void sched_pairs() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(MASK, 1, 0);
    sched_pairs<N - 1, MASK>();
  }
}

// One sub-step of MF MFMAs: RD fragment reads, then OT ops of kind OMASK,
// each paired with one MFMA; the remaining MFMAs back to back.
template <int MF, int RD, int OT, int OMASK>
__device__ __forceinline__ void sched_substep() {
  constexpr int r = RD < MF ? RD : MF;
  constexpr int o = OT < MF - r ? OT : MF - r;
  sched_pairs<r, 0x100>();
  sched_pairs<o, OMASK>();
  if constexpr (MF - r - o > 0) __builtin_amdgcn_sched_group_barrier(0x008, MF - r - o, 0);
}

// ---------------------------------------------------------------------------
// tile scheduling
// ---------------------------------------------------------------------------

__device__ __forceinline__ void tile_coords(const GemmArgs& p, int& tm, int& tn, int L) {
  if (p.tri) {
    int m = (int)((sqrtf(8.0f * (float)L + 1.0f) - 1.0f) * 0.5f);
    while ((m + 1) * (m + 2) / 2 <= L) ++m;
    while (m * (m + 1) / 2 > L) --m;
    tm = m;
    tn = L - m * (m + 1) / 2;
    return;
  }
  if (p.no_xcd == 2 && L >= p.skm_base) {
    // stream-K tile j: XCD x's runs cover tiles [x n, (x + 1) n), n = br bc,
    // placed as one br x bc block; tile i = q k + d of the block belongs to
    // K-phase group d (the runs that work at the same K offset at the same
    // time), placed as a gr x gc sub-block, so concurrent runs share operand
    // panels in the XCD's L2
    const int j = L - p.skm_base, n = p.skm_br * p.skm_bc;
    const int x = j / n, i = j - (j / n) * n;
    const int k = i / p.skm_q, d = i - (i / p.skm_q) * p.skm_q;
    const int gpr = p.skm_bc / p.skm_gc, bpr = p.tiles_m / p.skm_br;
    tm = (x % bpr) * p.skm_br + (d / gpr) * p.skm_gr + k % p.skm_gr;
    tn = p.skm_col0 + (x / bpr) * p.skm_bc + (d % gpr) * p.skm_gc + k / p.skm_gr;
    return;
  }
  if (p.xcd_br > 0) {
    // block L runs on XCD x = L mod 8 as its i-th block (i = L / 8): XCD x
    // owns the x-th block of the grid, so the operand panels its tiles share
    // stay in its own L2; inside the block, strips of xcd_g tile-rows,
    // column by column
    const int x = L & 7, i = L >> 3;
    const int nbc = p.tiles_n / p.xcd_bc;
    const int per = p.xcd_g * p.xcd_bc, grp = i / per, w = i - grp * per;
    tm = (x / nbc) * p.xcd_br + grp * p.xcd_g + w % p.xcd_g;
    tn = (x % nbc) * p.xcd_bc + w / p.xcd_g;
    return;
  }
  const int tiles = p.tiles_m * p.tiles_n;
  if (!p.no_xcd) {
    // same-XCD runs of tiles: block L runs on XCD x = L mod 8 as its i-th
    // block (i = L / 8); XCD x takes the x-th run of consecutive tiles, runs
    // of q = tiles / 8 tiles plus one for the first tiles mod 8 XCDs
    const int x = L & 7, i = L >> 3, q = tiles >> 3, r = tiles & 7;
    L = x * q + min(x, r) + i;
  }
  const int per_group = p.group_m * p.tiles_n;
  const int grp = L / per_group, first = grp * p.group_m;
  const int gs = min(p.tiles_m - first, p.group_m);
  const int w = L - grp * per_group;
  tm = first + w % gs;
  tn = w / gs;
  if (p.kmode == K_LOWER) tm = p.tiles_m - 1 - tm;  // longest K ranges first
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// ROLE only names the instantiation (one kernel symbol per GEMM of the layer,
// so profilers attribute time per GEMM); it does not change the code.
// KSEG = 3 runs the K loop over (A, B), (A, B2) and (A2, B) in turn.
template <class Cfg, bool AK, bool BKM, int EPI, typename TO, int ROLE, int KSEG = 1, bool TAIL = false,
          bool SCHED = true>
__global__ void __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::NT / 256, Cfg::NT / 256))) gemm_kernel(const GemmArgs p) {
  using T = typename Cfg::T;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT, BK = Cfg::BK;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, WTM = Cfg::WTM, WTN = Cfg::WTN;
  __shared__ uint4 smem[2 * (BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WN, wn = wave - (wave / Cfg::WN) * Cfg::WN;

  int tm, tn;
  tile_coords(p, tm, tn, blockIdx.x);
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.z, z1 = z / p.zdiv, z2 = z - (z / p.zdiv) * p.zdiv;
  const long aoff = z1 * p.a_s1 + z2 * p.a_s2, boff = z1 * p.b_s1 + z2 * p.b_s2;
  const T* A = static_cast<const T*>(p.A) + aoff;
  const T* B = static_cast<const T*>(p.B) + boff;

  using LA = typename LoaderSel<AK, T, BM, NT>::type;
  using LB = typename LoaderSel<BKM, T, BN, NT>::type;
  LA la;
  LB lb;
  la.init(p.lda, m0, p.M, tid);
  lb.init(p.ldb, n0, p.N, tid);

  // K tiles: one run [kb, ke), or KSEG runs of kseg_len over operand pairs
  int kb = 0, ke = p.K, nk, nkd = 1;
  if constexpr (KSEG > 1) {
    nkd = (p.kseg_len + BK - 1) / BK;
    nk = KSEG * nkd;
  } else {
    if (p.kmode == K_LOWER) ke = min(ke, m0 + BM);
    else if (p.kmode == K_UPPER) kb = m0;
    if constexpr (EPI == EPI_PARTIAL) {
      kb = blockIdx.y * p.k_chunk;
      ke = min(ke, kb + p.k_chunk);
    }
    nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;
  }
  // operand origins of K tile kt and the k range left in its run
  auto src = [&](int kt, const T*& a, const T*& b, int& kvalid) {
    if constexpr (KSEG > 1) {
      const int seg = kt / nkd;
      const int k0 = (kt - seg * nkd) * BK;
      kvalid = p.kseg_len - k0;
      a = LA::advance(seg == 2 ? static_cast<const T*>(p.A2) + aoff : A, p.lda, k0);
      b = LB::advance(seg == 1 ? static_cast<const T*>(p.B2) + boff : B, p.ldb, k0);
    } else {
      const int k0 = kb + kt * BK;
      kvalid = ke - k0;
      a = LA::advance(A, p.lda, k0);
      b = LB::advance(B, p.ldb, k0);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Pipeline: while the MFMAs of tile kt run from LDS buffer kt&1, tile kt+1
  // (already in registers) is written to the other buffer and tile kt+2 is
  // fetched from global memory into the registers. Past the last tile the
  // fetches repeat the last tile (in bounds) and the stores go to the idle
  // buffer, so the loop body is one branch-free block. One barrier per tile.
  const int r32 = lane & 31, g = lane >> 5;
  const int arow = (wm * WTM + r32) * 8, brow = (wn * WTN + r32) * 8;
  if (nk > 0) {
    const T *a, *b;
    int kv;
    src(0, a, b, kv);
    la.template load<TAIL>(a, p.lda, kv, tid);
    lb.template load<TAIL>(b, p.ldb, kv, tid);
    la.store(smem, tid);
    lb.store(smem + BM * 8, tid);
    src(min(1, nk - 1), a, b, kv);
    la.template load<TAIL>(a, p.lda, kv, tid);
    lb.template load<TAIL>(b, p.ldb, kv, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const uint4* As = smem + (kt & 1) * (BM + BN) * 8;
    const uint4* Bs = As + BM * 8;
    uint4* An = smem + ((kt + 1) & 1) * (BM + BN) * 8;
    uint4 af[2][TM], bq[2][TN];
    {
      const int ch = g ^ (r32 & 7);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[0][i] = As[arow + i * 32 * 8 + ch];
#pragma unroll
      for (int j = 0; j < TN; ++j) bq[0][j] = Bs[brow + j * 32 * 8 + ch];
    }
    la.store(An, tid);
    lb.store(An + BM * 8, tid);
    {
      const T *a, *b;
      int kv;
      src(min(kt + 2, nk - 1), a, b, kv);
      la.template load<TAIL>(a, p.lda, kv, tid);
      lb.template load<TAIL>(b, p.ldb, kv, tid);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < 4) {
        const int ch = (2 * (ks + 1) + g) ^ (r32 & 7);
#pragma unroll
        for (int i = 0; i < TM; ++i) af[cur ^ 1][i] = As[arow + i * 32 * 8 + ch];
#pragma unroll
        for (int j = 0; j < TN; ++j) bq[cur ^ 1][j] = Bs[brow + j * 32 * 8 + ch];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mma16(bq[cur][j], af[cur][i], acc[i][j], T{});
    }
    if constexpr (SCHED && LA::TOTAL % NT == 0 && LB::TOTAL % NT == 0) {
      // Interleave, one LDS or global op per MFMA: sub-step 0's fragment
      // reads first; in every sub-step the next sub-step's fragment reads;
      // the stores of tile kt+1 in sub-steps 0-1, the global fetches of tile
      // kt+2 (which reuse the store registers) in sub-steps 2-3.
      constexpr int MF = TM * TN * (sizeof(T) == 2 ? 1 : 4);  // MFMAs per sub-step
      constexpr int NRD = TM + TN;
      constexpr int NWR = LA::STORES + LB::STORES;
      constexpr int NLD = LA::LOADS + LB::LOADS;
      __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
      sched_substep<MF, NRD, NWR / 2, 0x200>();
      sched_substep<MF, NRD, NWR - NWR / 2, 0x200>();
      sched_substep<MF, NRD, NLD / 2, 0x020>();
      sched_substep<MF, 0, NLD - NLD / 2, 0x020>();
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = m0 + wm * WTM + i * 32 + r32;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int col = n0 + wn * WTN + j * 32 + jj * 8 + g * 4;
        float v[4] = {acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2], acc[i][j][4 * jj + 3]};
        if (row < p.M && col < p.N) epi_apply<EPI, T, TO>(p, z1, z2, row, col, v, blockIdx.y);
      }
    }
  }
}

// Fixed-order sum of split-K partials followed by the real epilogue (batch 1).
template <int EPI, typename T, typename TO, int ROLE>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const GemmArgs p) {
  const long n4 = p.N / 4;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)p.M * n4) return;
  const int row = (int)(idx / n4), col = (int)(idx - (idx / n4) * n4) * 4;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  // pieces in order, two loads in flight per step
  int s = 0;
  for (; s + 2 <= p.splits; s += 2) {
    float x[4], y[4];
    Elt<float>::load4(p.part + ((long)s * p.M + row) * (long)p.N + col, x);
    Elt<float>::load4(p.part + ((long)(s + 1) * p.M + row) * (long)p.N + col, y);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (v[e] + x[e]) + y[e];
  }
  if (s < p.splits) {
    float x[4];
    Elt<float>::load4(p.part + ((long)s * p.M + row) * (long)p.N + col, x);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += x[e];
  }
  epi_apply<EPI, T, TO>(p, 0, 0, row, col, v, 0);
}

}  // namespace tpl
