// libtplayer: C ABI for one tensor-parallel rank's share of a GPT layer on
// gfx950. Host code validates arguments, lays out the saved activations and
// the workspace, and enqueues the kernels of gemm.hpp / aux_kernels.hpp on
// the caller's stream. The library allocates no device memory; its only
// state is the calling thread's last HIP error text and, while profiling is
// switched on, the HIP events of the profiled launches.
//
// Block flows (rank r; paper-graph page, section 3 "Tensor Model
// Parallelism: The Megatron Partitioning"; "parallelism" blog, "Tensor
// parallelism: split every matrix" and "The backward pass"):
//   ATTN fwd:  QKV = X Wqkv_r + b (GEMM, bias epilogue)
//              S = Q K^T / sqrt(d) per (sequence, head), causal tiles only
//              P = causal softmax(S);  C = P V (causal K range)
//              partial = C Wo_r
//   MLP fwd:   U = H W1_r + b1, Z = GELU(U) (one GEMM, dual-store epilogue)
//              partial = Z W2_r
//   MLP bwd:   dU = (dY W2_r^T) * GELU'(U);  dW2_r = Z^T dY;  db2 = sum dY
//              dH_r = dU W1_r^T;  dW1_r = H^T dU;  db1 = sum dU
//   ATTN bwd:  dC = dH Wo_r^T;  dWo_r = C^T dH;  dbo = sum dH
//              D = rowsum(dC * C);  dS = P * (dC V^T - D) / sqrt(d)
//              dV = P^T dC;  dQ = dS K;  dK = dS^T Q   (written into dQKV)
//              dX_r = dQKV Wqkv_r^T;  dWqkv_r = X^T dQKV;  db_qkv = sum dQKV
// The replicated output bias and the residual (and the residual gradient)
// are added after the all-reduce, by tp_reduce_partials (paper-graph page,
// "Computation Optimizations": bias + dropout + residual add, fused).

#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <cmath>
#include <mutex>
#include <type_traits>
#include <vector>

#include "tp_layer.h"
#include "aux_kernels.hpp"
#include "gemm.hpp"
#include "flash_attn.hpp"
#include "gemm_direct.hpp"
#include "layernorm.hpp"

using namespace tpl;

namespace {

thread_local char g_hip_err[256] = "";

int hip_fail(hipError_t e) {
  snprintf(g_hip_err, sizeof(g_hip_err), "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return TP_EHIP;
}

// ---------------------------------------------------------------------------
// kernel roles (one kernel symbol per GEMM of the layer) and profiling
// ---------------------------------------------------------------------------

enum Role : int {
  R_QKV_FWD, R_SCORES, R_SOFTMAX, R_PV, R_O_FWD, R_FC1_FWD, R_FC2_FWD,
  R_FC2_DGRAD, R_FC2_WGRAD, R_DB2, R_FC1_DGRAD, R_FC1_WGRAD, R_DB1,
  R_O_DGRAD, R_O_WGRAD, R_DBO, R_ROWDOT, R_DS, R_DV, R_DQ, R_DK,
  R_QKV_DGRAD, R_QKV_WGRAD, R_DBQKV, R_REDUCE, R_GEMM,
  R_FC2_BWD, R_FC1_BWD, R_O_BWD, R_QKV_BWD, R_ATT_FWD, R_ATT_DKV, R_ATT_DQ, R_LN_FWD, R_LN_BWD, R_COUNT
};

const char* const kRoleName[R_COUNT] = {
  "qkv_fwd", "scores", "softmax", "pv", "o_fwd", "fc1_fwd", "fc2_fwd",
  "fc2_dgrad", "fc2_wgrad", "db2", "fc1_dgrad", "fc1_wgrad", "db1",
  "o_dgrad", "o_wgrad", "dbo", "rowdot", "ds", "dv", "dq", "dk",
  "qkv_dgrad", "qkv_wgrad", "dbqkv", "reduce", "gemm",
  "fc2_dgrad+wgrad", "fc1_dgrad+wgrad", "o_dgrad+wgrad", "qkv_dgrad+wgrad",
  "attn_fwd", "attn_dkv", "attn_dq", "ln_fwd", "ln_bwd"};

namespace prof {
struct Rec {
  int role;
  hipEvent_t a, b;
  double flops, bytes;
};
std::atomic<bool> on{false};
// set for the duration of a tp_layer_bwd_noalloc call: no events are created
// or recorded, so that call makes no allocating runtime call even while
// profiling is on
thread_local bool suppressed = false;
std::mutex mu;
std::vector<Rec> recs;
std::vector<hipEvent_t> pool;

hipEvent_t take() {
  {
    std::lock_guard<std::mutex> g(mu);
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records a start event now and a stop event when it goes out of scope,
// around the kernels enqueued in between (only while profiling is on).
struct Scope {
  int role;
  double flops, bytes;
  hipStream_t st;
  hipEvent_t a = nullptr;
  Scope(int r, double f, double by, hipStream_t s) : role(r), flops(f), bytes(by), st(s) {
    if (on.load(std::memory_order_relaxed) && !suppressed) {
      a = take();
      if (a) (void)hipEventRecord(a, st);
    }
  }
  ~Scope() {
    if (!a) return;
    hipEvent_t b = take();
    if (!b) return;
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> g(mu);
    recs.push_back({role, a, b, flops, bytes});
  }
};
}  // namespace prof

// ---------------------------------------------------------------------------
// dimensions and buffer layout
// ---------------------------------------------------------------------------

struct Dims {
  long h, a, s, b, t;
  int dt;
  long T, d, ar, hr, fr, q3, z;
  size_t es;
};

// Largest matrix (elements) a kernel may address: byte offsets of bf16
// operands from their origin stay below 2^32.
constexpr long kMaxElems = 1L << 31;

int check_args(long h, long a, long s, long b, long t, long rank, int dt, int blk) {
  if (h <= 0 || a <= 0 || s <= 0 || b <= 0 || t <= 0) return TP_EINVAL;
  if (dt != TP_BF16 && dt != TP_FP32) return TP_EINVAL;
  if (blk != TP_ATTN && blk != TP_MLP) return TP_EINVAL;
  if (rank < 0 || rank >= t) return TP_EINVAL;
  if (h % a != 0 || a % t != 0) return TP_EINVAL;  // heads stay whole on a rank
  const long d = h / a, hr = h / t;
  if (s % 16 != 0 || d % 16 != 0 || hr % 16 != 0) return TP_EUNSUPPORTED;
  // rows and columns are 32-bit in the kernels; batch counts fit a grid dimension
  if (s * b > (1L << 30) || 4 * h > (1L << 30) || b * (a / t) > 65535) return TP_EUNSUPPORTED;
  // The tile loaders address an operand with 32-bit byte offsets from its
  // origin, so every matrix the layer reads or writes holds fewer than 2^31
  // elements: activations [T, h] and [T, 4h/t], weight shards up to
  // [h, 4h/t], and on the materialised attention path (fp32, or head widths
  // the fused kernels are not built for) one sequence's [s, s] matrix.
  const long T = s * b, fr = 4 * h / t;
  if (T * h >= kMaxElems || T * fr >= kMaxElems || h * fr >= kMaxElems) return TP_EUNSUPPORTED;
  const bool fused = dt == TP_BF16 && (d == 64 || d == 96 || d == 128 || d == 160);
  if (!fused && s * s >= kMaxElems) return TP_EUNSUPPORTED;
  return TP_OK;
}

Dims make_dims(long h, long a, long s, long b, long t, int dt) {
  Dims D;
  D.h = h; D.a = a; D.s = s; D.b = b; D.t = t; D.dt = dt;
  D.T = s * b; D.d = h / a; D.ar = a / t; D.hr = h / t; D.fr = 4 * h / t; D.q3 = 3 * h / t;
  D.z = b * D.ar;
  D.es = dt == TP_BF16 ? 2 : 4;
  return D;
}

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// Tile configurations.
using CfgBig = TileCfg<bf16_t, 256, 256, 2, 2>;  // linear GEMMs
using CfgB192 = TileCfg<bf16_t, 192, 256, 2, 4>;  // linear GEMMs of one partial wave (8 waves: 2 per SIMD)
using CfgN192 = TileCfg<bf16_t, 256, 192, 2, 2>;  // linear GEMMs that 192-column tiles fill in whole waves
using CfgHalf = TileCfg<bf16_t, 256, 128, 2, 2>;              // the columns past whole waves
using CfgMid = TileCfg<bf16_t, 128, 128, 2, 2>;  // attention products
using CfgF32 = TileCfg<float, 64, 64, 2, 2>;     // fp32 configuration

// Split-K for GEMMs with too few output tiles to fill half of the 256 CUs.
// From 128 tiles on, one partial wave of whole tiles is faster: the busy
// CUs run at a higher clock and share operand panels in L2, while split or
// stream-K pieces add fp32 partial traffic and a reduction.
int choose_splits(long M, long N, long K) {
  const long tiles = cdivl(M, CfgBig::BM) * cdivl(N, CfgBig::BN);
  if (tiles >= 128 || K < 2048) return 1;
  long s = (256 + tiles / 2) / tiles;
  s = std::min(s, K / 1024);
  if (s < 2) return 1;
  const long chunk = cdivl(cdivl(K, s), CfgBig::BK) * CfgBig::BK;
  return (int)cdivl(K, chunk);
}

// Causal [s, s] matrices (scores, P, dS) are defined up to the next multiple
// of the attention tile in every row; all causal GEMMs use this tile.
int att_tile(int dt) { return dt == TP_BF16 ? CfgMid::BM : CfgF32::BM; }

// The bf16 path runs attention as fused flash kernels (flash_attn.hpp) for
// the head widths they are built for; other widths and the fp32
// configuration materialise the causal s x s matrices with the GEMM kernels.
bool flash(const Dims& D) {
  if (D.dt != TP_BF16) return false;
  // (check_args keeps [T, 3h/t] below 2^31 elements, as the tile loads' 32-bit
  // byte offsets need)
  return D.d == 64 || D.d == 96 || D.d == 128 || D.d == 160;
}

// Flash attention chunk size for blocks of bq rows when `slots` workgroups
// run on the chip at once: when the heads' blocks alone keep them busy twice
// over, blocks run whole; otherwise their tile ranges are cut into chunks of
// 8 tiles (the causal ranges differ up to s / 64 : 1 in length) and merged by
// a combine kernel. (8 is a multiple of bq / 64, so every query row sees the
// first key of each chunk of its block.)
int fa_chunk_tiles(const Dims& D, int bq, long slots) {
  const long nblk = cdivl(D.s, bq), ntot = cdivl(D.s, fa::BT);
  if (D.z * nblk >= 2 * slots) return (int)(ntot + (ntot & 1));
  return 8;
}
// Backward kernels: 128-row blocks; dK/dV one workgroup per CU, dQ two.
int fa_chunk_tiles(const Dims& D) { return fa_chunk_tiles(D, fa::BQ, 2 * 256); }
// Forward: 256-query blocks of 8 waves (one workgroup per CU) for d <= 128,
// 128-query blocks of 4 waves for d = 160.
int fa_fwd_bq(const Dims& D) { return D.d <= 128 ? fa::BQF : fa::BQ; }
int fa_fwd_chunk_tiles(const Dims& D) { return fa_chunk_tiles(D, fa_fwd_bq(D), 256); }
// fp32 partials of split blocks: forward C (+ m, l per row) or backward dK, dV
// (the dQ partials reuse the region after the dK/dV combine).
size_t fa_part_bytes(const Dims& D, int blk) {
  if (blk != TP_ATTN) return 0;
  // z x blocks x chunks x rows per block
  const size_t fs = (size_t)fa::part_slot((int)D.z, 0, 0, (int)D.s, fa_fwd_chunk_tiles(D), 1, fa_fwd_bq(D));
  const size_t bs = (size_t)fa::part_slot((int)D.z, 0, 0, (int)D.s, fa_chunk_tiles(D), 1);
  return 4 * std::max<size_t>(fs * (D.d + 2), bs * 2 * D.d);
}

// ATTN keeps QKV, P and C (and, for bf16, C in fp32 for the softmax
// backward's row term), or with the flash kernels QKV, the Q/K residuals,
// C (bf16 and fp32) and the per-query log-sum-exp; MLP keeps U and Z.
struct SavedLayout {
  size_t qkv, qkv_lo, lse, p, c, c32, u, z, total;
};
SavedLayout saved_layout(const Dims& D, int blk) {
  SavedLayout L{};
  size_t o = 0;
  if (blk == TP_ATTN && flash(D)) {  // QKV, the Q/K rounding residuals, C (bf16, fp32), LSE
    L.qkv = o;    o = al(o + (size_t)D.T * D.q3 * D.es);
    L.qkv_lo = o; o = al(o + (size_t)D.T * 2 * D.hr * D.es);
    L.c = o;      o = al(o + (size_t)D.T * D.hr * D.es);
    L.c32 = o;    o = al(o + (size_t)D.T * D.hr * 4);
    L.lse = o;    o = al(o + (size_t)D.z * D.s * 4);
  } else if (blk == TP_ATTN) {
    L.qkv = o; o = al(o + (size_t)D.T * D.q3 * D.es);
    L.p = o;   o = al(o + (size_t)D.z * D.s * D.s * D.es);
    L.c = o;   o = al(o + (size_t)D.T * D.hr * D.es);
    if (D.dt == TP_BF16) {
      L.c32 = o; o = al(o + (size_t)D.T * D.hr * 4);
    } else {
      L.c32 = L.c;
    }
  } else {
    L.u = o; o = al(o + (size_t)D.T * D.fr * D.es);
    L.z = o; o = al(o + (size_t)D.T * D.fr * D.es);
  }
  L.total = o;
  return L;
}

// Fewest tiles for which stream-K over a lone partial wave pays.
constexpr long kSkMinTiles = 160;
// Stream-K plan for a bf16 GEMM on 256x256 tiles with whole 64-deep K steps
// (units = 0: not worth it). Whole waves of tiles run as they are; the last,
// partial wave's K iterations are spread over all 256 CUs. Without a whole
// wave in front, the pieces start at staggered K offsets, so no two CUs of
// an XCD share an operand slice in L2 and every piece's panels come from
// beyond L2 (measured: 10x the operand bytes for a 144-tile GEMM); below
// kSkMinTiles tiles a partial wave of whole tiles wins instead. Chosen when the
// modelled time beats the plain (or split-K) launch; the model counts one
// tile-iteration as ~1.95 us and charges the fp32 fragments' write + read at
// ~5 TB/s plus a launch gap for the fix-up.
SkPlan sk_plan(long M, long N, long K) {
  SkPlan s{};
  if (K % CfgBig::BK != 0 || N % 8 != 0) return s;
  const long tiles = cdivl(M, CfgBig::BM) * cdivl(N, CfgBig::BN);
  const long I = K / CfgBig::BK;
  const long W = tiles / 256, R = tiles % 256;
  if (R == 0 || I < 8) return s;
  if (W == 0 && tiles < kSkMinTiles) return s;  // too few tiles: a partial wave of whole tiles
  const double t_it = 1.95e-6, frag = 4.0 * CfgBig::BM * CfgBig::BN;
  double plain = (double)cdivl(tiles, 256) * I * t_it;
  const int sp = choose_splits(M, N, K);
  if (sp > 1) {
    const long chunk = cdivl(I, sp);
    plain = (double)cdivl(tiles * sp, 256) * chunk * t_it + 2.0 * sp * M * N * 4.0 / 5e12 + 5e-6;
  }
  const long c = cdivl(R * I, 256);
  const double sk = (double)(W * I + c) * t_it + 2.0 * (256 + R) * frag / 5e12 + 5e-6;
  if (sk >= 0.97 * plain) return s;
  s.dp_tiles = (int)(W * 256);
  s.sk_tiles = (int)R;
  s.iters = (int)I;
  s.c = (int)c;
  s.units = 256;
  int f = 1;
  for (long j = 0; j < R; ++j) f = std::max<int>(f, (int)(((j + 1) * I - 1) / c - (j * I) / c + 1));
  s.f = f;
  return s;
}


// Placement of a stream-K region's tiles (GemmArgs skm_*; no_xcd = 2) when
// every XCD's 32 runs cover whole tiles and the region is whole tile-columns
// of at most 8 tile-rows (one ordering group, so the whole tiles before it
// are the columns before it): the XCD's tiles as one compact block, and the
// tiles its runs work on at the same K offset (a period of q tiles) as
// compact sub-blocks. 175B FC1 forward: 2 x 12 blocks, 3 groups of 2 x 4.
void sk_place(GemmArgs& p, const SkPlan& s) {
  const long per = (long)(s.units / 8) * s.c;
  if (s.units % 8 || per % s.iters || p.tiles_m > 8 || s.sk_tiles % p.tiles_m || s.dp_tiles % p.tiles_m) return;
  const int n = (int)(per / s.iters), cols = s.sk_tiles / p.tiles_m;
  long g = s.c, b = s.iters;
  while (b) { const long r = g % b; g = b; b = r; }
  const int q = (int)(s.c / g);
  if (n % q) return;
  const int m = n / q;  // tiles of one K-phase group
  int best = 1 << 30;
  for (int br = 1; br <= p.tiles_m; ++br) {
    if (p.tiles_m % br || n % br) continue;
    const int bc = n / br;
    if (cols % bc || (p.tiles_m / br) * (cols / bc) != 8) continue;
    for (int gr = 1; gr <= br; ++gr) {
      if (br % gr || m % gr) continue;
      const int gc = m / gr;
      if (bc % gc || (br / gr) * (bc / gc) != q || gr + gc >= best) continue;
      best = gr + gc;
      p.no_xcd = 2;
      p.skm_base = s.dp_tiles;
      p.skm_col0 = s.dp_tiles / p.tiles_m;
      p.skm_br = br; p.skm_bc = bc; p.skm_q = q; p.skm_gr = gr; p.skm_gc = gc;
    }
  }
}

size_t partial_bytes(const Dims& D, long M, long N, long K) {
  if (D.dt != TP_BF16) return 0;
  const int sp = choose_splits(M, N, K);
  size_t b = sp > 1 ? al((size_t)sp * M * N * 4) : 0;
  const SkPlan s = sk_plan(M, N, K);
  if (s.units) b = std::max(b, al((size_t)s.sk_tiles * s.f * CfgBig::BM * CfgBig::BN * 4));
  return b;
}

// Grouped launch of two GEMMs (M0 x N0 x K0 first, M1 x N1 x K1 second):
// problem 0 may be split along K so that its pieces and problem 1's tiles
// fill the 256 CUs together. The dispatcher hands the blocks out in order
// (the problem with the longer units first) to whichever CU frees first; the
// plan simulates exactly that for each split count and takes the fastest,
// counting a per-unit epilogue cost and, for a split, the HBM traffic of the
// fp32 partials (written by the pieces, read back by the reduction, which
// also writes the result). Returns the split count and its chunk (a multiple
// of BK).
struct PairPlan {
  int splits;
  long chunk;
};

// Finish time of handing n1 units of length l1, then n2 of length l2, in
// order, each to whichever of the 256 CUs frees first. CUs free at the same
// time are kept as one bucket, so a step places a whole batch of units.
double dispatch_makespan(long n1, double l1, long n2, double l2) {
  std::map<double, long> free_at{{0.0, 256}};
  auto place = [&](long n, double len) {
    while (n > 0) {
      auto it = free_at.begin();
      const double t = it->first;
      const long k = std::min(it->second, n);
      if (k == it->second) free_at.erase(it);
      else it->second -= k;
      free_at[t + len] += k;
      n -= k;
    }
  };
  place(n1, l1);
  place(n2, l2);
  return free_at.rbegin()->first;
}

PairPlan pair_plan(long M0, long N0, long K0, long M1, long N1, long K1, bool gelu0 = false) {
  const long t0 = cdivl(M0, CfgBig::BM) * cdivl(N0, CfgBig::BN);
  const long t1 = cdivl(M1, CfgBig::BM) * cdivl(N1, CfgBig::BN);
  const long it0 = cdivl(K0, CfgBig::BK), it1 = cdivl(K1, CfgBig::BK);
  const double t_it = 1.6e-6;                   // one K step of a 256 x 256 tile, all CUs busy
  const double epi = 2.0, epi_part = 3.0;       // epilogue in K steps: bf16 tile, fp32 partial tile
  PairPlan best{1, K0};
  double best_t = 0.0, whole_t = 0.0;
  const long max_sp = K0 % CfgBig::BK == 0 ? std::min<long>(16, it0 / 8) : 1;
  for (long sp = 1; sp <= std::max<long>(1, max_sp); ++sp) {
    const long chunk = cdivl(it0, sp);
    if (cdivl(it0, chunk) != sp) continue;  // the same split as a smaller count
    const double l0 = (double)chunk + (sp > 1 ? epi_part : epi), l1 = (double)it1 + epi;
    const double span = l0 >= l1 ? dispatch_makespan(t0 * sp, l0, t1, l1) : dispatch_makespan(t1, l1, t0 * sp, l0);
    double t = span * t_it;
    if (sp > 1) t += (double)M0 * N0 * (8.0 * sp + 2.0 + (gelu0 ? 2.0 : 0.0)) / 4.5e12 + 4e-6;  // partials
    if (sp == 1) whole_t = best_t = t;
    // a split must win clearly: its partials also evict cached operands that
    // the kernels after it would read again
    else if (t < best_t && t < 0.97 * whole_t) {
      best_t = t;
      best = PairPlan{(int)sp, chunk * CfgBig::BK};
    }
  }
  return best;
}
size_t pair_partial_bytes(const Dims& D, long M0, long N0, long K0, long M1, long N1, long K1, bool gelu0) {
  if (D.dt != TP_BF16) return 0;
  const PairPlan P = pair_plan(M0, N0, K0, M1, N1, K1, gelu0);
  return P.splits > 1 ? al((size_t)P.splits * M0 * N0 * 4) : 0;
}

struct WsLayout {
  size_t s, qkv_lo;         // attn fwd: fp32 scores, bf16 residuals of Q and K
  size_t dc, D, ds, dqkv;   // attn bwd
  size_t du;                // mlp bwd
  size_t part, part_bytes;  // split-K partials
  size_t total;
};
WsLayout ws_layout(const Dims& D, int blk) {
  WsLayout W{};
  size_t pb = 0;
  auto upd = [&](long M, long N, long K) { pb = std::max(pb, partial_bytes(D, M, N, K)); };
  // input- and weight-gradient GEMMs of one weight, grouped
  auto upd2 = [&](long M0, long N0, long K0, long M1, long N1, long K1, bool gelu0) {
    upd(M0, N0, K0);
    upd(M1, N1, K1);
    pb = std::max(pb, pair_partial_bytes(D, M0, N0, K0, M1, N1, K1, gelu0));
  };
  // the flash attention chunks share the partials region (every user runs in
  // turn on the stream)
  if (flash(D)) pb = std::max(pb, al(fa_part_bytes(D, blk)));
  if (blk == TP_ATTN) {
    upd(D.T, D.q3, D.h); upd(D.T, D.h, D.hr);
    upd2(D.T, D.hr, D.h, D.hr, D.h, D.T, false); upd2(D.T, D.h, D.q3, D.h, D.q3, D.T, false);
    const bool fl = flash(D);
    size_t fwd = fl ? 0 : al((size_t)D.z * D.s * D.s * 4);
    W.qkv_lo = fwd;
    if (D.dt == TP_BF16 && !fl) fwd = al(fwd + (size_t)D.T * D.q3 * D.es);
    size_t o = 0;
    W.dc = o;   o = al(o + (size_t)D.T * D.hr * D.es);
    W.D = o;    o = al(o + (size_t)D.z * D.s * 4);
    W.ds = o;   if (!fl) o = al(o + (size_t)D.z * D.s * D.s * D.es);
    W.dqkv = o; o = al(o + (size_t)D.T * D.q3 * D.es);
    W.s = 0;
    W.part = std::max(fwd, o);
  } else {
    upd(D.T, D.fr, D.h); upd(D.T, D.h, D.fr);
    upd2(D.T, D.fr, D.h, D.fr, D.h, D.T, true); upd2(D.T, D.h, D.fr, D.h, D.fr, D.T, false);
    W.du = 0;
    W.part = al((size_t)D.T * D.fr * D.es);
  }
  W.part_bytes = pb;
  W.total = W.part + pb;
  return W;
}

// ---------------------------------------------------------------------------
// GEMM dispatch
// ---------------------------------------------------------------------------

enum Kind { KIND_BIG = 0, KIND_MID = 1 };

// Does any K run of this GEMM end inside a K tile? (Then the kernel variant
// that zero-fills k beyond the run is needed.) Runs start at 0, at m0 (a
// multiple of BM, itself a multiple of BK), or at split-K chunk boundaries
// (multiples of BK), and end at K, m0 + BM, a chunk boundary, or kseg_len.
template <class Cfg>
bool ragged_k(const GemmArgs& p, int kseg) {
  if (kseg > 1) return p.kseg_len % Cfg::BK != 0;
  return p.K % Cfg::BK != 0;
}

// The direct kernel needs whole K tiles and writes its epilogue in 8-column
// pieces (N, ldc and the other column strides multiples of 8).
template <class Cfg>
bool direct_ok(const GemmArgs& p, int kseg) {
  return !ragged_k<Cfg>(p, kseg) && p.N % 8 == 0;
}

template <class Cfg, bool AK, bool BKM, int EPI, typename TO, int ROLE, int KSEG = 1>
hipError_t launch(GemmArgs p, int batch, hipStream_t st) {
  p.tiles_m = cdiv(p.M, Cfg::BM);
  p.tiles_n = cdiv(p.N, Cfg::BN);
  if (p.group_m <= 0) p.group_m = 8;
  if (p.zdiv <= 0) p.zdiv = 1;
  const int tiles = p.tri ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
  if (tiles == 0 || batch == 0) return hipSuccess;
  // bf16 tiles with whole 64-deep K steps take the direct global->LDS kernel
  constexpr bool BF = sizeof(typename Cfg::T) == 2;
  if constexpr (EPI != EPI_SOFTMAX_BWD && KSEG == 1) {
    if (p.splits > 1) {
      p.k_chunk = (int)(cdivl(cdivl(p.K, p.splits), Cfg::BK) * Cfg::BK);
      const dim3 grid(tiles, p.splits, 1);
      bool done = false;
      if constexpr (BF) {
        if (direct_ok<Cfg>(p, 1)) {
          hipLaunchKernelGGL((gemm_direct_kernel<Cfg, AK, BKM, EPI_PARTIAL, float, ROLE, 1>), grid, dim3(Cfg::NT), 0,
                             st, p);
          done = true;
        }
      }
      if (done) {
      } else if (ragged_k<Cfg>(p, 1))
        hipLaunchKernelGGL((gemm_kernel<Cfg, AK, BKM, EPI_PARTIAL, float, ROLE, 1, true>), grid, dim3(Cfg::NT), 0,
                           st, p);
      else
        hipLaunchKernelGGL((gemm_kernel<Cfg, AK, BKM, EPI_PARTIAL, float, ROLE, 1, false>), grid, dim3(Cfg::NT), 0,
                           st, p);
      const long n4 = (long)p.M * p.N / 4;
      hipLaunchKernelGGL((splitk_reduce_kernel<EPI, typename Cfg::T, TO, ROLE>), dim3((unsigned)cdivl(n4, 256)),
                         dim3(256), 0, st, p);
      return hipGetLastError();
    }
  }
  const dim3 grid(tiles, 1, batch);
  if constexpr (BF) {
    if (direct_ok<Cfg>(p, KSEG)) {
      hipLaunchKernelGGL((gemm_direct_kernel<Cfg, AK, BKM, EPI, TO, ROLE, KSEG>), grid, dim3(Cfg::NT), 0, st, p);
      return hipGetLastError();
    }
  }
  if (ragged_k<Cfg>(p, KSEG))
    hipLaunchKernelGGL((gemm_kernel<Cfg, AK, BKM, EPI, TO, ROLE, KSEG, true>), grid, dim3(Cfg::NT), 0, st, p);
  else
    hipLaunchKernelGGL((gemm_kernel<Cfg, AK, BKM, EPI, TO, ROLE, KSEG, false>), grid, dim3(Cfg::NT), 0, st, p);
  return hipGetLastError();
}

// One GEMM call site of the layer: fixed operand layout, epilogue and role;
// the element type comes from the call's dtype.
template <bool AK, bool BKM, int EPI, int ROLE, int KIND, bool OUTF32 = false, int KSEG = 1>
hipError_t run(const Dims& D, GemmArgs p, int batch, hipStream_t st) {
  if (D.dt == TP_FP32) {
    if constexpr (EPI == EPI_BIAS_SPLIT || EPI == EPI_DUAL_F32 || KSEG != 1) {
      return hipErrorInvalidValue;  // bf16-only variants
    } else {
      p.splits = 1;
      return launch<CfgF32, AK, BKM, EPI, float, 0>(p, batch, st);
    }
  }
  if constexpr (KIND == KIND_BIG) {
    return launch<CfgBig, AK, BKM, EPI, bf16_t, ROLE>(p, batch, st);
  } else {
    p.splits = 1;
    return launch<CfgMid, AK, BKM, EPI, std::conditional_t<OUTF32, float, bf16_t>, ROLE, KSEG>(p, batch, st);
  }
}

GemmArgs gargs(long M, long N, long K) {
  GemmArgs p;
  memset(&p, 0, sizeof(p));
  p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.zdiv = 1; p.alpha = 1.0f; p.splits = 1; p.group_m = 8;
  return p;
}

#define TRY_E(x)                     \
  do {                               \
    hipError_t e_ = (x);             \
    if (e_ != hipSuccess) return e_; \
  } while (0)

// A launch of whole 256 x 256 tiles that leaves CUs idle (fewer tiles than
// CUs) spreads the same work over more CUs with 192-row tiles when those
// still fit one wave: 175B QKV 144 -> 198 tiles. The shorter tile does 3/4
// of the work at about 0.82 of the 256-row tile's rate, so this pays when
// it adds more than a few tiles.
bool tall_tiles_pay(const GemmArgs& p) {
  const long t256 = cdivl(p.M, 256) * cdivl(p.N, 256), t192 = cdivl(p.M, 192) * cdivl(p.N, 256);
  return direct_ok<CfgB192>(p, 1) && t256 < 256 && t192 <= 256 && (double)t192 >= 1.15 * (double)t256;
}

// Columns of a whole-tile launch that fill whole waves of 256 CUs with
// 256 x 256 tiles when the other tiles (at most half a wave) would run as a
// partial wave. Those remaining columns then run as 256 x 128 tiles, twice as
// many, which still fit one wave and take about half as long: 175B O
// projection, 384 tiles = 1.5 waves -> 256 tiles, then 256 half tiles.
// 0 when the split does not apply.
long whole_wave_cols(const GemmArgs& p) {
  const long tm = cdivl(p.M, 256), tn = cdivl(p.N, 256), tiles = tm * tn;
  const long W = tiles / 256, R = tiles % 256;
  if (W < 1 || R == 0 || R > 128 || (256 * W) % tm != 0) return 0;
  const long n1 = 256 * (256 * W / tm);
  if (n1 >= p.N || (p.N - n1) % 8 != 0) return 0;
  return n1;
}

// 256 x 192 tiles, when they fill one or two whole waves of the 256 CUs and
// 256 x 256 tiles do not (a partial last wave, or stream-K fragments and a
// fix-up). With more waves the stream-K plan of 256 x 256 tiles is faster
// (a 256 x 192 K step costs ~0.9 of a 256 x 256 one for 0.75 of its work).
bool n192_fills(const GemmArgs& p) {
  const long t256 = cdivl(p.M, 256) * cdivl(p.N, 256), t192 = cdivl(p.M, 256) * cdivl(p.N, 192);
  return p.N % 192 == 0 && p.K % 64 == 0 && !p.resid && t256 % 256 != 0 && t192 % 256 == 0 && t192 <= 512;
}

// Linear (weight) GEMM M x N x K: split-K chosen for the bf16 path.
template <bool AK, bool BKM, int EPI, int ROLE>
hipError_t linear(const Dims& D, GemmArgs p, float* part, hipStream_t st) {
  const double extra = (EPI == EPI_BIAS_GELU || EPI == EPI_GELU_BWD || p.resid) ? 1.0 : 0.0;
  prof::Scope sc(ROLE, 2.0 * p.M * p.N * p.K,
                 (double)D.es * ((double)p.M * p.K + (double)p.K * p.N + (1.0 + extra) * p.M * p.N), st);
  if (D.dt == TP_BF16) {
    if constexpr (AK && !BKM && (EPI == EPI_LINEAR || EPI == EPI_BIAS_GELU)) {
      if (n192_fills(p)) {
        p.tiles_m = cdiv(p.M, CfgN192::BM);
        p.tiles_n = cdiv(p.N, CfgN192::BN);
        if (p.group_m <= 0) p.group_m = 8;
        if (p.zdiv <= 0) p.zdiv = 1;
        p.splits = 1;
        hipLaunchKernelGGL((gemm_direct_kernel<CfgN192, AK, BKM, EPI, bf16_t, ROLE, 1>),
                           dim3(p.tiles_m * p.tiles_n, 1, 1), dim3(CfgN192::NT), 0, st, p);
        return hipGetLastError();
      }
    }
    SkPlan s = sk_plan(p.M, p.N, p.K);
    if (s.units) {
      s.part = part;
      p.tiles_m = cdiv(p.M, CfgBig::BM);
      p.tiles_n = cdiv(p.N, CfgBig::BN);
      p.group_m = 8;
      p.no_xcd = 1;
      sk_place(p, s);
      p.splits = 1;
      hipLaunchKernelGGL((gemm_sk_kernel<CfgBig, AK, BKM, EPI, bf16_t, ROLE>), dim3(s.dp_tiles + s.units),
                         dim3(CfgBig::NT), 0, st, p, s);
      hipLaunchKernelGGL((sk_fixup_kernel<CfgBig, EPI, bf16_t, ROLE>),
                         dim3(CfgBig::BM * CfgBig::BN / 8 / 256, s.sk_tiles), dim3(256), 0, st, p, s);
      return hipGetLastError();
    }
    p.splits = choose_splits(p.M, p.N, p.K);
    p.part = part;
    // (the M-contiguous A loader is laid out for 256-row tiles only)
    if constexpr (AK && (ROLE == R_QKV_FWD || ROLE == R_O_FWD || ROLE == R_FC1_FWD || ROLE == R_FC2_FWD ||
                         ROLE == R_GEMM)) {
      if (p.splits == 1 && tall_tiles_pay(p)) return launch<CfgB192, AK, BKM, EPI, bf16_t, ROLE>(p, 1, st);
    }
    if constexpr (EPI == EPI_LINEAR && (ROLE == R_O_FWD || ROLE == R_FC2_FWD || ROLE == R_GEMM)) {
      const long n1 = (p.splits == 1 && !p.resid && direct_ok<CfgBig>(p, 1)) ? whole_wave_cols(p) : 0;
      if (n1 > 0) {
        GemmArgs a = p;
        a.N = (int)n1;
        TRY_E((launch<CfgBig, AK, BKM, EPI, bf16_t, ROLE>(a, 1, st)));
        GemmArgs b = p;
        b.N = p.N - (int)n1;
        b.B = static_cast<const bf16_t*>(p.B) + (BKM ? n1 * p.ldb : n1);
        b.C = static_cast<bf16_t*>(p.C) + n1;
        if (p.bias) b.bias = static_cast<const bf16_t*>(p.bias) + n1;
        return launch<CfgHalf, AK, BKM, EPI, bf16_t, ROLE>(b, 1, st);
      }
    }
  }
  return run<AK, BKM, EPI, ROLE, KIND_BIG>(D, p, 1, st);
}

// One block of tiles per XCD (GemmArgs xcd_*): when the tile grid splits into
// 8 equal blocks, the split with the shortest block perimeter (the fewest
// operand panels per XCD), walked in strips of g tile-rows (g dividing the
// block's rows). Used for the weight-gradient problem of the grouped
// backward launches, whose K = T tiles are many and short: an XCD's tiles
// then share their operand panels in its own L2, which cuts the launch's
// counter traffic at the same or slightly better speed. (For the
// input-gradient problem, long-K tiles that start together, the plain runs
// of tile-rows measured faster.)
constexpr int kXcdStrip = 4;
void xcd_blocks(GemmArgs& p, int g) {
  int best = 1 << 30;
  for (int nr = 1; nr <= 8; nr *= 2) {
    const int nc = 8 / nr;
    if (p.tiles_m % nr || p.tiles_n % nc) continue;
    const int br = p.tiles_m / nr, bc = p.tiles_n / nc;
    if (br % std::min(g, br) || br + bc >= best) continue;
    best = br + bc;
    p.xcd_br = br;
    p.xcd_bc = bc;
    p.xcd_g = std::min(g, br);
  }
}

// A block's input-gradient GEMM (problem 0: dY W^T, K-contiguous operands,
// epilogue E0) and weight-gradient GEMM (problem 1: X^T dY) in one launch
// when both run on the direct bf16 kernel; otherwise two launches.
// Attention backward: D = rowsum(dC * C) may ride on the split-K sum of dC.
struct RowdotFuse {
  const float* C;  // fp32 context [T, hr]
  float* D;        // [b, a_r, s]
};

// csum (bf16 [N1], may be NULL): the column sums of problem 1's B operand
// (the bias gradient), formed inside the grouped launch by the tiles of
// tile-row 0; *csum_done tells whether that happened (else the caller runs
// the column-sum kernel).
template <int E0, int ROLE, int ROLE0, int ROLE1>
hipError_t pair(const Dims& D, GemmArgs p0, GemmArgs p1, float* part, hipStream_t st,
                const RowdotFuse* rd = nullptr, bool* rd_done = nullptr, void* csum = nullptr,
                bool* csum_done = nullptr) {
  using K0 = GemmKind<true, true, E0, bf16_t>;
  using K1 = GemmKind<false, false, EPI_LINEAR, bf16_t>;
  const bool direct = D.dt == TP_BF16 && direct_ok<CfgBig>(p0, 1) && direct_ok<CfgBig>(p1, 1);
  if (!direct) {
    TRY_E((linear<true, true, E0, ROLE0>(D, p0, part, st)));
    return linear<false, false, EPI_LINEAR, ROLE1>(D, p1, part, st);
  }
  const double extra = (E0 == EPI_GELU_BWD) ? 1.0 : 0.0;
  prof::Scope sc(ROLE, 2.0 * p0.M * p0.N * p0.K + 2.0 * p1.M * p1.N * p1.K,
                 (double)D.es * ((double)p0.M * p0.K + (double)p0.K * p0.N + (1.0 + extra) * p0.M * p0.N +
                                 (double)p1.M * p1.K + (double)p1.K * p1.N + (double)p1.M * p1.N),
                 st);
  for (GemmArgs* q : {&p0, &p1}) {
    q->tiles_m = cdiv(q->M, CfgBig::BM);
    q->tiles_n = cdiv(q->N, CfgBig::BN);
    q->group_m = 8;
    q->zdiv = 1;
    q->splits = 1;
  }
  const int tiles0 = p0.tiles_m * p0.tiles_n, tiles1 = p1.tiles_m * p1.tiles_n;
  xcd_blocks(p1, kXcdStrip);
  const PairPlan P = pair_plan(p0.M, p0.N, p0.K, p1.M, p1.N, p1.K, E0 == EPI_GELU_BWD);
  const int splits = P.splits;
  if (splits > 1) {
    p0.splits = splits;
    p0.k_chunk = (int)P.chunk;
    p0.part = part;
  }
  const int units0 = tiles0 * splits;
  const int first1 = p1.K > P.chunk ? 1 : 0;
  p1.csum = csum;
  if (csum_done) *csum_done = csum != nullptr;
  if (splits > 1) {
    hipLaunchKernelGGL((gemm_pair_kernel<CfgBig, GemmKind<true, true, EPI_PARTIAL, float>, K1, ROLE>),
                       dim3(units0 + tiles1), dim3(CfgBig::NT), 0, st, p0, p1, tiles0, units0, tiles1, first1);
    if (rd && E0 == EPI_LINEAR && !p0.bias && !p0.resid && p0.alpha == 1.0f && p0.M == D.T && p0.N == D.hr &&
        p0.ldc == D.hr) {
      hipLaunchKernelGGL(splitk_rowdot_kernel, dim3((unsigned)D.T), dim3(256), 0, st, part, splits,
                         static_cast<bf16_t*>(p0.C), rd->C, rd->D, (int)D.T, (int)D.b, (int)D.ar, (int)D.d, (int)D.s);
      if (rd_done) *rd_done = true;
    } else {
      const long n4 = (long)p0.M * p0.N / 4;
      hipLaunchKernelGGL((splitk_reduce_kernel<E0, bf16_t, bf16_t, ROLE>), dim3((unsigned)cdivl(n4, 256)), dim3(256),
                         0, st, p0);
    }
  } else {
    hipLaunchKernelGGL((gemm_pair_kernel<CfgBig, K0, K1, ROLE>), dim3(units0 + tiles1), dim3(CfgBig::NT), 0, st, p0,
                       p1, tiles0, units0, tiles1, first1);
  }
  return hipGetLastError();
}

// Column sums (bias gradients), one fixed-order pass.
constexpr int kColsumThreads = 256;  // 32 row groups x 8 column threads (1024 measured no faster)

template <int ROLE>
hipError_t colsum(const Dims& D, const void* X, void* out, long R, long N, long ld, hipStream_t st) {
  prof::Scope sc(ROLE, (double)R * N, (double)D.es * (R * N + N), st);
  if (D.dt == TP_BF16)
    hipLaunchKernelGGL((colsum_kernel<bf16_t, kColsumThreads>), dim3((unsigned)cdivl(N, 64)), dim3(kColsumThreads), 0,
                       st, (const bf16_t*)X, (bf16_t*)out, (int)R, (int)N, ld);
  else
    hipLaunchKernelGGL((colsum_kernel<float, kColsumThreads>), dim3((unsigned)cdivl(N, 32)), dim3(kColsumThreads), 0,
                       st, (const float*)X, (float*)out, (int)R, (int)N, ld);
  return hipGetLastError();
}

template <typename T>
hipError_t softmax_t(const Dims& D, const float* S, void* P, hipStream_t st) {
  const long rows = D.z * D.s;
  const unsigned blocks = (unsigned)cdivl(rows, 4);
  const int pad = att_tile(D.dt);
  if (D.s <= 2048)
    hipLaunchKernelGGL((causal_softmax_kernel<T, 8>), dim3(blocks), dim3(256), 0, st, S, (T*)P, rows, (int)D.s, pad);
  else
    hipLaunchKernelGGL((causal_softmax_long_kernel<T>), dim3(blocks), dim3(256), 0, st, S, (T*)P, rows, (int)D.s, pad);
  return hipGetLastError();
}

template <typename T>
hipError_t rowdot_t(const Dims& D, const void* dC, const float* C, float* Dv, hipStream_t st) {
  hipLaunchKernelGGL(rowdot_kernel<T>, dim3((unsigned)D.T), dim3(256), 0, st, (const T*)dC, C, Dv, (int)D.b,
                     (int)D.ar, (int)D.d, (int)D.s);
  return hipGetLastError();
}

#define TRY(x)                                 \
  do {                                         \
    hipError_t e_ = (x);                       \
    if (e_ != hipSuccess) return hip_fail(e_); \
  } while (0)

char* B8(void* p, size_t off) { return static_cast<char*>(p) + off; }
const char* B8(const void* p, size_t off) { return static_cast<const char*>(p) + off; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool misaligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) != 0; }

// Algorithmic cost of one batched attention product over z (sequence, head)
// pairs: model FLOPs count the full s x s square (Eq. 3 of the paper-graph
// page); bytes count the lower triangle of the s x s operand / result.
double att_flops(const Dims& D) { return 2.0 * D.z * D.s * D.s * D.d; }
double tri_elems(const Dims& D) { return (double)D.z * D.s * (D.s + 1) / 2.0; }

// Flash attention launches (256 threads): the main kernels on a 1-D grid of
// z * items workgroups, the combines on (blocks * d / 8, z).
FaArgs fa_args(const Dims& D) {
  FaArgs a;
  memset(&a, 0, sizeof(a));
  a.s = (int)D.s; a.b = (int)D.b; a.ar = (int)D.ar; a.d = (int)D.d; a.hr = (int)D.hr; a.q3 = (int)D.q3;
  a.z = (int)D.z;
  a.ct = fa_chunk_tiles(D);
  a.sc = (float)(1.0 / std::sqrt((double)D.d));
  a.sl2 = (float)(1.4426950408889634 / std::sqrt((double)D.d));  // log2(e) / sqrt(d)
  return a;
}

#define TPL_FA_SWITCH(KERNEL_D, GRID)                                                         \
  do {                                                                                        \
    switch (D.d) {                                                                            \
      case 64: hipLaunchKernelGGL(KERNEL_D(64), GRID, dim3(256), 0, st, a); break;            \
      case 96: hipLaunchKernelGGL(KERNEL_D(96), GRID, dim3(256), 0, st, a); break;            \
      case 128: hipLaunchKernelGGL(KERNEL_D(128), GRID, dim3(256), 0, st, a); break;          \
      case 160: hipLaunchKernelGGL(KERNEL_D(160), GRID, dim3(256), 0, st, a); break;          \
      default: return hipErrorInvalidValue;                                                   \
    }                                                                                         \
  } while (0)
// Head widths up to 128 run the dQ kernel with single-buffered tiles, two
// workgroups per CU (it fits 256 registers per lane); d = 160 and the dK/dV
// kernel keep one double-buffered workgroup per CU.
#define TPL_FA_DKV(DD) fa_bwd_dkv_kernel<DD>
template <int DD>
constexpr auto fa_dq_kernel() {
  if constexpr (DD <= 128) return fa_bwd_dq2_kernel<DD>;
  else return fa_bwd_dq_kernel<DD>;
}
#define TPL_FA_DQ(DD) (fa_dq_kernel<DD>())
#define TPL_FA_KV_COMBINE(DD) (fa_bwd_combine_kernel<DD, true>)
#define TPL_FA_Q_COMBINE(DD) (fa_bwd_combine_kernel<DD, false>)

bool fa_split(const Dims& D, const FaArgs& a) { return a.ct < cdivl(D.s, fa::BT); }
dim3 fa_combine_grid(const Dims& D) { return dim3((unsigned)(cdivl(D.s, fa::BQ) * (D.d / 8)), (unsigned)D.z); }

hipError_t fa_fwd(const Dims& D, FaArgs a, hipStream_t st) {
  const int bq = fa_fwd_bq(D);
  a.ct = fa_fwd_chunk_tiles(D);
  a.items = fa::items_per_head(a.s, a.ct, false, bq);
  const dim3 grid((unsigned)(a.z * a.items));
  const dim3 cgrid((unsigned)(cdivl(D.s, bq) * (bq / 32) * (D.d / 32)), (unsigned)D.z);
  const bool split = fa_split(D, a);
  switch (D.d) {
    case 64:
      hipLaunchKernelGGL(fa_fwd8_kernel<64>, grid, dim3(512), 0, st, a);
      if (split) hipLaunchKernelGGL((fa_fwd_combine_kernel<64, 8>), cgrid, dim3(256), 0, st, a);
      break;
    case 96:
      hipLaunchKernelGGL(fa_fwd8_kernel<96>, grid, dim3(512), 0, st, a);
      if (split) hipLaunchKernelGGL((fa_fwd_combine_kernel<96, 8>), cgrid, dim3(256), 0, st, a);
      break;
    case 128:
      hipLaunchKernelGGL(fa_fwd8_kernel<128>, grid, dim3(512), 0, st, a);
      if (split) hipLaunchKernelGGL((fa_fwd_combine_kernel<128, 8>), cgrid, dim3(256), 0, st, a);
      break;
    case 160:
      hipLaunchKernelGGL(fa_fwd_kernel<160>, grid, dim3(256), 0, st, a);
      if (split) hipLaunchKernelGGL((fa_fwd_combine_kernel<160, 4>), cgrid, dim3(256), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
hipError_t fa_dkv(const Dims& D, FaArgs a, hipStream_t st) {
  a.items = fa::items_per_head(a.s, a.ct, true);
  TPL_FA_SWITCH(TPL_FA_DKV, dim3((unsigned)(a.z * a.items)));
  if (fa_split(D, a)) TPL_FA_SWITCH(TPL_FA_KV_COMBINE, fa_combine_grid(D));
  return hipGetLastError();
}
hipError_t fa_dq(const Dims& D, FaArgs a, hipStream_t st) {
  a.items = fa::items_per_head(a.s, a.ct, false);
  TPL_FA_SWITCH(TPL_FA_DQ, dim3((unsigned)(a.z * a.items)));
  if (fa_split(D, a)) TPL_FA_SWITCH(TPL_FA_Q_COMBINE, fa_combine_grid(D));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// attention block
// ---------------------------------------------------------------------------

int attn_fwd(const Dims& D, const void* x, const tp_block_weights* w, void* y, void* saved, void* ws,
             hipStream_t st) {
  const SavedLayout S = saved_layout(D, TP_ATTN);
  const WsLayout W = ws_layout(D, TP_ATTN);
  void* qkv = B8(saved, S.qkv);
  void* P = B8(saved, S.p);
  void* C = B8(saved, S.c);
  void* C32 = B8(saved, S.c32);
  float* scores = reinterpret_cast<float*>(B8(ws, W.s));
  void* qkv_lo = B8(ws, W.qkv_lo);
  float* part = reinterpret_cast<float*>(B8(ws, W.part));
  const double es = (double)D.es, sde = (double)D.z * D.s * D.d * es;
  const bool bf = D.dt == TP_BF16, fl = flash(D);

  {  // QKV_r = X Wqkv_r + b_qkv_r; bf16 also keeps the rounding residual of Q and K
    GemmArgs p = gargs(D.T, D.q3, D.h);
    p.A = x; p.lda = D.h;
    p.B = w->w_in; p.ldb = D.q3;
    p.C = qkv; p.ldc = D.q3;
    p.bias = w->b_in;
    if (bf) {
      // flash: residuals saved for the backward, [T, 2 h/t]; else workspace, row pitch 3h/t
      p.C2 = fl ? B8(saved, S.qkv_lo) : qkv_lo;
      p.ldc2 = fl ? 2 * D.hr : D.q3;
      p.c2_cols = (int)(2 * D.hr);
      TRY((linear<true, false, EPI_BIAS_SPLIT, R_QKV_FWD>(D, p, part, st)));
    } else {
      TRY((linear<true, false, EPI_LINEAR, R_QKV_FWD>(D, p, part, st)));
    }
  }
  if (fl) {  // C = causal softmax(Q K^T / sqrt(d)) V in one pass, online softmax; LSE saved
    prof::Scope sc(R_ATT_FWD, 2.0 * att_flops(D), 8.0 * sde + 4.0 * D.z * D.s, st);
    FaArgs a = fa_args(D);
    a.qkv = static_cast<const bf16_t*>(qkv);
    a.qkv_lo = reinterpret_cast<const bf16_t*>(B8(saved, S.qkv_lo));
    a.ctx = static_cast<bf16_t*>(C);
    a.ctx32 = static_cast<float*>(C32);
    a.lse = reinterpret_cast<float*>(B8(saved, S.lse));
    a.part = part;
    TRY(fa_fwd(D, a, st));
  } else {
  {  // S_z = Q_z K_z^T / sqrt(d), lower-triangular tiles, fp32.
     // bf16: Q = Qh + Ql, K = Kh + Kl (Ql, Kl the bf16 rounding residuals);
     // S = Qh Kh^T + Qh Kl^T + Ql Kh^T in one K-segmented MFMA pass, which
     // keeps the logits of peaked softmax rows accurate to about 2^-16.
    prof::Scope sc(R_SCORES, att_flops(D), (bf ? 4 : 2) * sde + 4.0 * tri_elems(D), st);
    GemmArgs p = gargs(D.s, D.s, D.d);
    p.zdiv = (int)D.ar;
    p.A = qkv; p.lda = D.b * D.q3; p.a_s1 = D.q3; p.a_s2 = D.d;
    p.B = B8(qkv, (size_t)D.hr * D.es); p.ldb = D.b * D.q3; p.b_s1 = D.q3; p.b_s2 = D.d;
    p.C = scores; p.ldc = D.s; p.c_s1 = D.ar * D.s * D.s; p.c_s2 = D.s * D.s;
    p.alpha = (float)(1.0 / std::sqrt((double)D.d));
    p.tri = 1;
    if (bf) {
      p.A2 = qkv_lo;
      p.B2 = B8(qkv_lo, (size_t)D.hr * D.es);
      p.kseg = 3; p.kseg_len = (int)D.d;
      TRY((run<true, true, EPI_LINEAR, R_SCORES, KIND_MID, true, 3>(D, p, (int)D.z, st)));
    } else {
      TRY((run<true, true, EPI_LINEAR, R_SCORES, KIND_MID, true>(D, p, (int)D.z, st)));
    }
  }
  {  // P = causal softmax(S)
    prof::Scope sc(R_SOFTMAX, 0.0, (4.0 + es) * tri_elems(D), st);
    if (D.dt == TP_BF16) TRY(softmax_t<bf16_t>(D, scores, P, st));
    else TRY(softmax_t<float>(D, scores, P, st));
  }
  {  // C_z = P_z V_z (keys <= query)
    prof::Scope sc(R_PV, att_flops(D), es * tri_elems(D) + 2 * sde, st);
    GemmArgs p = gargs(D.s, D.d, D.s);
    p.zdiv = (int)D.ar;
    p.A = P; p.lda = D.s; p.a_s1 = D.ar * D.s * D.s; p.a_s2 = D.s * D.s;
    p.B = B8(qkv, (size_t)2 * D.hr * D.es); p.ldb = D.b * D.q3; p.b_s1 = D.q3; p.b_s2 = D.d;
    p.C = C; p.ldc = D.b * D.hr; p.c_s1 = D.hr; p.c_s2 = D.d;
    p.kmode = K_LOWER;
    if (bf) {
      p.C2 = C32;
      TRY((run<true, false, EPI_DUAL_F32, R_PV, KIND_MID>(D, p, (int)D.z, st)));
    } else {
      TRY((run<true, false, EPI_LINEAR, R_PV, KIND_MID>(D, p, (int)D.z, st)));
    }
  }
  }  // materialised attention
  if (y) {  // partial = C Wo_r (skipped when the forward is re-run for the backward)
    GemmArgs p = gargs(D.T, D.h, D.hr);
    p.A = C; p.lda = D.hr;
    p.B = w->w_out; p.ldb = D.h;
    p.C = y; p.ldc = D.h;
    TRY((linear<true, false, EPI_LINEAR, R_O_FWD>(D, p, part, st)));
  }
  return TP_OK;
}

int attn_bwd(const Dims& D, const void* x, const tp_block_weights* w, const void* saved, const void* dy, void* dx,
             const tp_block_grads* g, void* ws, hipStream_t st) {
  const SavedLayout S = saved_layout(D, TP_ATTN);
  const WsLayout W = ws_layout(D, TP_ATTN);
  const void* qkv = B8(saved, S.qkv);
  const void* P = B8(saved, S.p);
  const void* C = B8(saved, S.c);
  const float* C32 = reinterpret_cast<const float*>(B8(saved, S.c32));
  void* dC = B8(ws, W.dc);
  float* Dv = reinterpret_cast<float*>(B8(ws, W.D));
  void* dS = B8(ws, W.ds);
  void* dqkv = B8(ws, W.dqkv);
  float* part = reinterpret_cast<float*>(B8(ws, W.part));
  const float scale = (float)(1.0 / std::sqrt((double)D.d));
  const double es = (double)D.es, sde = (double)D.z * D.s * D.d * es;

  bool rd_done = false;
  {  // dC = dH Wo_r^T
    GemmArgs p = gargs(D.T, D.hr, D.h);
    p.A = dy; p.lda = D.h;
    p.B = w->w_out; p.ldb = D.h;
    p.C = dC; p.ldc = D.hr;
    // dWo_r = C^T dH
    GemmArgs q = gargs(D.hr, D.h, D.T);
    q.A = C; q.lda = D.hr;
    q.B = dy; q.ldb = D.h;
    q.C = g->dw_out; q.ldc = D.h;
    // (a split-K dC also gives D = rowsum(dC * C) in its summing pass)
    // (and dbo = sum over tokens of dH, a replica, from the weight-gradient
    // tiles' dH fragments)
    const RowdotFuse rdf{C32, Dv};
    bool cs_done = false;
    TRY((pair<EPI_LINEAR, R_O_BWD, R_O_DGRAD, R_O_WGRAD>(D, p, q, part, st, &rdf, &rd_done, g->db_out, &cs_done)));
    if (!cs_done) TRY(colsum<R_DBO>(D, dy, g->db_out, D.T, D.h, D.h, st));
  }
  if (!rd_done) {  // D = rowsum(dC * C) per (sequence, head, query)
    prof::Scope sc(R_ROWDOT, 2.0 * D.T * D.hr, D.T * D.hr * (es + 4.0) + 4.0 * D.z * D.s, st);
    if (D.dt == TP_BF16) TRY(rowdot_t<bf16_t>(D, dC, C32, Dv, st));
    else TRY(rowdot_t<float>(D, dC, C32, Dv, st));
  }
  if (flash(D)) {  // dK, dV per key block; dQ per query block (P and dP recomputed)
    FaArgs a = fa_args(D);
    a.qkv = static_cast<const bf16_t*>(qkv);
    a.qkv_lo = reinterpret_cast<const bf16_t*>(B8(saved, S.qkv_lo));
    a.lse = const_cast<float*>(reinterpret_cast<const float*>(B8(saved, S.lse)));
    a.dctx = static_cast<const bf16_t*>(dC);
    a.dsum = Dv;
    a.dqkv = static_cast<bf16_t*>(dqkv);
    a.part = part;
    {
      prof::Scope sc(R_ATT_DKV, 3.0 * att_flops(D), 8.0 * sde + 8.0 * D.z * D.s, st);
      TRY(fa_dkv(D, a, st));
    }
    {
      prof::Scope sc(R_ATT_DQ, att_flops(D), 7.0 * sde + 8.0 * D.z * D.s, st);
      TRY(fa_dq(D, a, st));
    }
  } else {
  {  // dS = P * (dC V^T - D) / sqrt(d), lower-triangular tiles
    prof::Scope sc(R_DS, att_flops(D), 2 * sde + 2 * es * tri_elems(D) + 4.0 * D.z * D.s, st);
    GemmArgs p = gargs(D.s, D.s, D.d);
    p.zdiv = (int)D.ar;
    p.A = dC; p.lda = D.b * D.hr; p.a_s1 = D.hr; p.a_s2 = D.d;
    p.B = B8(qkv, (size_t)2 * D.hr * D.es); p.ldb = D.b * D.q3; p.b_s1 = D.q3; p.b_s2 = D.d;
    p.C = dS; p.ldc = D.s; p.c_s1 = D.ar * D.s * D.s; p.c_s2 = D.s * D.s;
    p.aux = P; p.ldx = D.s; p.x_s1 = D.ar * D.s * D.s; p.x_s2 = D.s * D.s;
    p.rowv = Dv; p.r_s1 = D.ar * D.s; p.r_s2 = D.s;
    p.alpha = scale;
    p.tri = 1;
    TRY((run<true, true, EPI_SOFTMAX_BWD, R_DS, KIND_MID>(D, p, (int)D.z, st)));
  }
  {  // dV = P^T dC  (queries >= key)
    prof::Scope sc(R_DV, att_flops(D), es * tri_elems(D) + 2 * sde, st);
    GemmArgs p = gargs(D.s, D.d, D.s);
    p.zdiv = (int)D.ar;
    p.A = P; p.lda = D.s; p.a_s1 = D.ar * D.s * D.s; p.a_s2 = D.s * D.s;
    p.B = dC; p.ldb = D.b * D.hr; p.b_s1 = D.hr; p.b_s2 = D.d;
    p.C = B8(dqkv, (size_t)2 * D.hr * D.es); p.ldc = D.b * D.q3; p.c_s1 = D.q3; p.c_s2 = D.d;
    p.kmode = K_UPPER;
    TRY((run<false, false, EPI_LINEAR, R_DV, KIND_MID>(D, p, (int)D.z, st)));
  }
  {  // dQ = dS K  (keys <= query); 1/sqrt(d) already in dS
    prof::Scope sc(R_DQ, att_flops(D), es * tri_elems(D) + 2 * sde, st);
    GemmArgs p = gargs(D.s, D.d, D.s);
    p.zdiv = (int)D.ar;
    p.A = dS; p.lda = D.s; p.a_s1 = D.ar * D.s * D.s; p.a_s2 = D.s * D.s;
    p.B = B8(qkv, (size_t)D.hr * D.es); p.ldb = D.b * D.q3; p.b_s1 = D.q3; p.b_s2 = D.d;
    p.C = dqkv; p.ldc = D.b * D.q3; p.c_s1 = D.q3; p.c_s2 = D.d;
    p.kmode = K_LOWER;
    TRY((run<true, false, EPI_LINEAR, R_DQ, KIND_MID>(D, p, (int)D.z, st)));
  }
  {  // dK = dS^T Q  (queries >= key)
    prof::Scope sc(R_DK, att_flops(D), es * tri_elems(D) + 2 * sde, st);
    GemmArgs p = gargs(D.s, D.d, D.s);
    p.zdiv = (int)D.ar;
    p.A = dS; p.lda = D.s; p.a_s1 = D.ar * D.s * D.s; p.a_s2 = D.s * D.s;
    p.B = qkv; p.ldb = D.b * D.q3; p.b_s1 = D.q3; p.b_s2 = D.d;
    p.C = B8(dqkv, (size_t)D.hr * D.es); p.ldc = D.b * D.q3; p.c_s1 = D.q3; p.c_s2 = D.d;
    p.kmode = K_UPPER;
    TRY((run<false, false, EPI_LINEAR, R_DK, KIND_MID>(D, p, (int)D.z, st)));
  }
  }  // materialised attention
  {  // dX_r = dQKV Wqkv_r^T
    GemmArgs p = gargs(D.T, D.h, D.q3);
    p.A = dqkv; p.lda = D.q3;
    p.B = w->w_in; p.ldb = D.q3;
    p.C = dx; p.ldc = D.h;
    // dWqkv_r = X^T dQKV
    GemmArgs q = gargs(D.h, D.q3, D.T);
    q.A = x; q.lda = D.h;
    q.B = dqkv; q.ldb = D.q3;
    q.C = g->dw_in; q.ldc = D.q3;
    // db_qkv = sum over tokens of dQKV
    bool cs_done = false;
    TRY((pair<EPI_LINEAR, R_QKV_BWD, R_QKV_DGRAD, R_QKV_WGRAD>(D, p, q, part, st, nullptr, nullptr, g->db_in,
                                                               &cs_done)));
    if (!cs_done) TRY(colsum<R_DBQKV>(D, dqkv, g->db_in, D.T, D.q3, D.q3, st));
  }
  return TP_OK;
}

// ---------------------------------------------------------------------------
// MLP block
// ---------------------------------------------------------------------------

int mlp_fwd(const Dims& D, const void* x, const tp_block_weights* w, void* y, void* saved, void* ws, hipStream_t st) {
  const SavedLayout S = saved_layout(D, TP_MLP);
  const WsLayout W = ws_layout(D, TP_MLP);
  void* U = B8(saved, S.u);
  void* Z = B8(saved, S.z);
  float* part = reinterpret_cast<float*>(B8(ws, W.part));
  {  // U = H W1_r + b1_r; Z = GELU(U)
    GemmArgs p = gargs(D.T, D.fr, D.h);
    p.A = x; p.lda = D.h;
    p.B = w->w_in; p.ldb = D.fr;
    p.C = U; p.ldc = D.fr;
    p.C2 = Z; p.ldc2 = D.fr;
    p.bias = w->b_in;
    TRY((linear<true, false, EPI_BIAS_GELU, R_FC1_FWD>(D, p, part, st)));
  }
  if (y) {  // partial = Z W2_r (skipped when the forward is re-run for the backward)
    GemmArgs p = gargs(D.T, D.h, D.fr);
    p.A = Z; p.lda = D.fr;
    p.B = w->w_out; p.ldb = D.h;
    p.C = y; p.ldc = D.h;
    TRY((linear<true, false, EPI_LINEAR, R_FC2_FWD>(D, p, part, st)));
  }
  return TP_OK;
}

int mlp_bwd(const Dims& D, const void* x, const tp_block_weights* w, const void* saved, const void* dy, void* dx,
            const tp_block_grads* g, void* ws, hipStream_t st) {
  const SavedLayout S = saved_layout(D, TP_MLP);
  const WsLayout W = ws_layout(D, TP_MLP);
  const void* U = B8(saved, S.u);
  const void* Z = B8(saved, S.z);
  void* dU = B8(ws, W.du);
  float* part = reinterpret_cast<float*>(B8(ws, W.part));
  {  // dU = (dY W2_r^T) * GELU'(U)
    GemmArgs p = gargs(D.T, D.fr, D.h);
    p.A = dy; p.lda = D.h;
    p.B = w->w_out; p.ldb = D.h;
    p.C = dU; p.ldc = D.fr;
    p.aux = U; p.ldx = D.fr;
    // dW2_r = Z^T dY
    GemmArgs q = gargs(D.fr, D.h, D.T);
    q.A = Z; q.lda = D.fr;
    q.B = dy; q.ldb = D.h;
    q.C = g->dw_out; q.ldc = D.h;
    // db2 = sum over tokens of dY (a replica)
    bool cs_done = false;
    TRY((pair<EPI_GELU_BWD, R_FC2_BWD, R_FC2_DGRAD, R_FC2_WGRAD>(D, p, q, part, st, nullptr, nullptr, g->db_out,
                                                                 &cs_done)));
    if (!cs_done) TRY(colsum<R_DB2>(D, dy, g->db_out, D.T, D.h, D.h, st));
  }
  {  // dH_r = dU W1_r^T
    GemmArgs p = gargs(D.T, D.h, D.fr);
    p.A = dU; p.lda = D.fr;
    p.B = w->w_in; p.ldb = D.fr;
    p.C = dx; p.ldc = D.h;
    // dW1_r = H^T dU
    GemmArgs q = gargs(D.h, D.fr, D.T);
    q.A = x; q.lda = D.h;
    q.B = dU; q.ldb = D.fr;
    q.C = g->dw_in; q.ldc = D.fr;
    // db1 = sum over tokens of dU
    bool cs_done = false;
    TRY((pair<EPI_LINEAR, R_FC1_BWD, R_FC1_DGRAD, R_FC1_WGRAD>(D, p, q, part, st, nullptr, nullptr, g->db_in,
                                                               &cs_done)));
    if (!cs_done) TRY(colsum<R_DB1>(D, dU, g->db_in, D.T, D.fr, D.fr, st));
  }
  return TP_OK;
}

// LayerNorm launches: a row takes one wave when it has at most 512 16-byte
// chunks, else the whole workgroup with NC chunks a thread.
constexpr long kLnMaxChunks = 256 * 16;

template <typename T>
hipError_t ln_fwd_launch(const LnFwdArgs& a, hipStream_t st) {
  const long nch = a.h / Elt<T>::VEC;
  if (nch <= 64 * 8) {
    hipLaunchKernelGGL((ln_fwd_kernel<T, 64, 8>), dim3((unsigned)cdivl(a.rows, 4)), dim3(256), 0, st, a);
  } else {
    const unsigned g = (unsigned)a.rows;
    if (nch <= 256 * 4) hipLaunchKernelGGL((ln_fwd_kernel<T, 256, 4>), dim3(g), dim3(256), 0, st, a);
    else if (nch <= 256 * 6) hipLaunchKernelGGL((ln_fwd_kernel<T, 256, 6>), dim3(g), dim3(256), 0, st, a);
    else if (nch <= 256 * 8) hipLaunchKernelGGL((ln_fwd_kernel<T, 256, 8>), dim3(g), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((ln_fwd_kernel<T, 256, 16>), dim3(g), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t ln_dparam_launch(const LnBwdArgs& a, hipStream_t st) {
  constexpr int W = 8 * Elt<T>::VEC;  // columns per workgroup
  hipLaunchKernelGGL(ln_bwd_dparam_kernel<T>, dim3((unsigned)cdiv(a.h, W)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T>
hipError_t ln_bwd_launch(const LnBwdArgs& a, hipStream_t st) {
  if (a.rows > 0) {
    const long nch = a.h / Elt<T>::VEC;
    if (nch <= 64 * 8) {
      hipLaunchKernelGGL((ln_bwd_dx_kernel<T, 64, 8>), dim3((unsigned)cdivl(a.rows, 4)), dim3(256), 0, st, a);
    } else {
      const unsigned g = (unsigned)a.rows;
      if (nch <= 256 * 4) hipLaunchKernelGGL((ln_bwd_dx_kernel<T, 256, 4>), dim3(g), dim3(256), 0, st, a);
      else if (nch <= 256 * 6) hipLaunchKernelGGL((ln_bwd_dx_kernel<T, 256, 6>), dim3(g), dim3(256), 0, st, a);
      else if (nch <= 256 * 8) hipLaunchKernelGGL((ln_bwd_dx_kernel<T, 256, 8>), dim3(g), dim3(256), 0, st, a);
      else hipLaunchKernelGGL((ln_bwd_dx_kernel<T, 256, 16>), dim3(g), dim3(256), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // no rows: the parameter gradients are empty sums (zeros)
  return a.dgamma ? ln_dparam_launch<T>(a, st) : hipSuccess;
}

// LayerNorm argument checks shared by the two entry points.
int ln_check(int dtype, long rows, long h) {
  if (dtype != TP_BF16 && dtype != TP_FP32) return TP_EINVAL;
  if (rows < 0 || h <= 0) return TP_EINVAL;
  if (h % 8 != 0 || h / (dtype == TP_BF16 ? 8 : 4) > kLnMaxChunks) return TP_EUNSUPPORTED;
  return TP_OK;
}

// ---------------------------------------------------------------------------
// library-owned scratch for callers that cannot allocate (tp_layer_bwd_noalloc)
// ---------------------------------------------------------------------------

// Each GPU that runs the library holds its own copy of this array until the
// process ends. In host code `scratch` names a host-side stand-in: kernels
// and copies take the device address from scratch_ptr() instead.
constexpr size_t kScratchBytes = (size_t)256 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return TP_EINVAL;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return TP_EHIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return TP_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int tp_check_args(int h, int a, int s, int b, int t, int rank, int dtype, int block) {
  return check_args(h, a, s, b, t, rank, dtype, block);
}

size_t tp_saved_bytes(int h, int a, int s, int b, int t, int dtype, int block) {
  if (check_args(h, a, s, b, t, 0, dtype, block) != TP_OK) return 0;
  return saved_layout(make_dims(h, a, s, b, t, dtype), block).total;
}

size_t tp_workspace_bytes(int h, int a, int s, int b, int t, int dtype, int block) {
  if (check_args(h, a, s, b, t, 0, dtype, block) != TP_OK) return 0;
  return ws_layout(make_dims(h, a, s, b, t, dtype), block).total;
}

int tp_layer_fwd(int h, int a, int s, int b, int t, int rank, int dtype, int block, const void* x,
                 const tp_block_weights* w, void* y_partial, void* saved, void* workspace, size_t workspace_bytes,
                 void* stream) {
  int rc = check_args(h, a, s, b, t, rank, dtype, block);
  if (rc != TP_OK) return rc;
  if (!x || !w || !w->w_in || !w->b_in || !w->w_out || !y_partial || !saved || !workspace) return TP_ENULL;
  if (misaligned(x) || misaligned(w->w_in) || misaligned(w->b_in) || misaligned(w->w_out) || misaligned(y_partial) ||
      misaligned(saved) || misaligned(workspace))
    return TP_EALIGN;
  const Dims D = make_dims(h, a, s, b, t, dtype);
  if (workspace_bytes < ws_layout(D, block).total) return TP_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return block == TP_ATTN ? attn_fwd(D, x, w, y_partial, saved, workspace, st)
                          : mlp_fwd(D, x, w, y_partial, saved, workspace, st);
}

int tp_layer_bwd(int h, int a, int s, int b, int t, int rank, int dtype, int block, const void* x,
                 const tp_block_weights* w, const void* saved, const void* dy, void* dx_partial,
                 const tp_block_grads* g, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_args(h, a, s, b, t, rank, dtype, block);
  if (rc != TP_OK) return rc;
  if (!x || !w || !w->w_in || !w->w_out || !saved || !dy || !dx_partial || !g || !g->dw_in || !g->db_in ||
      !g->dw_out || !g->db_out || !workspace)
    return TP_ENULL;
  if (misaligned(x) || misaligned(w->w_in) || misaligned(w->w_out) || misaligned(saved) || misaligned(dy) ||
      misaligned(dx_partial) || misaligned(g->dw_in) || misaligned(g->db_in) || misaligned(g->dw_out) ||
      misaligned(g->db_out) || misaligned(workspace))
    return TP_EALIGN;
  const Dims D = make_dims(h, a, s, b, t, dtype);
  if (workspace_bytes < ws_layout(D, block).total) return TP_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return block == TP_ATTN ? attn_bwd(D, x, w, saved, dy, dx_partial, g, workspace, st)
                          : mlp_bwd(D, x, w, saved, dy, dx_partial, g, workspace, st);
}

size_t tp_noalloc_scratch_bytes(void) { return kScratchBytes; }

int tp_layer_bwd_noalloc(int h, int a, int s, int b, int t, int rank, int dtype, int block, const void* x,
                         const tp_block_weights* w, const void* saved, const void* dy, void* dx_partial,
                         const tp_block_grads* g, void* stream) {
  int rc = check_args(h, a, s, b, t, rank, dtype, block);
  if (rc != TP_OK) return rc;
  if (ws_layout(make_dims(h, a, s, b, t, dtype), block).total > kScratchBytes) return TP_ESCRATCH;
  void* ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc != TP_OK) return rc;
  // same checks and kernels as tp_layer_bwd, on the library's scratch (no
  // kernel relies on the scratch's contents at entry, so nothing is cleared)
  prof::suppressed = true;
  rc = tp_layer_bwd(h, a, s, b, t, rank, dtype, block, x, w, saved, dy, dx_partial, g, ws, kScratchBytes, stream);
  prof::suppressed = false;
  return rc;
}

int tp_reduce_partials(int dtype, long rows, long cols, int t, const void* partials, const void* bias,
                       const void* residual, void* out, void* stream) {
  if (dtype != TP_BF16 && dtype != TP_FP32) return TP_EINVAL;
  if (t <= 0 || rows < 0 || cols <= 0 || cols % 8 != 0) return TP_EINVAL;
  if (!partials || !out) return TP_ENULL;
  if (misaligned(partials) || misaligned(out) || misaligned(bias) || misaligned(residual)) return TP_EALIGN;
  if (rows == 0) return TP_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long n = rows * cols;
  const size_t es = dtype == TP_BF16 ? 2 : 4;
  prof::Scope sc(R_REDUCE, (double)t * n, (double)es * n * (t + 1 + (residual ? 1 : 0)), st);
  const unsigned blocks = (unsigned)cdivl(n / 4, 256);
  if (dtype == TP_BF16)
    hipLaunchKernelGGL(reduce_partials_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)partials,
                       (const bf16_t*)bias, (const bf16_t*)residual, (bf16_t*)out, rows, cols, t);
  else
    hipLaunchKernelGGL(reduce_partials_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)partials,
                       (const float*)bias, (const float*)residual, (float*)out, rows, cols, t);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_fail(e);
}

int tp_layernorm_fwd(int dtype, long rows, long h, float eps, const void* x, const void* bias, const void* residual,
                     const void* gamma, const void* beta, void* sum_out, void* y, float* stats, void* stream) {
  int rc = ln_check(dtype, rows, h);
  if (rc != TP_OK) return rc;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return TP_EINVAL;
  if (rows == 0) return TP_OK;  // no tokens: nothing is read or written
  if (!x) return TP_ENULL;
  if (gamma ? (!beta || !y || !stats) : !sum_out) return TP_ENULL;
  if (misaligned(x) || misaligned(bias) || misaligned(residual) || misaligned(gamma) || misaligned(beta) ||
      misaligned(sum_out) || misaligned(y) || misaligned8(stats))
    return TP_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  LnFwdArgs a{x, bias, residual, gamma, beta, sum_out, gamma ? y : nullptr, gamma ? stats : nullptr,
              rows, (int)h, eps};
  const double es = dtype == TP_BF16 ? 2.0 : 4.0, n = (double)rows * h;
  const double bytes = es * n * (1 + (residual ? 1 : 0) + (sum_out ? 1 : 0) + (gamma ? 1 : 0)) +
                       es * h * ((bias ? 1 : 0) + (gamma ? 2 : 0)) + (gamma ? 8.0 * rows : 0.0);
  prof::Scope sc(R_LN_FWD, 0.0, bytes, st);
  hipError_t e = dtype == TP_BF16 ? ln_fwd_launch<bf16_t>(a, st) : ln_fwd_launch<float>(a, st);
  return e == hipSuccess ? TP_OK : hip_fail(e);
}

int tp_layernorm_bwd(int dtype, long rows, long h, const void* dy, const void* v, const float* stats,
                     const void* gamma, const void* dresid, void* dx, void* dgamma, void* dbeta, void* stream) {
  int rc = ln_check(dtype, rows, h);
  if (rc != TP_OK) return rc;
  if ((!dgamma) != (!dbeta)) return TP_ENULL;
  if (rows > 0 && (!dy || !v || !stats || !gamma || !dx)) return TP_ENULL;  // no tokens: only dgamma, dbeta
  if (misaligned(dy) || misaligned(v) || misaligned8(stats) || misaligned(gamma) || misaligned(dresid) ||
      misaligned(dx) || misaligned(dgamma) || misaligned(dbeta))
    return TP_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const double es = dtype == TP_BF16 ? 2.0 : 4.0, n = (double)rows * h;
  const double bytes = es * n * (3 + (dresid ? 1 : 0)) + es * h * (1 + (dgamma ? 2 : 0)) + 8.0 * rows;
  prof::Scope sc(R_LN_BWD, 0.0, bytes, st);
  LnBwdArgs a{dy, v, gamma, dresid, stats, dx, dgamma, dbeta, rows, (int)h};
  hipError_t e = dtype == TP_BF16 ? ln_bwd_launch<bf16_t>(a, st) : ln_bwd_launch<float>(a, st);
  return e == hipSuccess ? TP_OK : hip_fail(e);
}

int tp_layer_bwd_recompute(int h, int a, int s, int b, int t, int rank, int dtype, int block, const void* x,
                           const tp_block_weights* w, const void* dy, void* dx_partial, const tp_block_grads* g,
                           void* scratch, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_args(h, a, s, b, t, rank, dtype, block);
  if (rc != TP_OK) return rc;
  if (!x || !w || !w->w_in || !w->b_in || !w->w_out || !dy || !dx_partial || !g || !g->dw_in || !g->db_in ||
      !g->dw_out || !g->db_out || !scratch || !workspace)
    return TP_ENULL;
  if (misaligned(x) || misaligned(w->w_in) || misaligned(w->b_in) || misaligned(w->w_out) || misaligned(dy) ||
      misaligned(dx_partial) || misaligned(g->dw_in) || misaligned(g->db_in) || misaligned(g->dw_out) ||
      misaligned(g->db_out) || misaligned(scratch) || misaligned(workspace))
    return TP_EALIGN;
  const Dims D = make_dims(h, a, s, b, t, dtype);
  if (workspace_bytes < ws_layout(D, block).total) return TP_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the forward again, up to (not including) the block's output product, into scratch
  rc = block == TP_ATTN ? attn_fwd(D, x, w, nullptr, scratch, workspace, st)
                        : mlp_fwd(D, x, w, nullptr, scratch, workspace, st);
  if (rc != TP_OK) return rc;
  return block == TP_ATTN ? attn_bwd(D, x, w, scratch, dy, dx_partial, g, workspace, st)
                          : mlp_bwd(D, x, w, scratch, dy, dx_partial, g, workspace, st);
}

size_t tp_gemm_workspace_bytes(int dtype, int M, int N, int K) {
  if ((dtype != TP_BF16 && dtype != TP_FP32) || M <= 0 || N <= 0 || K <= 0) return 0;
  return partial_bytes(make_dims(16, 1, 16, 1, 1, dtype), M, N, K);
}

int tp_gemm(int dtype, int M, int N, int K, float alpha, const void* A, long lda, int a_kmajor, const void* B, long ldb,
            int b_kmajor, const void* bias, void* C, long ldc, void* workspace, size_t workspace_bytes,
            void* stream) {
  if (dtype != TP_BF16 && dtype != TP_FP32) return TP_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0) return TP_EINVAL;
  if (M % 16 || N % 16 || K % 16 || lda % 8 || ldb % 8 || ldc % 8) return TP_EUNSUPPORTED;
  if (lda < (a_kmajor ? K : M) || ldb < (b_kmajor ? K : N) || ldc < N) return TP_EINVAL;
  // each operand and the output span fewer than 2^31 elements (32-bit byte
  // offsets in the tile loaders)
  if ((long)(a_kmajor ? M : K) * lda >= kMaxElems || (long)(b_kmajor ? N : K) * ldb >= kMaxElems ||
      (long)M * ldc >= kMaxElems)
    return TP_EUNSUPPORTED;
  if (!A || !B || !C) return TP_ENULL;
  if (misaligned(A) || misaligned(B) || misaligned(C) || misaligned(bias)) return TP_EALIGN;
  const Dims D = make_dims(16, 1, 16, 1, 1, dtype);  // only the dtype is used
  const size_t need = partial_bytes(D, M, N, K);
  if (workspace_bytes < need) return TP_EWORKSPACE;
  if (need && !workspace) return TP_ENULL;
  if (misaligned(workspace)) return TP_EALIGN;
  GemmArgs p = gargs(M, N, K);
  p.A = A; p.lda = lda; p.B = B; p.ldb = ldb; p.C = C; p.ldc = ldc;
  p.bias = bias; p.alpha = alpha;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
  hipError_t e;
  if (a_kmajor && !b_kmajor) e = linear<true, false, EPI_LINEAR, R_GEMM>(D, p, part, st);
  else if (a_kmajor && b_kmajor) e = linear<true, true, EPI_LINEAR, R_GEMM>(D, p, part, st);
  else if (!a_kmajor && !b_kmajor) e = linear<false, false, EPI_LINEAR, R_GEMM>(D, p, part, st);
  else e = linear<false, true, EPI_LINEAR, R_GEMM>(D, p, part, st);
  return e == hipSuccess ? TP_OK : hip_fail(e);
}

int tp_prof_enable(int on) {
  std::lock_guard<std::mutex> g(prof::mu);
  if (on) {
    for (auto& r : prof::recs) {
      prof::pool.push_back(r.a);
      prof::pool.push_back(r.b);
    }
    prof::recs.clear();
  }
  prof::on.store(on != 0);
  return TP_OK;
}

int tp_prof_read(tp_prof_entry* out, int max_entries) {
  if (!out && max_entries > 0) return TP_ENULL;
  std::vector<prof::Rec> recs;
  {
    std::lock_guard<std::mutex> g(prof::mu);
    recs.swap(prof::recs);
  }
  tp_prof_entry acc[R_COUNT];
  memset(acc, 0, sizeof(acc));
  int err = TP_OK;
  for (auto& r : recs) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) err = hip_fail(e);
    tp_prof_entry& a = acc[r.role];
    a.launches += 1;
    a.ms += ms;
    a.flops += r.flops;
    a.bytes += r.bytes;
  }
  {
    std::lock_guard<std::mutex> g(prof::mu);
    for (auto& r : recs) {
      prof::pool.push_back(r.a);
      prof::pool.push_back(r.b);
    }
  }
  if (err != TP_OK) return err;
  int n = 0;
  for (int i = 0; i < R_COUNT; ++i) {
    if (acc[i].launches == 0) continue;
    if (n < max_entries) {
      out[n] = acc[i];
      snprintf(out[n].name, sizeof(out[n].name), "%s", kRoleName[i]);
    }
    ++n;
  }
  return n;
}

const char* tp_strerror(int code) {
  switch (code) {
    case TP_OK: return "ok";
    case TP_EINVAL: return "invalid argument (dims, heads not divisible by t, rank out of range, or bad enum)";
    case TP_EUNSUPPORTED:
      return "unsupported shape (s, d and h/t must be multiples of 16; every matrix below 2^31 elements)";
    case TP_ENULL: return "a required pointer is NULL";
    case TP_EALIGN: return "a pointer is not 16-byte aligned";
    case TP_EWORKSPACE: return "workspace smaller than tp_workspace_bytes()";
    case TP_ESCRATCH: return "the call needs more scratch than the library's static buffer (tp_noalloc_scratch_bytes())";
    case TP_EHIP: return g_hip_err[0] ? g_hip_err : "HIP error";
  }
  return "unknown error code";
}

}  // extern "C"
