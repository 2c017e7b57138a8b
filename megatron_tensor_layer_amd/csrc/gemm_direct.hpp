// bf16 MFMA GEMM for gfx950 with direct global -> LDS tile loads.
//
// Same contract as gemm_kernel (gemm.hpp): C = epilogue(op(A) op(B)), fp32
// accumulation, one 256x256 (or 128x128) output tile per block of four waves.
// The operand tiles travel from HBM straight into LDS with
// global_load_lds_dwordx4 (each lane's 16 bytes land at dst + 16 * lane), so
// the K loop needs no staging registers and no LDS store instructions, and a
// tile's loads have a whole K step of MFMA work to hide behind:
//
//   iteration kt:  issue loads of tile kt+1 into the idle LDS buffer
//                  4 sub-steps x (fragment reads + MFMAs) on tile kt
//                  wait for the loads, barrier
//
// LDS layouts (one 64-deep K tile):
//  * K-contiguous operand: row = m (or n), 128 bytes = 64 k; the eight
//    16-byte chunks of row r are stored at chunk ^ kswz(r). MFMA fragments
//    (8 consecutive k of one row) are single ds_read_b128, conflict free.
//  * M/N-contiguous operand: row = k, BM*2 (BN*2) bytes of m (n); the 32-byte
//    segments of row k are stored at segment ^ tsw(k). Fragments come from
//    two ds_read_b64_tr_b16 per lane: within each 16-lane group, lane i gets
//    element i%4 of the 8-byte chunks addressed by lanes 4c + i/4 (c = 0..3),
//    so addressing rows k = 4c' + ... and columns 16*(g%2) + 4*(i%4) hands
//    every lane 4 consecutive k of one column; the XOR keeps the four rows
//    of a group on distinct banks.
// The swizzles are applied by choosing which global chunk each lane loads.
// Rows (columns) beyond M (N) are clamped to the last valid one: they only
// feed outputs that are never stored. K runs must be multiples of 64; ragged
// K uses gemm_kernel.
#pragma once

#include "gemm.hpp"

namespace tpl {

typedef short v4i16_t __attribute__((ext_vector_type(4)));
#define TPL_LDS __attribute__((address_space(3)))
#define TPL_GLOBAL __attribute__((address_space(1)))

// global_load_lds_dwordx4 with a wave-uniform base (SGPRs), a per-lane
// 32-bit byte offset and the wave's LDS destination in M0. Issued as inline
// assembly so that the compiler does not serialize the tile's LDS fragment
// reads behind these loads (it cannot tell that they target the other
// buffer); the kernel waits for them explicitly (vmcnt(0)) before each
// barrier. Loads the compiler issues itself stay correctly ordered: extra
// outstanding loads only make its own vmcnt waits more conservative.
__device__ __forceinline__ const bf16_t* uniform_ptr(const bf16_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const bf16_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void load_lds16(const bf16_t* base, uint32_t byte_off, uint4* lds_dst) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(byte_off), "s"(uniform_ptr(base))
               : "memory", "m0");
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint2 read_tr(const uint4* lds, uint32_t byte_off) {
  const TPL_LDS v4i16_t* p = (const TPL_LDS v4i16_t*)((const TPL_LDS char*)lds + byte_off);
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((TPL_LDS v4i16_t*)p));
}

// Sum of the 8 bf16 of a fragment, added to acc: v_dot2_f32_bf16 against
// (1, 1), one instruction per dword, in a fixed order.
__device__ __forceinline__ float colsum8(const uint4& f, float acc) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 one = __builtin_bit_cast(bf2, 0x3f803f80u);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, f.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, f.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, f.z), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, f.w), one, acc, false);
  return acc;
}

// One operand's tile loader + fragment reader. R = rows of the operand tile
// along M (or N); KMAJ = operand stored K-contiguous in HBM.
// XOR swizzle of the 16-byte chunks of K-contiguous LDS row `row`: distinct for
// any 8 consecutive rows, and for the 8 even (odd) rows of any 16, so that a
// ds_read_b128 of 32 consecutive rows is bank-conflict free whether the LDS
// serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int kswz(int row) {
  return ((row >> 1) ^ ((row & 1) << 2)) & 7;
}

// Segment swizzle of M/N-contiguous rows: segment ^ tsw(k). The four k rows a
// 16-lane group of ds_read_b64_tr_b16 touches land on four distinct segments
// mod 4, and together with the neighbouring group's segment (s ^ 1) on eight
// distinct segments, so the read is conflict free with 16 or 32 lanes per
// LDS cycle.
__device__ __forceinline__ int tsw(int k) { return (0x7520 >> (4 * (k & 3))) & 0xF; }

// VALID < R (M/N-major only): the tile is laid out R wide but only its first
// VALID columns are loaded; lanes whose chunk lies beyond them issue no load.
template <bool KMAJ, int R, int NT, int VALID = R>
struct DirectOperand {
  static constexpr int BK = 64;
  static constexpr int TILE_BYTES = R * BK * 2;
  static constexpr int INSTS = TILE_BYTES / 1024;  // wave-wide 1 KB loads per tile
  static constexpr int WAVES = NT / 64;
  static_assert(INSTS % WAVES == 0, "tile must split evenly over the waves");
  static constexpr int PER_WAVE = INSTS / WAVES;
  static constexpr int ROW_UNITS = R / 8;  // 16-byte units per k-row (M/N-major)
  static_assert(KMAJ || 64 % ROW_UNITS == 0, "an M/N-major load instruction covers whole k-rows of the tile");
  static_assert(VALID == R || (!KMAJ && VALID % 8 == 0 && VALID < R), "partial loads: M/N-major tiles only");
  static_assert(PER_WAVE <= 32, "one mask bit per load");
  uint32_t off[PER_WAVE];                  // element offsets at the tile's k origin
  uint32_t live;                           // VALID < R: bit i set if load i has a chunk to fetch

  __device__ __forceinline__ void init(long ld, int mn0, int lim, int wave, int lane) {
    live = 0;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int inst = wave * PER_WAVE + i;
      if constexpr (KMAJ) {
        const int row = inst * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ kswz(row);
        const int g = min(mn0 + row, lim - 1);
        off[i] = (uint32_t)((long)g * ld + chunk * 8);
      } else {
        constexpr int ROWS_PER_INST = 64 / ROW_UNITS;
        const int k = inst * ROWS_PER_INST + lane / ROW_UNITS;
        const int unit = (lane % ROW_UNITS) ^ (2 * tsw(k));
        const int col = min(mn0 + unit * 8, lim - 8);
        off[i] = (uint32_t)((long)k * ld + col);
        if (unit * 8 < VALID) live |= 1u << i;
      }
    }
  }
  // base: operand origin advanced to the tile's first k
  __device__ __forceinline__ void issue(const bf16_t* base, uint4* lds, int wave) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) issue_one(base, lds, wave, i);
  }
  __device__ __forceinline__ void issue_one(const bf16_t* base, uint4* lds, int wave, int i) const {
    if (VALID == R || ((live >> i) & 1u)) load_lds16(base, off[i] * 2u, lds + (wave * PER_WAVE + i) * 64);
  }
  __device__ __forceinline__ static const bf16_t* advance(const bf16_t* base, long ld, int k) {
    return KMAJ ? base + k : base + (long)k * ld;
  }
  // Fragment for rows [r0, r0 + 32) and k [16 ks, 16 ks + 16): lane l gets
  // row r0 + l % 32, k = 16 ks + 8 (l / 32) + (0..7).
  __device__ __forceinline__ uint4 frag(const uint4* lds, int r0, int ks, int lane) const {
    if constexpr (KMAJ) {
      const int row = r0 + (lane & 31);
      return lds[row * 8 + ((2 * ks + (lane >> 5)) ^ kswz(row))];
    } else {
      const int g = lane >> 4, i = lane & 15;
      const int col = r0 + 16 * (g & 1) + 4 * (i & 3);
      const int kb = 16 * ks + 8 * (g >> 1) + (i >> 2);
      uint2 lo, hi;
      {
        const int k = kb;
        lo = read_tr(lds, (uint32_t)(k * R * 2 + (((col >> 3) ^ (2 * tsw(k))) << 4) + 2 * (col & 7)));
      }
      {
        const int k = kb + 4;
        hi = read_tr(lds, (uint32_t)(k * R * 2 + (((col >> 3) ^ (2 * tsw(k))) << 4) + 2 * (col & 7)));
      }
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
};

// Width of the LDS layout of a B tile. An N-contiguous B tile of 192 columns
// is laid out as 256 (a 384-byte row fits neither the whole-rows-per-load-
// instruction mapping nor the segment swizzle); only its 192 columns are
// loaded and read.
template <bool BKM, int BN>
__host__ __device__ constexpr int b_load_cols() {
  return (!BKM && BN == 192) ? 256 : BN;
}

// One output tile: linear tile index L (ordered by tile_coords), split-K
// piece `split`, batch z. LDS buffers are passed in (two per operand).
// EPI_SK_PART: K range [kb_, ke_) and the fp32 fragment goes to skdst as a
// row-major BM x BN tile.
// CSUM: the tile also sums its B operand over its whole K range, column by
// column (p.csum[n] = sum over k of B[k, n], rounded once to bf16): a bias
// gradient is the column sum of the weight-gradient GEMM's right operand
// (db = sum over tokens of dY, with dW = X^T dY), so the tiles of tile-row 0
// produce it from the B fragments they already hold. Each lane holds 8
// consecutive k of one column per fragment and adds them with two-element
// bf16 dot products against (1, 1) in a fixed order; lanes l and l + 32
// hold the two k halves of a column and are added at the end.
template <class Cfg, bool AK, bool BKM, int EPI, typename TO, int KSEG, bool CSUM = false>
__device__ __forceinline__ void direct_tile(const GemmArgs& p, int L, int split, int z, uint4* sa0, uint4* sb0,
                                            uint4* sa1, uint4* sb1, int kb_ = 0, int ke_ = 0,
                                            float* skdst = nullptr) {
  static_assert(sizeof(typename Cfg::T) == 2, "direct path is bf16");
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT, BK = 64;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, WTM = Cfg::WTM, WTN = Cfg::WTN;
  using OA = DirectOperand<AK, BM, NT>;
  using OB = DirectOperand<BKM, b_load_cols<BKM, BN>(), NT, BN>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WN, wn = wave - (wave / Cfg::WN) * Cfg::WN;

  int tm, tn;
  tile_coords(p, tm, tn, L);
  const int m0 = tm * BM, n0 = tn * BN;
  const int z1 = z / p.zdiv, z2 = z - (z / p.zdiv) * p.zdiv;
  const long aoff = z1 * p.a_s1 + z2 * p.a_s2, boff = z1 * p.b_s1 + z2 * p.b_s2;
  const bf16_t* A = static_cast<const bf16_t*>(p.A) + aoff;
  const bf16_t* B = static_cast<const bf16_t*>(p.B) + boff;

  OA oa;
  OB ob;
  oa.init(p.lda, m0, p.M, wave, lane);
  ob.init(p.ldb, n0, p.N, wave, lane);

  int kb = 0, ke = p.K, nk, nkd = 1;
  if constexpr (KSEG > 1) {
    nkd = p.kseg_len / BK;
    nk = KSEG * nkd;
  } else {
    if (p.kmode == K_LOWER) ke = min(ke, m0 + BM);
    else if (p.kmode == K_UPPER) kb = m0;
    if constexpr (EPI == EPI_PARTIAL) {
      kb = split * p.k_chunk;
      ke = min(ke, kb + p.k_chunk);
    } else if constexpr (EPI == EPI_SK_PART) {
      kb = kb_;
      ke = ke_;
    }
    nk = ke > kb ? (ke - kb) / BK : 0;
  }
  auto next_ptrs = [&](int kt, const bf16_t*& a, const bf16_t*& b) {
    if constexpr (KSEG > 1) {
      const int seg = kt / nkd;
      const int k0 = (kt - seg * nkd) * BK;
      a = OA::advance(seg == 2 ? static_cast<const bf16_t*>(p.A2) + aoff : A, p.lda, k0);
      b = OB::advance(seg == 1 ? static_cast<const bf16_t*>(p.B2) + boff : B, p.ldb, k0);
    } else {
      const int k0 = kb + kt * BK;
      a = OA::advance(A, p.lda, k0);
      b = OB::advance(B, p.ldb, k0);
    }
  };
  auto issue = [&](int kt, uint4* la, uint4* lb) {
    const bf16_t *a, *b;
    if constexpr (KSEG > 1) {
      const int seg = kt / nkd;
      const int k0 = (kt - seg * nkd) * BK;
      a = OA::advance(seg == 2 ? static_cast<const bf16_t*>(p.A2) + aoff : A, p.lda, k0);
      b = OB::advance(seg == 1 ? static_cast<const bf16_t*>(p.B2) + boff : B, p.ldb, k0);
    } else {
      const int k0 = kb + kt * BK;
      a = OA::advance(A, p.lda, k0);
      b = OB::advance(B, p.ldb, k0);
    }
    oa.issue(a, la, wave);
    ob.issue(b, lb, wave);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Main loop. A K tile is four 16-deep sub-steps of MF = TM x TN MFMAs per
  // wave. Each sub-step is written out as MF slots in program order, one
  // MFMA per slot, with a scheduling barrier after each slot: the next
  // sub-step's NR fragment reads (A, then B) are spread one per slot at a
  // stride of MF / NR, and the global->LDS loads of the next tile one per
  // slot at a stride of MF / DPS, half a stride later. Fragment registers
  // alternate between two sets by sub-step, so every read has a whole
  // sub-step of MFMAs to land.
  //
  // Software pipeline across the per-tile barrier: the first DPS loads of
  // tile kt + 1 go out during sub-step 3 of tile kt - 1 (right after that
  // tile's barrier, into the buffers it has just freed), the other NLD - DPS
  // during sub-step 0 of tile kt. Sub-step 3 of tile kt runs after the
  // barrier, while the first fragment reads of tile kt + 1 are in flight.
  constexpr int MF = TM * TN;
  uint4 af[2][TM], bq[2][TN];
  auto read_frags = [&](const uint4* As, const uint4* Bs, int ks, int set) {
#pragma unroll
    for (int i = 0; i < TM; ++i) af[set][i] = oa.frag(As, wm * WTM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) bq[set][j] = ob.frag(Bs, wn * WTN + j * 32, ks, lane);
  };
  constexpr int NLD = OA::PER_WAVE + OB::PER_WAVE;  // global->LDS loads per tile and wave
  constexpr int NR = TM + TN, DPS = (NLD + 1) / 2;
  float cs[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) cs[j] = 0.0f;
  auto slot_step = [&](int set_mma, const uint4* Ar, const uint4* Br, int ks_rd, int set_rd, int dq0,
                       const bf16_t* na, const bf16_t* nb, uint4* la, uint4* lb) {
#pragma unroll
    for (int q = 0; q < MF; ++q) {
      const int j = q / TM, i = q - (q / TM) * TM;
      mma16(bq[set_mma][j], af[set_mma][i], acc[i][j], bf16_t{});
      if constexpr (CSUM) {
        if (i == 0) cs[j] = colsum8(bq[set_mma][j], cs[j]);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if ((r * MF) / NR == q) {
          if (r < TM) af[set_rd][r] = oa.frag(Ar, wm * WTM + r * 32, ks_rd, lane);
          else bq[set_rd][r - TM] = ob.frag(Br, wn * WTN + (r - TM) * 32, ks_rd, lane);
        }
      }
#pragma unroll
      for (int e = 0; e < DPS; ++e) {
        if ((e * MF) / DPS + MF / DPS / 2 == q) {
          const int d = dq0 + e;
          if (d < OA::PER_WAVE) oa.issue_one(na, la, wave, d);
          else if (d < NLD) ob.issue_one(nb, lb, wave, d - OA::PER_WAVE);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Past the last tile the prefetch repeats the last tile into the idle
  // buffer (in bounds, never read), keeping the loop free of divergence.
  if (nk > 0) issue(0, sa0, sb0);
  wait_loads();
  __syncthreads();
  if (nk > 1) {
    const bf16_t *na, *nb;
    next_ptrs(1, na, nb);
#pragma unroll
    for (int d = 0; d < DPS; ++d) {
      if (d < OA::PER_WAVE) oa.issue_one(na, sa1, wave, d);
      else if (d < NLD) ob.issue_one(nb, sb1, wave, d - OA::PER_WAVE);
    }
  }
  if (nk > 0) read_frags(sa0, sb0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const bool odd = kt & 1;
    const uint4* As = odd ? sa1 : sa0;
    const uint4* Bs = odd ? sb1 : sb0;
    uint4* An = odd ? sa0 : sa1;
    uint4* Bn = odd ? sb0 : sb1;
    const bf16_t *na, *nb;
    next_ptrs(min(kt + 1, nk - 1), na, nb);
    slot_step(0, As, Bs, 1, 1, DPS, na, nb, An, Bn);
    slot_step(1, As, Bs, 2, 0, NLD, na, nb, An, Bn);
    slot_step(0, As, Bs, 3, 1, NLD, na, nb, An, Bn);
    wait_loads();
    __syncthreads();
    next_ptrs(min(kt + 2, nk - 1), na, nb);
    // (near the end the clamped index repeats tile nk - 1 into a buffer no
    // later fragment read uses; in bounds, drained after the loop)
    slot_step(1, An, Bn, 0, 0, 0, na, nb, const_cast<uint4*>(As), const_cast<uint4*>(Bs));
  }
  wait_loads();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (CSUM) {
    // waves of the first wave-row hold every column of the tile once
    if (wm == 0 && tm == 0) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const float v = cs[j] + __shfl_xor(cs[j], 32);
        const int col = n0 + wn * WTN + j * 32 + lane;
        if (lane < 32 && col < p.N) static_cast<bf16_t*>(p.csum)[col] = f2bf(v);
      }
    }
  }

  // bf16 output of the plain epilogue (no residual term): scale and bias are
  // applied in registers and the tile is staged through LDS already rounded
  // to bf16, two 32-row blocks of every wave per pass (half the LDS traffic
  // and half the passes of the fp32 staging below; the same operations and
  // the same single rounding per element). 16-byte chunk q of staged row r
  // sits at chunk q ^ (r mod C16), so the 32 rows a write instruction
  // touches, and the chunks of one row that a read instruction takes, fall
  // on distinct banks.
  if constexpr (EPI == EPI_LINEAR && std::is_same<TO, bf16_t>::value && TM % 2 == 0) {
    if (!p.resid) {
      constexpr int C16 = BN / 8;            // 16-byte chunks per staged row
      constexpr int PR2 = 2 * Cfg::WM * 32;  // rows staged per pass
      constexpr int PER2 = PR2 * C16 / NT;   // chunks per thread and pass
      // (XOR with a mask below the largest power of two dividing C16 keeps a
      // chunk inside its row)
      constexpr int XM = (C16 & (C16 - 1)) == 0 ? C16 - 1 : (C16 % 16 == 0 ? 15 : 7);
      static_assert(C16 % (XM + 1) == 0 && (PR2 * C16) % NT == 0, "bf16 staging layout");
      static_assert(PR2 * BN * 2 <= 2 * (BM + BN) * 128, "staging must fit the operand buffers");
      __syncthreads();  // every wave is past its last fragment read and LDS load
      unsigned char* const st8 = reinterpret_cast<unsigned char*>(sa0);
      const int r32 = lane & 31, g = lane >> 5;
      bf16_t* const C = static_cast<bf16_t*>(p.C) + z1 * p.c_s1 + z2 * p.c_s2;
      // (the scale and bias are uniform: with neither, the pass is a
      // conversion and one 8-byte LDS write per 4 values, without the
      // per-element selects and guarded bias loads of the general form)
      const bool plain = p.alpha == 1.0f && !p.bias;
      const bool full = m0 + BM <= p.M && n0 + BN <= p.N;
      // Whole tile, no scale or bias: every wave stages its own WTM x WTN
      // block in a region of its own and stores it from there, with no
      // further barrier (LDS operations of one wave complete in order).
      // Row r of a wave's block is WTN * 2 bytes, its 16-byte chunk q at
      // q ^ (r mod 16); a read instruction takes whole row segments.
      constexpr int WC = WTN / 8;  // 16-byte chunks per row of a wave's block
      if constexpr (WTM * WTN * 2 * (NT / 64) <= 2 * (BM + BN) * 128 && WC % 16 == 0) {
        if (plain && full) {
          unsigned char* const wst = st8 + wave * (WTM * WTN * 2);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const int r = i * 32 + r32;
                float v[4] = {acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2], acc[i][j][4 * jj + 3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(v[e]));
                const f32x4_t x = {v[0], v[1], v[2], v[3]};
                *reinterpret_cast<bf16x4_t*>(wst + r * (WTN * 2) + (((4 * j + jj) ^ (r & 15)) << 4) + 8 * g) =
                    __builtin_convertvector(x, bf16x4_t);
              }
          constexpr int RPI = 64 / WC;             // rows per read instruction
          constexpr int NRD = WTM * WC / 64;       // reads (and stores) per lane
          const int q = lane % WC, rq = lane / WC;
          bf16_t* const Cw = C + (long)(m0 + wm * WTM) * p.ldc + n0 + wn * WTN + 8 * q;
          auto rd = [&](int k) {
            const int r = k * RPI + rq;
            return *reinterpret_cast<const uint4*>(wst + r * (WTN * 2) + ((q ^ (r & 15)) << 4));
          };
          uint4 x = rd(0);
#pragma unroll
          for (int k = 0; k < NRD; ++k) {
            uint4 x1;
            if (k + 1 < NRD) x1 = rd(k + 1);
            *reinterpret_cast<uint4*>(Cw + (long)(k * RPI + rq) * p.ldc) = x;
            __builtin_amdgcn_sched_barrier(0);
            x = x1;
          }
          return;
        }
      }
      auto write_pass = [&](int pp, auto general) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ps = 2 * pp + h, rl = h * (Cfg::WM * 32) + wm * 32 + r32;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int cb = wn * WTN + j * 32 + jj * 8;  // the lane's 4 columns: cb + 4 g ..
              float v[4] = {acc[ps][j][4 * jj], acc[ps][j][4 * jj + 1], acc[ps][j][4 * jj + 2],
                            acc[ps][j][4 * jj + 3]};
              // (copied out here, so that the accumulators themselves are
              // used only by MFMAs and stay in the accumulation registers)
#pragma unroll
              for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(v[e]));
              if constexpr (decltype(general)::value) {
                if (p.alpha != 1.0f) {
#pragma unroll
                  for (int e = 0; e < 4; ++e) v[e] *= p.alpha;
                }
                if (p.bias && n0 + cb + 4 * g < p.N) {
                  float bb[4];
                  loadv<bf16_t, 4>(static_cast<const bf16_t*>(p.bias) + n0 + cb + 4 * g, bb);
#pragma unroll
                  for (int e = 0; e < 4; ++e) v[e] += bb[e];
                }
              }
              const f32x4_t x = {v[0], v[1], v[2], v[3]};
              *reinterpret_cast<bf16x4_t*>(st8 + rl * (BN * 2) + (((cb >> 3) ^ (rl & XM)) << 4) + 8 * g) =
                  __builtin_convertvector(x, bf16x4_t);
            }
        }
      };
#pragma unroll
      for (int pp = 0; pp < TM / 2; ++pp) {
        if (plain) write_pass(pp, std::false_type{});
        else write_pass(pp, std::true_type{});
        __syncthreads();
        auto chunk = [&](int k, int& row, int& col) {
          const int c = tid + k * NT;
          const int rs = c / C16, q = c - (c / C16) * C16;
          const int h = rs / (Cfg::WM * 32), r = rs - h * (Cfg::WM * 32);
          row = m0 + (r >> 5) * WTM + (2 * pp + h) * 32 + (r & 31);
          col = n0 + 8 * q;
          return *reinterpret_cast<const uint4*>(st8 + rs * (BN * 2) + ((q ^ (rs & XM)) << 4));
        };
        if (full) {
          // whole tile: no guards; one LDS read ahead of each store (a
          // burst of all the pass's stores at once runs slower)
          int row, col;
          uint4 x = chunk(0, row, col);
#pragma unroll
          for (int k = 0; k < PER2; ++k) {
            int row1 = 0, col1 = 0;
            uint4 x1;
            if (k + 1 < PER2) x1 = chunk(k + 1, row1, col1);
            *reinterpret_cast<uint4*>(C + (long)row * p.ldc + col) = x;
            __builtin_amdgcn_sched_barrier(0);
            x = x1;
            row = row1;
            col = col1;
          }
        } else {
#pragma unroll
          for (int k = 0; k < PER2; ++k) {
            int row, col;
            const uint4 x = chunk(k, row, col);
            if (row < p.M && col < p.N) *reinterpret_cast<uint4*>(C + (long)row * p.ldc + col) = x;
          }
        }
        if (pp + 1 < TM / 2) __syncthreads();
      }
      return;
    }
  }

  // Epilogue through LDS. Stored straight from the MFMA layout, a lane holds
  // 4 columns of one row and a store instruction touches 32 rows, which
  // serialises on the memory channel whenever the row pitch is a large power
  // of two (every layer output). Instead the tile goes through LDS in TM
  // passes: pass ps stages the 32-row block i = ps of every wave (fp32,
  // 16-byte chunks XOR-swizzled by row), then each lane takes 8 consecutive
  // columns of one row, so global loads and stores are 16-32 byte pieces of
  // contiguous row segments.
  constexpr int CH = BN / 4;          // 16-byte fp32 chunks per staged row
  constexpr int C8 = BN / 8;          // 8-column chunks per row
  constexpr int PR = Cfg::WM * 32;    // rows staged per pass
  constexpr int PER = PR * C8 / NT;   // 8-column chunks per thread and pass
  static_assert(CH >= 16 && (PR * C8) % NT == 0, "staging layout");
  static_assert(PR * BN * 4 <= 2 * (BM + BN) * 128, "staging must fit the operand buffers");
  __syncthreads();  // every wave is past its last fragment read and LDS load
  float4* stage = reinterpret_cast<float4*>(sa0);
  const int r32 = lane & 31, g = lane >> 5;
  // Bias epilogues: the bias of a thread's chunks is loaded once, here, rather
  // than once per chunk behind each chunk's LDS read. Chunk k of a thread sits
  // in the same 8 columns in every pass; when NT is a multiple of the chunks
  // per row, all of a thread's chunks do (one set, else PER).
  constexpr bool PRE_BIAS = EPI == EPI_BIAS_SPLIT || EPI == EPI_BIAS_GELU;
  constexpr int NBQ = PRE_BIAS ? (NT % C8 == 0 ? 1 : PER) : 1;
  float bia[NBQ][8];
  if constexpr (PRE_BIAS) {
#pragma unroll
    for (int k = 0; k < NBQ; ++k)
      loadv<bf16_t, 8>(static_cast<const bf16_t*>(p.bias) + min(n0 + 8 * ((tid + k * NT) % C8), p.N - 8), bia[k]);
  }
#pragma unroll
  for (int ps = 0; ps < TM; ++ps) {
    const int rl = wm * 32 + r32;
    // GELU backward: the pass's U values are loaded ahead of the staging, so
    // that their latency passes under it (rows and columns clamped into the
    // matrix; the stores below stay guarded)
    uint4 ux[EPI == EPI_GELU_BWD ? PER : 1];
    if constexpr (EPI == EPI_GELU_BWD) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int c = tid + k * NT;
        const int rs = c / C8, q = c - (c / C8) * C8;
        const int row = min(m0 + (rs >> 5) * WTM + ps * 32 + (rs & 31), p.M - 1), col = min(n0 + 8 * q, p.N - 8);
        ux[k] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(p.aux) + (long)row * p.ldx + col);
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int ch = (wn * WTN + j * 32 + jj * 8) / 4 + g;
        stage[rl * CH + (ch ^ (rl & 15))] =
            make_float4(acc[ps][j][4 * jj], acc[ps][j][4 * jj + 1], acc[ps][j][4 * jj + 2], acc[ps][j][4 * jj + 3]);
      }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int c = tid + k * NT;
      const int rs = c / C8, q = c - (c / C8) * C8;
      const float4 x0 = stage[rs * CH + ((2 * q) ^ (rs & 15))];
      const float4 x1 = stage[rs * CH + ((2 * q + 1) ^ (rs & 15))];
      float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const int rt = (rs >> 5) * WTM + ps * 32 + (rs & 31);  // row within the tile
      if constexpr (EPI == EPI_SK_PART) {
        storev<float, 8>(skdst + rt * BN + 8 * q, v);  // the unit's fragment, tile-row-major
      } else if constexpr (EPI == EPI_GELU_BWD) {
        const int row = m0 + rt, col = n0 + 8 * q;
        if (row < p.M && col < p.N) {
          const uint32_t w[4] = {ux[k].x, ux[k].y, ux[k].z, ux[k].w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            v[e] *= gelu_grad_f(__uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16)));
          storev<TO, 8>(static_cast<TO*>(p.C) + z1 * p.c_s1 + z2 * p.c_s2 + (long)row * p.ldc + col, v);
        }
      } else if constexpr (PRE_BIAS) {
        const int row = m0 + rt, col = n0 + 8 * q;
        if (row < p.M && col < p.N) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += bia[NBQ == 1 ? 0 : k][e];
          if constexpr (EPI == EPI_BIAS_GELU) {
            float gv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[e] = gelu_f(v[e]);
            storev<bf16_t, 8>(static_cast<bf16_t*>(p.C2) + (long)row * p.ldc2 + col, gv);
          } else if (col < p.c2_cols) {
            float lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) lo[e] = v[e] - bf2f(f2bf(v[e]));
            storev<bf16_t, 8>(static_cast<bf16_t*>(p.C2) + (long)row * p.ldc2 + col, lo);
          }
          storev<TO, 8>(static_cast<TO*>(p.C) + z1 * p.c_s1 + z2 * p.c_s2 + (long)row * p.ldc + col, v);
        }
      } else {
        const int row = m0 + rt, col = n0 + 8 * q;
        if (row < p.M && col < p.N) epi_apply<EPI, bf16_t, TO, 8>(p, z1, z2, row, col, v, split);
      }
    }
    if (ps + 1 < TM) __syncthreads();
  }
}

// Two K-tile buffers per operand in one contiguous array (the epilogue
// stages the output tile across them).
#define TPL_DIRECT_LDS(BM, BN)                                              \
  __shared__ __attribute__((aligned(1024))) uint4 lds_[2 * ((BM) + (BN)) * 8]; \
  uint4* const sa0 = lds_;                                                  \
  uint4* const sb0 = lds_ + (BM) * 8;                                       \
  uint4* const sa1 = lds_ + ((BM) + (BN)) * 8;                              \
  uint4* const sb1 = lds_ + (2 * (BM) + (BN)) * 8;

template <class Cfg, bool AK, bool BKM, int EPI, typename TO, int ROLE, int KSEG = 1>
__global__ void __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::NT / 256, Cfg::NT / 256)))
gemm_direct_kernel(const GemmArgs p) {
  TPL_DIRECT_LDS(Cfg::BM, (b_load_cols<BKM, Cfg::BN>()))
  direct_tile<Cfg, AK, BKM, EPI, TO, KSEG>(p, blockIdx.x, blockIdx.y, blockIdx.z, sa0, sb0, sa1, sb1);
}

// Stream-K launch (plan in SkPlan). Consecutive blocks go to different XCDs,
// so block b is remapped to (b mod 8) * (n / 8) + b / 8: each XCD takes one
// contiguous run of whole tiles and one contiguous run of stream-K units,
// and the tiles of a run share operand panels in that XCD's L2.
template <class Cfg, bool AK, bool BKM, int EPI, typename TO, int ROLE>
__global__ void __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::NT / 256, Cfg::NT / 256)))
gemm_sk_kernel(const GemmArgs p, const SkPlan s) {
  TPL_DIRECT_LDS(Cfg::BM, Cfg::BN)
  const int b = blockIdx.x;
  if (b < s.dp_tiles) {
    const int L = (b & 7) * (s.dp_tiles >> 3) + (b >> 3);
    direct_tile<Cfg, AK, BKM, EPI, TO, 1>(p, L, 0, 0, sa0, sb0, sa1, sb1);
    return;
  }
  const int sb = b - s.dp_tiles;
  const int u = (sb & 7) * (s.units >> 3) + (sb >> 3);
  const long total = (long)s.sk_tiles * s.iters;
  long it = (long)u * s.c;
  const long end = min(it + s.c, total);
  while (it < end) {
    const int j = (int)(it / s.iters);
    const int k0 = (int)(it - (long)j * s.iters);
    const int k1 = (int)min((long)s.iters, k0 + (end - it));
    const int slot = u - (int)(((long)j * s.iters) / s.c);
    float* dst = s.part + ((long)j * s.f + slot) * (long)(Cfg::BM * Cfg::BN);
    direct_tile<Cfg, AK, BKM, EPI_SK_PART, float, 1>(p, s.dp_tiles + j, 0, 0, sa0, sb0, sa1, sb1,
                                                                   k0 * 64, k1 * 64, dst);
    it += k1 - k0;
    __syncthreads();  // the next run's first loads reuse this run's LDS buffers
  }
}

// Stream-K fix-up: for each tile of the stream-K region, the fixed-order sum
// of its fragments (each stored tile-row-major), then the epilogue. Eight
// consecutive columns of one row per thread.
template <class Cfg, int EPI, typename TO, int ROLE>
__global__ void __launch_bounds__(256) sk_fixup_kernel(const GemmArgs p, const SkPlan s) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, C8 = BN / 8;
  const int j = blockIdx.y;
  const int q = blockIdx.x * 256 + threadIdx.x;  // 8-column chunk within the tile
  const int rt = q / C8, ct = 8 * (q - (q / C8) * C8);
  int tm, tn;
  tile_coords(p, tm, tn, s.dp_tiles + j);
  const int row = tm * BM + rt, col = tn * BN + ct;
  if (rt >= BM || row >= p.M || col >= p.N) return;
  const int uf = (int)(((long)j * s.iters) / s.c), ul = (int)(((long)(j + 1) * s.iters - 1) / s.c);
  const float* src = s.part + (long)j * s.f * (BM * BN) + (long)rt * BN + ct;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // fragments in slot order, two loads in flight per step
  const int nf = ul - uf + 1;
  int k = 0;
  for (; k + 2 <= nf; k += 2) {
    float x[8], y[8];
    loadv<float, 8>(src + (long)k * (BM * BN), x);
    loadv<float, 8>(src + (long)(k + 1) * (BM * BN), y);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (v[e] + x[e]) + y[e];
  }
  if (k < nf) {
    float x[8];
    loadv<float, 8>(src + (long)k * (BM * BN), x);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += x[e];
  }
  epi_apply<EPI, bf16_t, TO, 8>(p, 0, 0, row, col, v, 0);
}

// Operand layouts and epilogue of one problem of a grouped launch.
template <bool AK_, bool BK_, int EPI_, typename TO_>
struct GemmKind {
  static constexpr bool AK = AK_, BK = BK_;
  static constexpr int EPI = EPI_;
  using TO = TO_;
};

// Two independent GEMMs in one launch (a block's weight-gradient and input-
// gradient products). Problem 0 has units0 = tiles0 x splits blocks (tile-
// major over its split-K pieces), problem 1 tiles1 blocks; first1 selects
// which problem's blocks come first. The host puts the longer K per tile
// first, so the long tiles start first and the short ones fill in around
// them (longest-processing-time order over the 256 CUs).
template <class Cfg, class K0, class K1, int ROLE>
__global__ void __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::NT / 256, Cfg::NT / 256)))
gemm_pair_kernel(const GemmArgs p0, const GemmArgs p1, int tiles0, int units0, int tiles1, int first1) {
  TPL_DIRECT_LDS(Cfg::BM, Cfg::BN)
  // blocks of the problem that goes first come first
  int u = blockIdx.x;
  const bool is0 = first1 ? (u >= tiles1) : (u < units0);
  if (first1) u = is0 ? u - tiles1 : u + units0;
  if (is0) {
    const int split = u / tiles0;
    direct_tile<Cfg, K0::AK, K0::BK, K0::EPI, typename K0::TO, 1>(p0, u - split * tiles0, split, 0, sa0,
                                                                                 sb0, sa1, sb1);
  } else {
    const int L = u - units0;
    int tm, tn;
    tile_coords(p1, tm, tn, L);
    if (p1.csum && tm == 0)
      direct_tile<Cfg, K1::AK, K1::BK, K1::EPI, typename K1::TO, 1, true>(p1, L, 0, 0, sa0, sb0, sa1, sb1);
    else
      direct_tile<Cfg, K1::AK, K1::BK, K1::EPI, typename K1::TO, 1>(p1, L, 0, 0, sa0, sb0, sa1, sb1);
  }
}

}  // namespace tpl
