// Newton-Schulz GEMM kernels of the Muon step (gfx950): the symmetric Gram
// A = X X^T, C = a I + b A + c A A, and the X update X' = C X, as templates
// over the output tile size.  muon_gemm256.hip and muon_gemm128.hip each
// instantiate one tile size.
//
// The iteration is the newtonschulz5 routine of "Muon optimizer: matrix-aware
// LLM" (airosetta.com, implementation section), in the expanded polynomial
// form of "AdamW vs Muon" (adg.csdn.net, section "2. Newton-Schulz
// iteration").
#pragma once
#include <hip/hip_runtime.h>
#include <utility>
#include <stdint.h>

#include "muon_device.h"

namespace muon {

// ---------------------------------------------------------------------------
// Newton-Schulz GEMM engine on bf16 MFMA (v_mfma_f32_16x16x32_bf16)
//
// Output tile TILE x TILE (128 or 256), 4 waves in a 2 x 2 grid, each wave
// (TILE/2) x (TILE/2) = NB x NB MFMA blocks of 16 x 16 with fp32
// accumulators (256 of them per lane at TILE = 256, held in AGPRs).
//
// Operand tiles of K step 32 go straight from global memory into a ring of
// four LDS stages (16 bytes per lane, no registers, no LDS store
// instructions), three steps ahead of their use.  One step is one 32-deep
// MFMA substep; its fragments were read during the previous step, so the
// MFMAs never wait for LDS, and the fragments of the next step are read in
// the first slots of this one.  One barrier per step.  With no staging
// registers the fragments of two steps fit beside the accumulators, and the
// 16 x 16 x 32 shape needs only two fresh 16-row fragments per instruction.
//
// An operand is "K-contiguous" (element (mn, k) at p[mn * ld + k]) or
// "MN-contiguous" (element (mn, k) at p[k * ld + mn]).
//   K-contiguous tiles sit in LDS as [mn][32 k] (64-byte rows); fragments
//     are 16-byte reads; the 16-byte chunk c of row r is stored at
//     c ^ (2 ((r >> 3) & 1)).
//   MN-contiguous tiles keep their memory layout, [k][TILE mn]; fragments
//     are assembled by the LDS transpose read (ds_read_b64_tr_b16: in each
//     16-lane group, lane 4a + b receives element b of the 8-byte blocks
//     addressed by lanes a, a + 4, a + 8, a + 12), so the transpose of a tall
//     matrix is never materialised.  The 16-byte chunk c of k row r is
//     stored at c ^ (2 (r & 3) + 8 ((r >> 3) & 1)).
// Both swizzles follow how the gfx950 LDS (64 banks of 4 bytes) serves the
// two read forms, as measured with its bank-conflict counter: a 16-byte
// read takes each half-wave in two cycles, lanes {0-3, 8-11, 20-23, 28-31}
// then {4-7, 12-15, 16-19, 24-27} (mod 32); a transposing 8-byte read
// takes 32 consecutive lanes per cycle.  For a fragment (lane l: row
// l & 15, chunk l >> 4; or k rows 8 (l >> 4) + (l & 15) / 4 for the
// transpose) each cycle then touches every bank once.
// ---------------------------------------------------------------------------
constexpr int BK = 32;
constexpr int kStages = 4;

template <int TILE>
struct Geo {
  static constexpr int T = TILE;
  static constexpr int WT = TILE / 2;      // wave tile
  static constexpr int NB = WT / 16;       // 16x16 MFMA blocks per wave side
  static constexpr int TE = TILE * BK;     // bf16 elements of one staged operand tile
  static constexpr int LPW = TILE / 64;    // 1 KB direct loads per wave per operand tile
  static constexpr int LDS = kStages * 2 * TE * 2;  // bytes
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N global -> LDS loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

struct Opnd {
  const uint16_t* p;
  int64_t ld;
};

// The work-item index as a value the compiler cannot re-derive: the lane-
// dependent LDS and global offsets are then formed once per tile and kept in
// registers, instead of being recomputed from the index inside the K loop
// (6-7 vector ALU instructions per 64 MFMAs instead of 33-35 where both
// operands are K-contiguous; 1-3 % on the Gram, C and X-update launches).
__device__ __forceinline__ int opaque_tid() {
  int t = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

// Global -> LDS, 16 bytes per lane, without registers: lane l's 16 bytes at
// sbase + voff land at LDS byte 16 l of the 1 KB block at lds_dst.  Written
// as a one-line asm statement: it writes only LDS (no register results),
// and the compiler would otherwise assume every later LDS read may alias
// these writes and wait for all of them.  Ordering is explicit instead:
// vm_wait<> on the issuing wave, then an LDS barrier, before any wave reads
// the stage.  The scalar base is wave-uniform by construction.
// Wait states: on gfx9 a memory instruction that reads a scalar register
// written by a vector instruction (v_readfirstlane_b32) must come 5 wait
// states after it.  The compiler pads its own loads for this but not an asm
// statement, and a load issued early takes the register's previous contents
// as its address.  So every caller forms `sbase` from scalar values (kernel
// arguments, block index, descriptor fields, a wave index taken through
// readfirstlane once, up front), and the readfirstlane below then folds away;
// tests/test_isa_hazards.py checks the compiled kernels for it.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint16_t* lds_dst) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) void*)lds_dst));
  // the base is wave-uniform; readfirstlane lets the compiler see it (and
  // folds away when the value already sits in scalar registers)
  // (readfirstlane returns int: each half goes back to uint32_t before it
  // is widened, or a low word with bit 31 set would sign-extend)
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint64_t u = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(reinterpret_cast<const char*>(u)),
               "{m0}"(m0));
}

// This wave's share of one operand's TILE x 32 tiles: LPW blocks of 1 KB per
// K step (block b of the tile belongs to wave b / LPW).  Block q of step kt
// is read at the wave-uniform base + kt kstep + q qstride plus a per-lane
// 32-bit offset, so the loads need one or two address registers in all.
//   K-contiguous: a block is 16 rows of 64 bytes; lane l reads row l / 4,
//     chunk (l % 4) ^ (2 ((row >> 3) & 1)) (the stored swizzle; the XOR term
//     depends on l only, since blocks start at multiples of 16 rows).
//   MN-contiguous: a block is 512 / TILE k rows of 2 TILE bytes; lane l reads
//     k row r = R b + l / CPR, chunk (l % CPR) ^ (2 (r & 3) + 8 ((r >> 3) & 1));
//     bit 3 of r is the parity of the wave, and at TILE = 256 r & 3 also
//     depends on the parity of the block: two offsets.
template <bool MN, int TILE>
struct DmaFeed {
  static constexpr int LPW = Geo<TILE>::LPW;
  const char* base;
  int64_t qstride, kstep;
  uint32_t voff[2];
  int w;
  __device__ __forceinline__ DmaFeed(const Opnd& op, int64_t mn0, int tid) {
    const int lane = tid & 63;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t ldb = op.ld * 2;
    const char* p = reinterpret_cast<const char*>(op.p);
    if constexpr (!MN) {
      const int row = lane >> 2, c = (lane & 3) ^ (2 * ((row >> 3) & 1));
      voff[0] = voff[1] = static_cast<uint32_t>(row * ldb + 16 * c);
      base = p + (mn0 + 16 * LPW * w) * ldb;
      qstride = 16 * ldb;
      kstep = BK * 2;
    } else {
      constexpr int CPR = TILE / 8, R = 512 / TILE;
      const int row = lane / CPR;
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int c = (lane % CPR) ^ (2 * ((R * par + row) & 3) + 8 * (w & 1));
        voff[par] = static_cast<uint32_t>(row * ldb + 16 * c);
      }
      base = p + (R * LPW * w) * ldb + mn0 * 2;
      qstride = R * ldb;
      kstep = BK * ldb;
    }
  }
  // block q of step kt into the operand tile at `tile`
  __device__ __forceinline__ void load(int64_t kt, int q, uint16_t* tile) const {
    dma16(base + kt * kstep + q * qstride, voff[q & 1], tile + (w * LPW + q) * 512);
  }
};

// MFMA operand fragment: 16 rows from rowbase, k = 0 .. 31 of a staged tile;
// lane l holds row rowbase + (l & 15), k = 8 (l >> 4) .. +7.
template <bool MN, int TILE>
__device__ __forceinline__ bf16x8_t frag(const uint16_t* tile, int rowbase, int lane) {
  if constexpr (!MN) {
    const int row = rowbase + (lane & 15);
    const int c = (lane >> 4) ^ (2 * ((row >> 3) & 1));
    return *reinterpret_cast<const bf16x8_t*>(tile + row * BK + c * 8);
  } else {
    // transpose reads: address lane j of a 16-lane group covers k row
    // k0 + (j >> 2), columns rowbase + 4 (j & 3) .. +3; lane i receives
    // k0 .. k0 + 3 of column rowbase + i
    const int g = lane >> 4, i = lane & 15;
    const int m = rowbase + 4 * (i & 3);
    const int k = 8 * g + (i >> 2);                      // + 4 below; k & 3 == i >> 2
    const int off = (((m >> 3) ^ (2 * (i >> 2) + 8 * (g & 1))) << 3) + (m & 4);
    const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(tile + k * TILE + off));
    const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(tile + (k + 4) * TILE + off));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

template <int NB>
__device__ __forceinline__ void zero_acc(f32x4_t (&acc)[NB][NB]) {
#pragma unroll
  for (int bi = 0; bi < NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < NB; ++bj)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[bi][bj][r] = 0.f;
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at compile time
// (a 64-slot MFMA body is past what the unroller expands on its own, and
// run-time indices would push the accumulators out of registers).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// acc += P[mp0 : mp0+TILE, :K] * Q[nq0 : nq0+TILE, :K]^T   (K a multiple of 128)
//
// Step kt lives in LDS stage kt mod 4.  Each step walks the NB x NB blocks
// in two passes over halves of the wave's rows (pass p: rows H p .. H p +
// H - 1, H = NB / 2, blocks column by column), one MFMA per slot, order
// pinned with scheduling barriers.  Fragment registers: one A fragment per
// row block and one B fragment per column block, each reloaded right after
// its last use in the step, with at least a pass of lead before it is used:
//   slots 0 .. H-1:            A rows of pass 1 of this step (stage kt)
//   slots H*NB .. H*NB+H-1:    A rows of pass 0 of step kt+1
//   after each column of pass 1: that column's B fragment of step kt+1
//   slots H, H + LSS, ...:     the loads of step kt+3 (spread as LSS says)
// The step opens with a wait for this wave's loads of step kt+1 and an LDS
// barrier: step kt+1 is then visible, and every wave is past its reads of
// step kt-1, so stage (kt+3) mod 4 is free.  Loads past the end re-read the
// last step (never consumed): the body has no branches.
//
// SWAP = true accumulates the transposed blocks (MFMA operands exchanged), so
// each lane ends up holding four consecutive output columns of one row.
template <int TILE, bool PMN, bool QMN, bool SWAP = false>
__device__ __forceinline__ void gemm_tile(const Opnd& P, const Opnd& Q, int64_t mp0, int64_t nq0,
                                          int64_t K, uint16_t* smem,
                                          f32x4_t (&acc)[Geo<TILE>::NB][Geo<TILE>::NB], int tid) {
  using G = Geo<TILE>;
  constexpr int NB = G::NB, H = NB / 2, PASS = H * NB, SLOTS = NB * NB;
  constexpr int LPS = 2 * G::LPW;                                // loads per wave per step
  // load spacing: over the whole step at TILE 256 (the 32 loads per CU and
  // step then never queue up behind each other and hold up the MFMA issue;
  // 1-2 % on the large sets), within the first pass at TILE 128 (where
  // spreading measured no better)
  constexpr int LSS = TILE == 256 ? (SLOTS - H) / LPS : ((PASS - H) / LPS > 0 ? (PASS - H) / LPS : 1);
  static_assert(H + (LPS - 1) * LSS < SLOTS, "load slots exceed the step");
  const int w = tid >> 6, lane = tid & 63;
  const int rowA = G::WT * (w >> 1), rowB = G::WT * (w & 1);
  const DmaFeed<PMN, TILE> fp(P, mp0, tid);
  const DmaFeed<QMN, TILE> fq(Q, nq0, tid);
  bf16x8_t fa[NB], fb[NB];
  const int64_t kt_n = K / BK;
  auto stage = [&](int64_t kt) { return smem + static_cast<int>(kt & (kStages - 1)) * (2 * G::TE); };
  auto load = [&](int64_t kt, int part) {  // part < LPW: P blocks, else Q blocks
    const int64_t kc = kt < kt_n ? kt : kt_n - 1;
    uint16_t* st = stage(kt);
    if (part < G::LPW) fp.load(kc, part, st);
    else fq.load(kc, part - G::LPW, st + G::TE);
  };

#pragma unroll
  for (int kt = 0; kt < kStages - 1; ++kt)
#pragma unroll
    for (int part = 0; part < LPS; ++part) load(kt, part);
  vm_wait<(kStages - 2) * LPS>();
  lds_barrier();
#pragma unroll
  for (int r = 0; r < H; ++r) fa[r] = frag<PMN, TILE>(smem, rowA + 16 * r, lane);
#pragma unroll
  for (int r = 0; r < NB; ++r) fb[r] = frag<QMN, TILE>(smem + G::TE, rowB + 16 * r, lane);

  for (int64_t kt = 0; kt < kt_n; ++kt) {
    vm_wait<LPS>();   // step kt+1 has landed (kt+2 may be in flight)
    lds_barrier();
    const uint16_t* cu = stage(kt);
    const uint16_t* nx = stage(kt + 1);
    static_for<SLOTS>([&](auto sc) __attribute__((always_inline)) {
      constexpr int s = decltype(sc)::value, pass = s / PASS, sp = s % PASS;
      constexpr int bi = pass * H + sp % H, bj = sp / H;
      acc[bi][bj] = SWAP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[bj], fa[bi], acc[bi][bj], 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[bi], fb[bj], acc[bi][bj], 0, 0, 0);
      if constexpr (s < H) fa[H + s] = frag<PMN, TILE>(cu, rowA + 16 * (H + s), lane);
      if constexpr (s >= PASS && s < PASS + H) fa[s - PASS] = frag<PMN, TILE>(nx, rowA + 16 * (s - PASS), lane);
      if constexpr (pass == 1 && sp % H == H - 1) fb[bj] = frag<QMN, TILE>(nx + G::TE, rowB + 16 * bj, lane);
      if constexpr (s >= H && (s - H) % LSS == 0 && (s - H) / LSS < LPS)
        load(kt + kStages - 1, (s - H) / LSS);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  vm_wait<0>();
  lds_barrier();  // every wave is done with every stage
}

// ---------------------------------------------------------------------------
// Symmetric tile epilogue (Gram and C = a I + b A + c A A), tile (ti <= tj).
//
// The bf16 results are staged in LDS column-major, T[col][row], in units of
// four rows (8 bytes) whose unit index is XORed with a 4-bit rotation of the
// column: the 16 columns one staging write covers, and the 4 columns x 4 units
// one transpose read covers, then fall on distinct banks.  From T:
//   the mirror tile (rows of A^T) leaves as coalesced 16-byte rows,
//   the tile itself leaves through transpose reads as 16-byte row pieces.
// A diagonal tile is first made exactly symmetric in LDS (lower half :=
// upper half) and written once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tswz(int col) { return ((col & 3) << 2) | ((col >> 2) & 3); }

template <int TILE>
__device__ __forceinline__ int tpos(int row, int col) {
  return col * TILE + ((((row >> 2) ^ tswz(col)) << 2) | (row & 3));
}

// Write the staged tile T (TILE x TILE, bf16) to out at (r0, c0), and its
// transpose at (c0, r0) when `mirror`.
template <int TILE>
__device__ __forceinline__ void store_staged(const uint16_t* T, uint16_t* out, int64_t ld,
                                             int64_t r0, int64_t c0, bool mirror, int tid) {
  const int t = tid, lane = t & 63, w = t >> 6;
  if (mirror) {  // out[c0 + col][r0 + 8k .. +7] = T[col][8k .. 8k+7]
    constexpr int CPL = TILE / 8;
#pragma unroll 4
    for (int idx = t; idx < TILE * CPL; idx += kGemmThreads) {
      const int col = idx / CPL, k = idx % CPL, f = tswz(col);
      u32x4 v = *reinterpret_cast<const u32x4*>(T + col * TILE + ((2 * k) ^ (f & 14)) * 4);
      if (f & 1) v = u32x4{v.z, v.w, v.x, v.y};
      gst<u32x4>(out + (c0 + col) * ld + r0 + 8 * k, v);
    }
  }
  // out[r0 + rb + i][c0 + cb + 8g .. +7] through two transpose reads per lane:
  // in each 16-lane group, lane i addresses T[cb + 8g + (i >> 2) (+4)][rb + 4 (i & 3)]
  // and receives T[cb + 8g + j (+4)][rb + i], j = 0..3.
  const int g = lane >> 4, i = lane & 15;
  constexpr int NBLK = (TILE / 16) * (TILE / 32);  // blocks of 16 rows x 32 cols
#pragma unroll 2
  for (int blk = w; blk < NBLK; blk += 4) {
    const int rb = (blk / (TILE / 32)) * 16, cb = (blk % (TILE / 32)) * 32;
    const int col = cb + 8 * g + (i >> 2);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(T + tpos<TILE>(rb + 4 * (i & 3), col)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(T + tpos<TILE>(rb + 4 * (i & 3), col + 4)));
    u32x4 v;
    v.x = __builtin_bit_cast(u32x2, lo).x;
    v.y = __builtin_bit_cast(u32x2, lo).y;
    v.z = __builtin_bit_cast(u32x2, hi).x;
    v.w = __builtin_bit_cast(u32x2, hi).y;
    gst<u32x4>(out + (r0 + rb + i) * ld + c0 + cb + 8 * g, v);
  }
}

// Make a staged diagonal tile symmetric: position (row, col), row > col, takes
// the value computed for (col, row).  Works on 4 x 4 blocks: the four 8-byte
// column pieces of the upper block (b, a) are read, transposed in registers
// and written as the columns of the lower block (a, b), a > b; a diagonal
// block keeps its upper half and mirrors it into its lower half.
template <int TILE>
__device__ __forceinline__ void symmetrize(uint16_t* T, int tid) {
  constexpr int U = TILE / 4;                 // 4 x 4 blocks per side
  constexpr int NBLK = U * (U + 1) / 2;       // blocks on or below the diagonal
  for (int idx = tid; idx < NBLK; idx += kGemmThreads) {
    int a = static_cast<int>((sqrtf(8.f * idx + 1.f) - 1.f) * 0.5f);
    if (a * (a + 1) / 2 > idx) --a;
    if ((a + 1) * (a + 2) / 2 <= idx) ++a;
    const int b = idx - a * (a + 1) / 2;      // b <= a
    uint16_t u[4][4];                         // u[j][i] = T(4b + i, 4a + j)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(T + tpos<TILE>(4 * b, 4 * a + j));
      u[j][0] = v.x & 0xffff; u[j][1] = v.x >> 16; u[j][2] = v.y & 0xffff; u[j][3] = v.y >> 16;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {             // column 4b + i, rows 4a .. 4a + 3
      uint16_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (a > b || j > i) ? u[j][i] : u[i][j];
      u32x2 v;
      v.x = o[0] | (static_cast<uint32_t>(o[1]) << 16);
      v.y = o[2] | (static_cast<uint32_t>(o[3]) << 16);
      *reinterpret_cast<u32x2*>(T + tpos<TILE>(4 * a, 4 * b + i)) = v;
    }
  }
}

//   GRAM2 == false:  out = bf16(acc)                          (A = X X^T)
//   GRAM2 == true:   C = a [row == col] + b A + c acc  (acc = A A), out = bf16(C),
//                    and out_lo = bf16(C - out) when out_lo is given.
// `smem` is free (the K loop ended with a barrier) and holds TILE x TILE bf16.
template <int TILE, bool GRAM2>
__device__ __forceinline__ void store_sym(const f32x4_t (&acc)[Geo<TILE>::NB][Geo<TILE>::NB],
                                          uint16_t* smem, uint16_t* out, uint16_t* out_lo,
                                          const uint16_t* src, int64_t ld, int64_t ti, int64_t tj,
                                          float a, float b, float c, int tid) {
  constexpr int NB = Geo<TILE>::NB;
  const bool diag = ti == tj;
  const int64_t r0 = ti * TILE, c0 = tj * TILE;
  const int lane = tid & 63, w = tid >> 6;
  const int rowA = Geo<TILE>::WT * (w >> 1), rowB = Geo<TILE>::WT * (w & 1);
  // GRAM2: A is symmetric, so A[r0+rr+e][c0+cc] = A[c0+cc][r0+rr+e]: the
  // values a lane needs for rows rr .. rr+3 of column cc are 8 contiguous
  // bytes of the mirrored tile.  At TILE = 256 every value is fetched up
  // front (one memory round trip): the mirrored tile comes into LDS by
  // whole-line direct loads (a wave instruction moves two A rows of 512
  // bytes; an 8-byte gather per block would touch 16 lines per instruction
  // and hold up the address unit), laid out [cc][rr] with its 16-byte units
  // XOR-rotated by cc & 15, so that the 8-byte reads of a half-wave (16
  // columns x two row pieces) touch every bank once.  (At TILE = 128 the
  // loads stay next to their use: the extra registers would cost the second
  // resident block per CU.)
  constexpr bool kBatch = GRAM2 && TILE == kTileBig;
  // Block (bi, bj): lane holds rows rr .. rr+3 of column cc (tile coordinates).
  auto rrow = [&](int bi) { return rowA + 16 * bi + 4 * (lane >> 4); };
  auto rcol = [&](int bj) { return rowB + 16 * bj + (lane & 15); };
  u32x2 asrc[kBatch ? NB : 1][kBatch ? NB : 1];
  if constexpr (kBatch) {
    constexpr int UPC = TILE / 8;             // 16-byte units per column
    constexpr int CPB = 64 / UPC;             // columns per 1 KB wave load
    constexpr int BPW = TILE / CPB / 4;       // wave loads per wave
    const uint32_t lb = static_cast<uint32_t>(ld * 2);
    // the wave index as a scalar, so that the load bases below are formed
    // by scalar instructions (see dma16)
    const int ws = __builtin_amdgcn_readfirstlane(w);
#pragma unroll 8
    for (int q = 0; q < BPW; ++q) {
      const int blk = ws * BPW + q, col = blk * CPB + lane / UPC, u = lane % UPC;
      dma16(reinterpret_cast<const char*>(src + (c0 + blk * CPB) * ld + r0),
            (lane / UPC) * lb + 16u * static_cast<uint32_t>(u ^ (col & 15)), smem + blk * 512);
    }
    vm_wait<0>();
    lds_barrier();
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NB; ++bj) {
        const int rr = rrow(bi), cc = rcol(bj);
        asrc[bi][bj] = *reinterpret_cast<const u32x2*>(
            smem + cc * TILE + ((((rr >> 3) ^ (cc & 15)) << 3) | (rr & 7)));
      }
    lds_barrier();                            // the staging below reuses the LDS
  }
  for (int pass = 0; pass < ((GRAM2 && out_lo) ? 2 : 1); ++pass) {
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NB; ++bj) {
          const int rr = rrow(bi), cc = rcol(bj);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[bi][bj][e];
          if constexpr (GRAM2) {
            u32x2 av;
            if constexpr (kBatch) av = asrc[bi][bj];
            else av = gld<u32x2>(src + (c0 + cc) * ld + r0 + rr);
            const float am[4] = {__uint_as_float(av.x << 16), __uint_as_float(av.x & 0xffff0000u),
                                 __uint_as_float(av.y << 16), __uint_as_float(av.y & 0xffff0000u)};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = fmaf(c, v[e], fmaf(b, am[e], (diag && rr + e == cc) ? a : 0.f));
          }
          uint16_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[e] = f2bf(v[e]);
            if (pass == 1) h[e] = f2bf(v[e] - bf2f(h[e]));
          }
          u32x2 m;
          m.x = h[0] | (static_cast<uint32_t>(h[1]) << 16);
          m.y = h[2] | (static_cast<uint32_t>(h[3]) << 16);
          *reinterpret_cast<u32x2*>(smem + tpos<TILE>(rr, cc)) = m;
        }
    lds_barrier();
    if (diag) {
      symmetrize<TILE>(smem, tid);
      lds_barrier();
    }
    store_staged<TILE>(smem, pass == 0 ? out : out_lo, ld, r0, c0, !diag, tid);
    lds_barrier();
  }
}

// Upper-triangle tile u of a t x t tile grid -> (ti <= tj).  Tiles are
// walked in bands of 8 tile rows, column by column inside a band, so the
// tiles in flight on one XCD form compact blocks that share operand rows
// and columns in its L2.
__device__ __forceinline__ void decode_sym(int64_t u, int64_t t, int64_t& ti, int64_t& tj) {
  constexpr int64_t GM = 8;
  int64_t lo = 0;
  for (;;) {
    const int64_t hi = lo + GM < t ? lo + GM : t;
    const int64_t band = (hi - lo) * t - (lo + hi - 1) * (hi - lo) / 2;
    if (u < band || hi == t) break;
    u -= band;
    lo = hi;
  }
  const int64_t hi = lo + GM < t ? lo + GM : t;
  for (tj = lo;; ++tj) {
    const int64_t rows = (tj < hi - 1 ? tj : hi - 1) - lo + 1;
    if (u < rows || tj == t - 1) break;
    u -= rows;
  }
  ti = lo + u;
}

__device__ __forceinline__ void decode_full(int64_t u64, int64_t tm, int64_t tn, int64_t& ti,
                                            int64_t& tj) {
  constexpr int GM = 8;  // groups of 8 tile rows walk the columns together
  // a matrix has fewer than 2^31 tiles; 32-bit arithmetic, results made
  // scalar so they do not hold vector registers across the K loop
  const int u = static_cast<int>(u64), n = static_cast<int>(tn), m = static_cast<int>(tm);
  const int group = u / (GM * n);
  const int first = group * GM;
  const int gm = m - first < GM ? m - first : GM;
  const int local = u - group * GM * n;
  ti = __builtin_amdgcn_readfirstlane(first + local % gm);
  tj = __builtin_amdgcn_readfirstlane(local / gm);
}

// K3a: A = X X^T for every matrix of the launch (upper tiles + mirror)
template <int TILE>
__global__ __launch_bounds__(kGemmThreads) void k_gram(const MatDesc* __restrict__ descs,
                                                       const int64_t* __restrict__ prefix, int n,
                                                       int64_t units, int parity) {
  using G = Geo<TILE>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStages * 2 * G::TE];
  const int tid = opaque_tid();
  const int64_t unit = xcd_remap(blockIdx.x, units);
  const int mi = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[mi];
  int64_t ti, tj;
  decode_sym(unit - prefix[mi], d.m_pad / TILE, ti, tj);
  const Opnd X{d.x[parity], d.cols_pad};
  f32x4_t acc[G::NB][G::NB];
  zero_acc<G::NB>(acc);
  if (d.flags & kFlagTall)
    gemm_tile<TILE, true, true>(X, X, ti * TILE, tj * TILE, d.rows_pad, smem, acc, tid);
  else
    gemm_tile<TILE, false, false>(X, X, ti * TILE, tj * TILE, d.cols_pad, smem, acc, tid);
  store_sym<TILE, false>(acc, smem, d.a, nullptr, nullptr, d.m_pad, ti, tj, 0.f, 0.f, 0.f, tid);
}

// K3b: C = a I + b A + c A A  (A symmetric: A A = A A^T, a K-contiguous product).
// Folding a X into C (X' = C X) keeps the large cancelling terms of the
// polynomial inside one fp32 sum before the single bf16 rounding.
template <int TILE>
__global__ __launch_bounds__(kGemmThreads) void k_gram2(const MatDesc* __restrict__ descs,
                                                        const int64_t* __restrict__ prefix, int n,
                                                        int64_t units, float a, float b, float c) {
  using G = Geo<TILE>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStages * 2 * G::TE];
  const int tid = opaque_tid();
  const int64_t unit = xcd_remap(blockIdx.x, units);
  const int mi = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[mi];
  int64_t ti, tj;
  decode_sym(unit - prefix[mi], d.m_pad / TILE, ti, tj);
  const Opnd A{d.a, d.m_pad};
  f32x4_t acc[G::NB][G::NB];
  zero_acc<G::NB>(acc);
  gemm_tile<TILE, false, false>(A, A, ti * TILE, tj * TILE, d.m_pad, smem, acc, tid);
  // the hi/lo split only exists for short sides <= 128, i.e. in the 128 class
  uint16_t* lo = (TILE == kTileSmall && (d.flags & kFlagSplitC)) ? d.blo : nullptr;
  store_sym<TILE, true>(acc, smem, d.b, lo, d.a, d.m_pad, ti, tj, a, b, c, tid);
}

// K4: X' = C X.  Wide (rows <= cols): X'[i][k] = sum_j C[i][j] X[j][k].
// Tall: the stored matrix is X^T, so X'^T = X^T C (C symmetric).
// Split matrices add the low part: X' = C_hi X + C_lo X.
template <int TILE>
__global__ __launch_bounds__(kGemmThreads) void k_xupdate(const MatDesc* __restrict__ descs,
                                                          const int64_t* __restrict__ prefix,
                                                          int n, int64_t units, int parity) {
  using G = Geo<TILE>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStages * 2 * G::TE];
  const int tid = opaque_tid();
  const int64_t unit = xcd_remap(blockIdx.x, units);
  const int mi = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[mi];
  int64_t ti, tj;
  decode_full(unit - prefix[mi], d.rows_pad / TILE, d.cols_pad / TILE, ti, tj);
  const uint16_t* x = d.x[parity];
  uint16_t* xn = d.x[parity ^ 1];
  const int64_t ld = d.cols_pad;
  // the hi/lo split only exists for short sides <= 128, i.e. in the 128 class
  const bool split = TILE == kTileSmall && (d.flags & kFlagSplitC) != 0;
  f32x4_t acc[G::NB][G::NB];
  zero_acc<G::NB>(acc);
  if (d.flags & kFlagTall) {
    gemm_tile<TILE, false, false, true>(Opnd{x, ld}, Opnd{d.b, d.m_pad}, ti * TILE, tj * TILE,
                                        d.m_pad, smem, acc, tid);
    if (split)
      gemm_tile<TILE, false, false, true>(Opnd{x, ld}, Opnd{d.blo, d.m_pad}, ti * TILE, tj * TILE,
                                          d.m_pad, smem, acc, tid);
  } else {
    // C is exactly symmetric, so its rows may also be read as MN-contiguous
    // columns.  At TILE = 128 both operands take the transpose-read path
    // (the mixed form compiles to accumulator copies there); at 256 C keeps
    // its cheaper 16-byte fragment reads.
    constexpr bool kCmn = TILE == kTileSmall;
    gemm_tile<TILE, kCmn, true, true>(Opnd{d.b, d.m_pad}, Opnd{x, ld}, ti * TILE, tj * TILE,
                                      d.m_pad, smem, acc, tid);
    if (split)
      gemm_tile<TILE, kCmn, true, true>(Opnd{d.blo, d.m_pad}, Opnd{x, ld}, ti * TILE, tj * TILE,
                                        d.m_pad, smem, acc, tid);
  }
  // Stage the bf16 tile in LDS, row-major with 8-byte units XORed by the row
  // (unit u of row r at u ^ (r & 31): a staging write, 32 rows at one unit,
  // then covers all banks), and write it out as whole 16-byte row chunks.
  // Transposed blocks: lane holds row rowA + 16 bi + (lane & 15), columns
  // rowB + 16 bj + 4 (lane >> 4) .. +3.
  const int lane = tid & 63, w = tid >> 6;
  const int rl = G::WT * (w >> 1) + (lane & 15);
  const int cl = G::WT * (w & 1) + 4 * (lane >> 4);
#pragma unroll
  for (int bi = 0; bi < G::NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < G::NB; ++bj) {
      u32x2 m;
      m.x = pack2(acc[bi][bj][0], acc[bi][bj][1]);
      m.y = pack2(acc[bi][bj][2], acc[bi][bj][3]);
      const int r = rl + 16 * bi, u = (cl + 16 * bj) >> 2;
      *reinterpret_cast<u32x2*>(smem + r * TILE + ((u ^ (r & 31)) << 2)) = m;
    }
  lds_barrier();
  constexpr int CPR = TILE / 8;  // 16-byte chunks per row
#pragma unroll 4
  for (int idx = tid; idx < TILE * CPR; idx += kGemmThreads) {
    const int r = idx / CPR, ch = idx % CPR;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(smem + r * TILE + (((2 * ch) ^ (r & 31)) << 2));
    const u32x2 hi = *reinterpret_cast<const u32x2*>(smem + r * TILE + (((2 * ch + 1) ^ (r & 31)) << 2));
    const u32x4 v{lo.x, lo.y, hi.x, hi.y};
    // at TILE 128 the new iterate is written non-temporally: the tiles in
    // flight then keep more of the cache for their operands (5 % on that
    // launch); at 256 it measured slower
    if constexpr (TILE == kTileSmall)
      __builtin_nontemporal_store(v, (__attribute__((address_space(1))) u32x4*)(xn + (ti * TILE + r) * ld + tj * TILE + 8 * ch));
    else
      gst<u32x4>(xn + (ti * TILE + r) * ld + tj * TILE + 8 * ch, v);
  }
}

// ---------------------------------------------------------------------------
// launchers (instantiated once per tile size, each in its own translation
// unit so that each can be compiled with the register form that suits it)
// ---------------------------------------------------------------------------
template <int TILE>
int launch_gram_t(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                  void* stream) {
  hipLaunchKernelGGL(k_gram<TILE>, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, units, parity);
  return static_cast<int>(hipGetLastError());
}

template <int TILE>
int launch_gram2_t(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float a, float b,
                   float c, void* stream) {
  hipLaunchKernelGGL(k_gram2<TILE>, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, units, a, b, c);
  return static_cast<int>(hipGetLastError());
}

template <int TILE>
int launch_xupdate_t(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                     void* stream) {
  hipLaunchKernelGGL(k_xupdate<TILE>, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, units, parity);
  return static_cast<int>(hipGetLastError());
}

}  // namespace muon
