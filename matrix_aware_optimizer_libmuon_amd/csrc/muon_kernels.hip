// gfx950 (CDNA4) kernels of the Muon step.
//
//   K1 momentum + Frobenius sum of squares   (HBM-bound, one fp64 atomic per workgroup)
//   K2 normalise + cast to bf16              (HBM-bound, writes the zero-padded X0)
//   K3a Gram      A = X X^T                  (bf16 MFMA, upper-triangle tiles, mirrored store)
//   K3b Gram^2    C = a I + b A + c A A      (bf16 MFMA, A symmetric so A A = A A^T)
//   K4  X update  X' = C X                   (bf16 MFMA; a X folded into C)
//   K5 apply      p <- p (1 - lr wd) - lr s O (HBM-bound)
//
// Every kernel is one grouped launch over all matrices of a call: workgroup
// -> (matrix, work unit) by binary search in a per-phase prefix array.
//
// The method (pages cited by title/section): momentum and update follow the
// Muon.step loop of "Muon optimizer: matrix-aware LLM" (airosetta.com) and
// _step_muon of "Muon meets Mamba" (wmrh.cn, section 4.2); the iteration is
// that article's newtonschulz5 routine, whose expanded polynomial form is in
// "AdamW vs Muon" (adg.csdn.net, section "2. Newton-Schulz iteration").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"

namespace muon {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Loads through the global address space: the pointers come from the
// descriptor table, so the compiler would otherwise emit generic (flat)
// accesses.
template <class T>
__device__ __forceinline__ T gld(const void* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}
template <class T>
__device__ __forceinline__ void gst(void* p, T v) {
  *(__attribute__((address_space(1))) T*)(p) = v;
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

// Largest i with prefix[i] <= unit (prefix[0] == 0, every matrix owns >= 1 unit).
__device__ __forceinline__ int find_matrix(const int64_t* __restrict__ prefix, int n,
                                           int64_t unit) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= unit) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Workgroups are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
// Map them so each XCD receives one contiguous range of logical units:
// neighbouring tiles share operand rows and then meet in the same L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t nb) {
  const int64_t per = nb >> 3, rem = nb & 7;
  const int64_t x = b & 7, i = b >> 3;
  return x * per + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ double block_sum_256(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) s = red[0] + red[1] + red[2] + red[3];
  return s;
}

// ---------------------------------------------------------------------------
// K1: M <- mu M + (1 - mu) G, and sum of M^2 (norm_only: sum of G^2, no update)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8_src(const void* src, bool bf16, int64_t e, float (&v)[8]) {
  if (bf16) {
    const u32x4 q = gld<u32x4>(static_cast<const uint16_t*>(src) + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(q[j] << 16);
      v[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
    }
  } else {
    const f32x4 a = gld<f32x4>(static_cast<const float*>(src) + e);
    const f32x4 b = gld<f32x4>(static_cast<const float*>(src) + e + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
}

__device__ __forceinline__ float load1_src(const void* src, bool bf16, int64_t e) {
  return bf16 ? bf2f(gld<uint16_t>(static_cast<const uint16_t*>(src) + e))
              : gld<float>(static_cast<const float*>(src) + e);
}

__global__ __launch_bounds__(kEwThreads) void k_momentum_norm(
    const MatDesc* __restrict__ descs, const int64_t* __restrict__ prefix, int n,
    float mu, float omu, int norm_only) {
  __shared__ double red[4];
  const int64_t unit = blockIdx.x;
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  const int64_t total = d.rows * d.cols;
  const int64_t begin = (unit - prefix[i]) * kChunk;
  const int64_t end = begin + kChunk < total ? begin + kChunk : total;
  const bool gbf = (d.flags & kFlagGradBf16) != 0;
  constexpr int S = kEwThreads * 8;  // elements per block-wide vector step
  float acc = 0.f;
  if (d.flags & kFlagVecFlat) {
    int64_t e = begin + threadIdx.x * 8;
    // two 8-element vectors in flight per thread
    for (; e + S < end; e += 2 * S) {
      float g0[8], g1[8];
      load8_src(d.grad, gbf, e, g0);
      load8_src(d.grad, gbf, e + S, g1);
      if (norm_only) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(g0[j], g0[j], fmaf(g1[j], g1[j], acc));
      } else {
        f32x4 m0 = gld<f32x4>(d.mom + e), m1 = gld<f32x4>(d.mom + e + 4);
        f32x4 m2 = gld<f32x4>(d.mom + e + S), m3 = gld<f32x4>(d.mom + e + S + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          m0[j] = fmaf(mu, m0[j], omu * g0[j]);
          m1[j] = fmaf(mu, m1[j], omu * g0[4 + j]);
          m2[j] = fmaf(mu, m2[j], omu * g1[j]);
          m3[j] = fmaf(mu, m3[j], omu * g1[4 + j]);
          acc = fmaf(m0[j], m0[j], acc);
          acc = fmaf(m1[j], m1[j], acc);
          acc = fmaf(m2[j], m2[j], acc);
          acc = fmaf(m3[j], m3[j], acc);
        }
        gst<f32x4>(d.mom + e, m0);
        gst<f32x4>(d.mom + e + 4, m1);
        gst<f32x4>(d.mom + e + S, m2);
        gst<f32x4>(d.mom + e + S + 4, m3);
      }
    }
    if (e < end) {
      float g[8];
      load8_src(d.grad, gbf, e, g);
      if (norm_only) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(g[j], g[j], acc);
      } else {
        f32x4 m0 = gld<f32x4>(d.mom + e), m1 = gld<f32x4>(d.mom + e + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          m0[j] = fmaf(mu, m0[j], omu * g[j]);
          m1[j] = fmaf(mu, m1[j], omu * g[4 + j]);
          acc = fmaf(m0[j], m0[j], acc);
          acc = fmaf(m1[j], m1[j], acc);
        }
        gst<f32x4>(d.mom + e, m0);
        gst<f32x4>(d.mom + e + 4, m1);
      }
    }
  } else {
    for (int64_t e = begin + threadIdx.x; e < end; e += kEwThreads) {
      const float g = load1_src(d.grad, gbf, e);
      if (norm_only) {
        acc = fmaf(g, g, acc);
      } else {
        const float m = fmaf(mu, gld<float>(d.mom + e), omu * g);
        gst<float>(d.mom + e, m);
        acc = fmaf(m, m, acc);
      }
    }
  }
  const double s = block_sum_256(static_cast<double>(acc), red);
  if (threadIdx.x == 0) unsafeAtomicAdd(d.nrm2, s);
}

// Walks a row-major block of rows [r0, r1) x [0, w) in steps of `step`
// elements per thread, keeping (row, col) without a division per step.
struct RowWalk {
  int64_t r, c;
  int sr, sc, w;
  __device__ RowWalk(int64_t r0, int first, int step, int width) : w(width) {
    r = r0 + first / width;
    c = first % width;
    sr = step / width;
    sc = step % width;
  }
  __device__ void next() {
    r += sr;
    c += sc;
    if (c >= w) {
      c -= w;
      ++r;
    }
  }
};

// ---------------------------------------------------------------------------
// K2: X0 = bf16(M / (||M|| + eps)) into the zero-padded rows_pad x cols_pad buffer.
// One work unit = rg_pad padded rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kEwThreads) void k_normalize(
    const MatDesc* __restrict__ descs, const int64_t* __restrict__ prefix, int n, float eps) {
  const int64_t unit = blockIdx.x;
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  const bool ortho = d.mom == nullptr;  // orthogonalize: the source is the input
  const void* src = ortho ? d.grad : static_cast<const void*>(d.mom);
  const bool sbf = ortho && (d.flags & kFlagGradBf16);
  const float inv = static_cast<float>(1.0 / (sqrt(gld<double>(d.nrm2)) + static_cast<double>(eps)));
  const int cp = d.cols_pad;
  const int64_t r0 = (unit - prefix[i]) * d.rg_pad;
  const int64_t r1 = r0 + d.rg_pad < d.rows_pad ? r0 + d.rg_pad : d.rows_pad;
  const int64_t count = (r1 - r0) * cp;
  const bool vec = (d.flags & kFlagVecRows) != 0;
  uint16_t* x0 = d.x[0];
  constexpr int S = kEwThreads * 8;
  RowWalk p(r0, threadIdx.x * 8, S, cp);
  for (int64_t e = threadIdx.x * 8; e < count; e += S, p.next()) {
    const int64_t r = p.r, c0 = p.c;
    float v[8];
    if (r < d.rows && vec && c0 + 8 <= d.cols) {
      load8_src(src, sbf, r * d.cols + c0, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = (r < d.rows && c0 + j < d.cols) ? load1_src(src, sbf, r * d.cols + c0 + j) : 0.f;
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack2(v[2 * j] * inv, v[2 * j + 1] * inv);
    gst<u32x4>(x0 + r * cp + c0, o);
  }
}

// ---------------------------------------------------------------------------
// K5: p <- p (1 - lr wd) - lr s O    (export_only: out <- O, unpadded).
// One work unit = rg rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kEwThreads) void k_apply(
    const MatDesc* __restrict__ descs, const int64_t* __restrict__ prefix, int n, int parity,
    float lr, float wd, int export_only) {
  const int64_t unit = blockIdx.x;
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  const uint16_t* o = d.x[parity];
  const int64_t cp = d.cols_pad;
  const int cols = static_cast<int>(d.cols);
  const int64_t r0 = (unit - prefix[i]) * d.rg;
  const int64_t r1 = r0 + d.rg < d.rows ? r0 + d.rg : d.rows;
  const int64_t count = (r1 - r0) * cols;
  const float decay = 1.0f - lr * wd;
  const float step = lr * d.scale;
  if (d.flags & kFlagVecRows) {
    constexpr int S = kEwThreads * 8;
    RowWalk p(r0, threadIdx.x * 8, S, cols);
    for (int64_t e = threadIdx.x * 8; e < count; e += S, p.next()) {
      const int64_t r = p.r, c = p.c, g = r * cols + c;
      const u32x4 q = gld<u32x4>(o + r * cp + c);
      if (export_only) {
        gst<u32x4>(d.out + g, q);
      } else {
        f32x4 p0 = gld<f32x4>(d.param + g), p1 = gld<f32x4>(d.param + g + 4);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          p0[2 * j] = fmaf(-step, __uint_as_float(q[j] << 16), p0[2 * j] * decay);
          p0[2 * j + 1] = fmaf(-step, __uint_as_float(q[j] & 0xffff0000u), p0[2 * j + 1] * decay);
          p1[2 * j] = fmaf(-step, __uint_as_float(q[2 + j] << 16), p1[2 * j] * decay);
          p1[2 * j + 1] = fmaf(-step, __uint_as_float(q[2 + j] & 0xffff0000u), p1[2 * j + 1] * decay);
        }
        gst<f32x4>(d.param + g, p0);
        gst<f32x4>(d.param + g + 4, p1);
      }
    }
  } else {
    RowWalk p(r0, threadIdx.x, kEwThreads, cols);
    for (int64_t e = threadIdx.x; e < count; e += kEwThreads, p.next()) {
      const int64_t r = p.r, c = p.c, g = r * cols + c;
      const uint16_t q = gld<uint16_t>(o + r * cp + c);
      if (export_only) gst<uint16_t>(d.out + g, q);
      else gst<float>(d.param + g, fmaf(-step, bf2f(q), gld<float>(d.param + g) * decay));
    }
  }
}

// ---------------------------------------------------------------------------
// Newton-Schulz GEMM engine on bf16 MFMA (v_mfma_f32_32x32x16_bf16)
//
// Output tile TILE x TILE (128 or 256), K step 32, 4 waves in a 2 x 2 grid,
// each wave (TILE/2) x (TILE/2) = NB x NB MFMA blocks of 32 x 32 with fp32
// accumulators (256 of them per lane at TILE = 256, held in AGPRs).
//
// Operand tiles go straight from global memory into LDS (16 bytes per lane,
// no register staging, no LDS store instructions): on this chip LDS stores
// from registers run at about two thirds of the LDS read rate and were the
// limit.  Four LDS stages; loads run three K steps ahead; one barrier per K
// step, placed between its two 16-deep MFMA substeps so the fragments of the
// next step are read while the second substep's MFMAs run.
//
// An operand is "K-contiguous" (element (mn, k) at p[mn * ld + k]) or
// "MN-contiguous" (element (mn, k) at p[k * ld + mn]).
//   K-contiguous tiles sit in LDS as [mn][32 k] (64-byte rows); fragments
//     are 16-byte reads; the 16-byte chunk c of row r is stored at
//     c ^ ((r >> 1) & 3), which spreads the 8 rows read per cycle over all
//     banks.
//   MN-contiguous tiles keep their memory layout, [k][TILE mn]; fragments
//     are assembled by the LDS transpose read (ds_read_b64_tr_b16: in each
//     16-lane group, lane 4a + b receives element b of the 8-byte blocks
//     addressed by lanes a, a + 4, a + 8, a + 12), so the transpose of a tall
//     matrix is never materialised, not even in registers.  The 16-byte
//     chunk c of k row r is stored at c ^ (2 (r & 3)): the four k rows one
//     transpose read touches then hit distinct banks.
// ---------------------------------------------------------------------------
constexpr int BK = 32;
constexpr int kStages = 4;

template <int TILE>
struct Geo {
  static constexpr int T = TILE;
  static constexpr int WT = TILE / 2;      // wave tile
  static constexpr int NB = WT / 32;       // 32x32 MFMA blocks per wave side
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

// Global -> LDS, 16 bytes per lane, without registers.  Written as a one-line
// asm statement: it writes only LDS (no register results), and the compiler
// would otherwise assume every later LDS read may alias these writes and wait
// for all of them.  Ordering is explicit instead: vm_wait<> on the issuing
// wave, then an LDS barrier, before any wave reads the stage.
__device__ __forceinline__ void dma16(const uint16_t* src, uint16_t* lds_dst) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) void*)lds_dst));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0));
}

// Block q of this wave's share of a TILE x 32 operand tile.  The tile is
// TILE * 64 bytes = TILE / 16 blocks of 1 KB; block b belongs to wave
// b / LPW, and lane l lands at byte 16 l of its block.
template <bool MN, int TILE>
__device__ __forceinline__ void dload(const Opnd& op, int64_t mn0, int64_t k0, uint16_t* tile,
                                      int q) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int blk = w * Geo<TILE>::LPW + q;
  const uint16_t* src;
  if constexpr (!MN) {  // 16 rows of 64 bytes per block
    const int row = blk * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 1) & 3);
    src = op.p + (mn0 + row) * op.ld + k0 + 8 * c;
  } else {              // 512 / TILE k rows of 2 TILE bytes per block
    constexpr int CPR = TILE / 8;  // 16-byte chunks per k row
    const int row = blk * (512 / TILE) + lane / CPR;
    const int c = (lane % CPR) ^ (2 * (row & 3));
    src = op.p + (k0 + row) * op.ld + mn0 + 8 * c;
  }
  dma16(src, tile + __builtin_amdgcn_readfirstlane(blk) * 512);
}

// MFMA fragment (32 rows from rowbase, k = 16 sub .. 16 sub + 15) of one operand tile.
template <bool MN, int TILE>
__device__ __forceinline__ bf16x8_t frag(const uint16_t* tile, int rowbase, int sub) {
  const int lane = threadIdx.x & 63;
  if constexpr (!MN) {
    const int row = rowbase + (lane & 31);
    const int c = (2 * sub + (lane >> 5)) ^ ((row >> 1) & 3);
    return *reinterpret_cast<const bf16x8_t*>(tile + row * BK + c * 8);
  } else {
    const int g = lane >> 4, i = lane & 15;
    const int m = rowbase + 16 * (g & 1) + 4 * (i & 3);
    const int k = 16 * sub + 8 * (g >> 1) + (i >> 2);   // + 4 t below; k & 3 == i >> 2
    const int off = (((m >> 3) ^ (2 * (i >> 2))) << 3) + (m & 4);
    const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(tile + k * TILE + off));
    const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(tile + (k + 4) * TILE + off));
    u32x4 v;
    v.x = __builtin_bit_cast(u32x2, r0).x;
    v.y = __builtin_bit_cast(u32x2, r0).y;
    v.z = __builtin_bit_cast(u32x2, r1).x;
    v.w = __builtin_bit_cast(u32x2, r1).y;
    return __builtin_bit_cast(bf16x8_t, v);
  }
}

template <int NB>
__device__ __forceinline__ void mfma_block(const bf16x8_t (&fa)[NB], const bf16x8_t (&fb)[NB],
                                           f32x16_t (&acc)[NB][NB]) {
#pragma unroll
  for (int bi = 0; bi < NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < NB; ++bj)
      acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[bi], fb[bj], acc[bi][bj], 0, 0, 0);
}

template <int NB>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[NB][NB]) {
#pragma unroll
  for (int bi = 0; bi < NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < NB; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;
}

// acc += P[mp0 : mp0+TILE, :K] * Q[nq0 : nq0+TILE, :K]^T   (K a multiple of 128)
//
// Iteration kt (stage kt mod 4 holds K step kt), instruction order pinned:
//   substep 0: its NB*NB MFMAs; between them the fragment reads of substep 1
//              and half of the loads of step kt+3 into stage (kt+3) mod 4
//              (its last reader finished before the previous barrier)
//   wait for this wave's loads of step kt+1; LDS barrier
//   substep 1: its MFMAs; between them the fragment reads of substep 0 of
//              step kt+1 and the other half of the loads of step kt+3
// The loads are spread one per two MFMAs: issued in bursts they back up the
// CU's vector memory pipe, and a wave whose load cannot issue cannot issue
// its next MFMA either.  MFMA blocks are walked column by column, so each B
// fragment is consumed at least 3 NB MFMAs after it was read.  Loads past
// the end re-read the last step (never consumed): the body has no branches.
//
// SWAP = true accumulates the transposed blocks (MFMA operands exchanged), so
// each lane ends up holding four consecutive output columns of one row.
template <int TILE, bool PMN, bool QMN, bool SWAP = false>
__device__ __forceinline__ void gemm_tile(const Opnd& P, const Opnd& Q, int64_t mp0, int64_t nq0,
                                          int64_t K, uint16_t* smem,
                                          f32x16_t (&acc)[Geo<TILE>::NB][Geo<TILE>::NB]) {
  using G = Geo<TILE>;
  constexpr int NB = G::NB;
  constexpr int LPS = 2 * G::LPW;       // loads per wave per stage
  constexpr int HALF = LPS / 2;         // loads per substep
  // MFMA slot of load j inside a substep (after the 2 NB fragment reads), or
  // -1 when the substep is too short and the load goes after its MFMAs
  constexpr int FIRST = 2 * NB + 1;
  const int w = threadIdx.x >> 6;
  const int rowA = G::WT * (w >> 1), rowB = G::WT * (w & 1);
  bf16x8_t fa0[NB], fb0[NB], fa1[NB], fb1[NB];
  const int64_t kt_n = K / BK;
  auto stage = [&](int64_t kt) { return smem + static_cast<int>(kt & (kStages - 1)) * (2 * G::TE); };
  auto load = [&](int64_t kt, int part) {  // part < LPW: P blocks, else Q blocks
    const int64_t k0 = (kt < kt_n ? kt : kt_n - 1) * BK;
    uint16_t* st = stage(kt);
    if (part < G::LPW) dload<PMN, TILE>(P, mp0, k0, st, part);
    else dload<QMN, TILE>(Q, nq0, k0, st + G::TE, part - G::LPW);
  };
  auto mfma = [&](const bf16x8_t (&fa)[NB], const bf16x8_t (&fb)[NB], int bi, int bj) {
    acc[bi][bj] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[bj], fa[bi], acc[bi][bj], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[bi], fb[bj], acc[bi][bj], 0, 0, 0);
  };
#pragma unroll
  for (int kt = 0; kt < kStages - 1; ++kt)
#pragma unroll
    for (int part = 0; part < LPS; ++part) load(kt, part);
  vm_wait<(kStages - 2) * LPS>();
  lds_barrier();
#pragma unroll
  for (int b = 0; b < NB; ++b) fa0[b] = frag<PMN, TILE>(smem, rowA + 32 * b, 0);
#pragma unroll
  for (int b = 0; b < NB; ++b) fb0[b] = frag<QMN, TILE>(smem + G::TE, rowB + 32 * b, 0);
  for (int64_t kt = 0; kt < kt_n; ++kt) {
    const uint16_t* cur = stage(kt);
    const int64_t kl = kt + kStages - 1;
#pragma unroll
    for (int idx = 0; idx < NB * NB; ++idx) {
      mfma(fa0, fb0, idx % NB, idx / NB);
      if (idx < NB) fa1[idx] = frag<PMN, TILE>(cur, rowA + 32 * idx, 1);
      else if (idx < 2 * NB) fb1[idx - NB] = frag<QMN, TILE>(cur + G::TE, rowB + 32 * (idx - NB), 1);
      else if (idx >= FIRST && (idx - FIRST) % 2 == 0 && (idx - FIRST) / 2 < HALF) load(kl, (idx - FIRST) / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < HALF; ++j)
      if (FIRST + 2 * j >= NB * NB) load(kl, j);
    // at most: the other half of step kt+3 is not issued yet; steps kt+2 and
    // the first half of kt+3 may still be in flight
    vm_wait<LPS + HALF>();
    lds_barrier();
    const uint16_t* nx = stage(kt + 1);
#pragma unroll
    for (int idx = 0; idx < NB * NB; ++idx) {
      mfma(fa1, fb1, idx % NB, idx / NB);
      if (idx < NB) fa0[idx] = frag<PMN, TILE>(nx, rowA + 32 * idx, 0);
      else if (idx < 2 * NB) fb0[idx - NB] = frag<QMN, TILE>(nx + G::TE, rowB + 32 * (idx - NB), 0);
      else if (idx >= FIRST && (idx - FIRST) % 2 == 0 && (idx - FIRST) / 2 < HALF) load(kl, HALF + (idx - FIRST) / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < HALF; ++j)
      if (FIRST + 2 * j >= NB * NB) load(kl, HALF + j);
  }
  vm_wait<0>();
  lds_barrier();  // every wave is done with every stage
}

// Position of accumulator element r of MFMA block (bi, bj) inside the tile.
template <int TILE>
__device__ __forceinline__ void acc_pos(int bi, int bj, int r, int& row, int& col) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  row = Geo<TILE>::WT * (w >> 1) + 32 * bi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  col = Geo<TILE>::WT * (w & 1) + 32 * bj + (lane & 31);
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
                                             int64_t r0, int64_t c0, bool mirror) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
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
// the value computed for (col, row).
template <int TILE>
__device__ __forceinline__ void symmetrize(uint16_t* T) {
  for (int idx = threadIdx.x; idx < TILE * TILE; idx += kGemmThreads) {
    const int row = idx / TILE, col = idx % TILE;
    if (row > col) T[tpos<TILE>(row, col)] = T[tpos<TILE>(col, row)];
  }
}

//   GRAM2 == false:  out = bf16(acc)                          (A = X X^T)
//   GRAM2 == true:   C = a [row == col] + b A + c acc  (acc = A A), out = bf16(C),
//                    and out_lo = bf16(C - out) when out_lo is given.
// `smem` is free (the K loop ended with a barrier) and holds TILE x TILE bf16.
template <int TILE, bool GRAM2>
__device__ __forceinline__ void store_sym(const f32x16_t (&acc)[Geo<TILE>::NB][Geo<TILE>::NB],
                                          uint16_t* smem, uint16_t* out, uint16_t* out_lo,
                                          const uint16_t* src, int64_t ld, int64_t ti, int64_t tj,
                                          float a, float b, float c) {
  constexpr int NB = Geo<TILE>::NB;
  const bool diag = ti == tj;
  const int64_t r0 = ti * TILE, c0 = tj * TILE;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rowA = Geo<TILE>::WT * (w >> 1), rowB = Geo<TILE>::WT * (w & 1);
  for (int pass = 0; pass < ((GRAM2 && out_lo) ? 2 : 1); ++pass) {
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NB; ++bj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // rows rr .. rr+3 of column cc (tile coordinates)
          const int rr = rowA + 32 * bi + 8 * q + 4 * (lane >> 5), cc = rowB + 32 * bj + (lane & 31);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[bi][bj][4 * q + e];
          if constexpr (GRAM2) {
            // A is symmetric: A[r0+rr+e][c0+cc] = A[c0+cc][r0+rr+e], one 8-byte load
            const u32x2 av = gld<u32x2>(src + (c0 + cc) * ld + r0 + rr);
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
      symmetrize<TILE>(smem);
      lds_barrier();
    }
    store_staged<TILE>(smem, pass == 0 ? out : out_lo, ld, r0, c0, !diag);
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

__device__ __forceinline__ void decode_full(int64_t u, int64_t tm, int64_t tn, int64_t& ti,
                                            int64_t& tj) {
  constexpr int64_t GM = 8;  // groups of 8 tile rows walk the columns together
  const int64_t group = u / (GM * tn);
  const int64_t first = group * GM;
  const int64_t gm = tm - first < GM ? tm - first : GM;
  const int64_t local = u - group * GM * tn;
  ti = first + local % gm;
  tj = local / gm;
}

// K3a: A = X X^T for every matrix of the launch (upper tiles + mirror)
template <int TILE>
__global__ __launch_bounds__(kGemmThreads) void k_gram(const MatDesc* __restrict__ descs,
                                                       const int64_t* __restrict__ prefix, int n,
                                                       int64_t units, int parity) {
  using G = Geo<TILE>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStages * 2 * G::TE];
  const int64_t unit = xcd_remap(blockIdx.x, units);
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  int64_t ti, tj;
  decode_sym(unit - prefix[i], d.m_pad / TILE, ti, tj);
  const Opnd X{d.x[parity], d.cols_pad};
  f32x16_t acc[G::NB][G::NB];
  zero_acc<G::NB>(acc);
  if (d.flags & kFlagTall)
    gemm_tile<TILE, true, true>(X, X, ti * TILE, tj * TILE, d.rows_pad, smem, acc);
  else
    gemm_tile<TILE, false, false>(X, X, ti * TILE, tj * TILE, d.cols_pad, smem, acc);
  store_sym<TILE, false>(acc, smem, d.a, nullptr, nullptr, d.m_pad, ti, tj, 0.f, 0.f, 0.f);
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
  const int64_t unit = xcd_remap(blockIdx.x, units);
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  int64_t ti, tj;
  decode_sym(unit - prefix[i], d.m_pad / TILE, ti, tj);
  const Opnd A{d.a, d.m_pad};
  f32x16_t acc[G::NB][G::NB];
  zero_acc<G::NB>(acc);
  gemm_tile<TILE, false, false>(A, A, ti * TILE, tj * TILE, d.m_pad, smem, acc);
  // the hi/lo split only exists for short sides <= 128, i.e. in the 128 class
  uint16_t* lo = (TILE == kTileSmall && (d.flags & kFlagSplitC)) ? d.blo : nullptr;
  store_sym<TILE, true>(acc, smem, d.b, lo, d.a, d.m_pad, ti, tj, a, b, c);
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
  const int64_t unit = xcd_remap(blockIdx.x, units);
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  int64_t ti, tj;
  decode_full(unit - prefix[i], d.rows_pad / TILE, d.cols_pad / TILE, ti, tj);
  const uint16_t* x = d.x[parity];
  uint16_t* xn = d.x[parity ^ 1];
  const int64_t ld = d.cols_pad;
  // the hi/lo split only exists for short sides <= 128, i.e. in the 128 class
  const bool split = TILE == kTileSmall && (d.flags & kFlagSplitC) != 0;
  f32x16_t acc[G::NB][G::NB];
  zero_acc<G::NB>(acc);
  if (d.flags & kFlagTall) {
    gemm_tile<TILE, false, false, true>(Opnd{x, ld}, Opnd{d.b, d.m_pad}, ti * TILE, tj * TILE,
                                        d.m_pad, smem, acc);
    if (split)
      gemm_tile<TILE, false, false, true>(Opnd{x, ld}, Opnd{d.blo, d.m_pad}, ti * TILE, tj * TILE,
                                          d.m_pad, smem, acc);
  } else {
    gemm_tile<TILE, false, true, true>(Opnd{d.b, d.m_pad}, Opnd{x, ld}, ti * TILE, tj * TILE,
                                       d.m_pad, smem, acc);
    if (split)
      gemm_tile<TILE, false, true, true>(Opnd{d.blo, d.m_pad}, Opnd{x, ld}, ti * TILE, tj * TILE,
                                         d.m_pad, smem, acc);
  }
  // transposed blocks: lane holds row rowA + 32 bi + (lane & 31), columns
  // rowB + 32 bj + 8 q + 4 (lane >> 5) .. +3  ->  one 8-byte store each
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t r0 = ti * TILE + G::WT * (w >> 1) + (lane & 31);
  const int64_t c0 = tj * TILE + G::WT * (w & 1) + 4 * (lane >> 5);
#pragma unroll
  for (int bi = 0; bi < G::NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < G::NB; ++bj)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 m;
        m.x = pack2(acc[bi][bj][4 * q], acc[bi][bj][4 * q + 1]);
        m.y = pack2(acc[bi][bj][4 * q + 2], acc[bi][bj][4 * q + 3]);
        gst<u32x2>(xn + (r0 + 32 * bi) * ld + c0 + 32 * bj + 8 * q, m);
      }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline int grid_ok(int64_t units) { return units > 0 && units < (int64_t(1) << 31); }

int launch_momentum_norm(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float mu,
                         int norm_only, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_momentum_norm, dim3(static_cast<unsigned>(units)), dim3(kEwThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, mu, 1.0f - mu, norm_only);
  return static_cast<int>(hipGetLastError());
}

int launch_normalize(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float eps,
                     void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_normalize, dim3(static_cast<unsigned>(units)), dim3(kEwThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, eps);
  return static_cast<int>(hipGetLastError());
}

int launch_gram(int tile, const MatDesc* d, const int64_t* prefix, int n, int64_t units,
                int parity, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (tile == 256)
    hipLaunchKernelGGL(k_gram<256>, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0, st,
                       d, prefix, n, units, parity);
  else
    hipLaunchKernelGGL(k_gram<128>, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0, st,
                       d, prefix, n, units, parity);
  return static_cast<int>(hipGetLastError());
}

int launch_gram2(int tile, const MatDesc* d, const int64_t* prefix, int n, int64_t units, float a,
                 float b, float c, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (tile == 256)
    hipLaunchKernelGGL(k_gram2<256>, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0, st,
                       d, prefix, n, units, a, b, c);
  else
    hipLaunchKernelGGL(k_gram2<128>, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0, st,
                       d, prefix, n, units, a, b, c);
  return static_cast<int>(hipGetLastError());
}

int launch_xupdate(int tile, const MatDesc* d, const int64_t* prefix, int n, int64_t units,
                   int parity, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (tile == 256)
    hipLaunchKernelGGL(k_xupdate<256>, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0,
                       st, d, prefix, n, units, parity);
  else
    hipLaunchKernelGGL(k_xupdate<128>, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0,
                       st, d, prefix, n, units, parity);
  return static_cast<int>(hipGetLastError());
}

int launch_apply(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                 float lr, float wd, int export_only, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_apply, dim3(static_cast<unsigned>(units)), dim3(kEwThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, parity, lr, wd, export_only);
  return static_cast<int>(hipGetLastError());
}

}  // namespace muon
